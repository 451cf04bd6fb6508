// Fine-grained FP8 quantisation: dynamic 1x128 activation slices and 128x128
// weight blocks, E4M3 codes with one FP32 scale each (Transformers PR #47844,
// implementation list: dynamic activations, E4M3 weights, 128 x 128 weight
// block size; validation list and the authors' reply: partial blocks when a
// dimension is not a multiple of 128).
//
// Rule for a slice or block: s = f32(amax / 448) with a correctly rounded
// FP32 division; code = E4M3 round-to-nearest-even of f32(v / s), saturated at
// +-448, sign bit kept; s == 0 gives all-zero codes. Partial slices and
// blocks take the amax over their valid elements only.
#include "dmoe_internal.h"
#include "quant_common.h"

namespace dmoe {

// 16 lanes per 128-column slice, 8 BF16 values (16 bytes) per lane; a
// 256-thread workgroup covers G rounds of 16 consecutive slices (slice
// (blockIdx.x G + u) 16 + lane / 16 in round u). The G loads of a lane are
// issued before any is used, so a wave has G 16-byte loads per lane in flight
// (G = 4 on large inputs: prefill quantise-h 0.074 -> 0.062 ms). Every input
// element is read once, so the loads carry the non-temporal policy (prefill
// quantise-h 0.078 -> 0.073 ms, EP-share quantise-x 0.062 -> 0.056 ms).
// skip_from != nullptr: rows [*skip_from, skip_to) are left untouched (the
// layer's routed rows past the real count M, which no GEMM wrote).
template <int G>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                        int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ scales, int64_t lds,
                                                        const int32_t* __restrict__ skip_from, int skip_to) {
  const int skip_lo = skip_from ? *skip_from : skip_to;
  const int nsl = (cols + 127) >> 7;
  const int64_t total = (int64_t)rows * nsl;
  const int64_t first = (int64_t)blockIdx.x * G * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  int64_t r[G];
  int c0[G];
  i32x4 raw[G];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int64_t slice = first + 16 * u;
    r[u] = slice / nsl;
    c0[u] = (int)(slice - r[u] * nsl) * 128 + sub * 8;
    // cols % 8 == 0: a chunk is wholly valid or wholly padding
    const bool skip = r[u] >= skip_lo && r[u] < skip_to;
    if (slice < total && c0[u] < cols && !skip)
      raw[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(x + r[u] * ldx + c0[u]));
    else raw[u] = i32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < G; ++u) {
    if (first + 16 * u >= total) break;  // whole 16-lane groups leave together
    if (r[u] >= skip_lo && r[u] < skip_to) continue;  // a whole group: one slice is one row
    const bool valid = c0[u] < cols;
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint32_t)raw[u][i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32((uint32_t)raw[u][i] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = wave_max_width(amax, 16);
    const float s = div_rn(amax, 448.f);
    uint32_t lo = 0, hi = 0;
    if (s != 0.f && valid) {
      // |v| <= amax, so |v / s| <= 448 (1 + 2^-23) < 464
      const ScaleDiv d = make_scale_div(s);
      float qv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = scale_div(d, v[i]);
      lo = e4m3x4_hw(qv[0], qv[1], qv[2], qv[3]);
      hi = e4m3x4_hw(qv[4], qv[5], qv[6], qv[7]);
    }
    *reinterpret_cast<uint2*>(q + r[u] * ldq + c0[u]) = make_uint2(lo, hi);
    if (sub == 0) scales[r[u] * lds + (c0[u] >> 7)] = s;
  }
}

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int64_t ldx, uint8_t* q, int64_t ldq,
                            float* scales, int64_t lds, hipStream_t stream, const int32_t* skip_from, int skip_to) {
  const int64_t slices = (int64_t)rows * ((cols + 127) / 128);
  if (slices == 0) return hipSuccess;
  if (slices >= 65536)
    quant_act_kernel<4><<<(unsigned)ceil_div(slices, 64), 256, 0, stream>>>(x, rows, cols, ldx, q, ldq, scales, lds,
                                                                           skip_from, skip_to);
  else
    quant_act_kernel<1><<<(unsigned)ceil_div(slices, 16), 256, 0, stream>>>(x, rows, cols, ldx, q, ldq, scales, lds,
                                                                           skip_from, skip_to);
  return hipGetLastError();
}

// One workgroup per 128x128 block (weight preparation, not on the timed path).
__global__ __launch_bounds__(256) void quant_weight_blocks_kernel(const float* __restrict__ w, int rows, int cols,
                                                                  int64_t ldw, uint8_t* __restrict__ q,
                                                                  int64_t ldq, float* __restrict__ scales) {
  __shared__ float red[4];
  const int br = blockIdx.y, bc = blockIdx.x;
  const int r0 = br * 128, c0 = bc * 128;
  // each thread: 4 consecutive columns of 16 rows
  const int cc = (threadIdx.x & 31) * 4;
  const int rr = threadIdx.x >> 5;  // 0..7
  float amax = 0.f;
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + rr + 8 * i;
    const int c = c0 + cc;
    if (r < rows && c < cols) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(w + (int64_t)r * ldw + c);
#pragma unroll
      for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fabsf(v[k]));  // cols % 4 == 0
    }
  }
  amax = wave_max_width(amax, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = div_rn(amax, 448.f);
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + rr + 8 * i;
    const int c = c0 + cc;
    uint32_t word = 0;
    if (r < rows && c < cols && s != 0.f) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(w + (int64_t)r * ldw + c);
#pragma unroll
      for (int k = 0; k < 4; ++k) word |= e4m3_encode(div_rn(v[k], s)) << (8 * k);
    }
    *reinterpret_cast<uint32_t*>(q + (int64_t)r * ldq + c) = word;
  }
  if (threadIdx.x == 0) scales[(int64_t)br * gridDim.x + bc] = s;
}

hipError_t launch_quant_weight_blocks(const float* w, int rows, int cols, int64_t ldw, uint8_t* q, int64_t ldq,
                                      float* scales, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(cols, 128), (unsigned)ceil_div(rows, 128));
  quant_weight_blocks_kernel<<<grid, 256, 0, stream>>>(w, rows, cols, ldw, q, ldq, scales);
  return hipGetLastError();
}

}  // namespace dmoe
