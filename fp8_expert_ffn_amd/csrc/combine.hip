// Deterministic gather combine of the expert outputs back into token order:
// y[t] = bf16( sum_k w[t,k] * o[token_row[t,k]] + shared[t] ), FP32 in slot
// order. The routed weights come from the renormalised top-K router
// (Dots3NoteTextConfig norm_topk_prob, routed_scaling_factor = 1) and the
// shared expert is added with weight 1 (n_shared_experts = 1).
#include "dmoe_internal.h"

namespace dmoe {

// Grid (T, ceil(H / 1024)): one workgroup per token and 1024-column chunk,
// 8 BF16 columns (16 bytes) per thread.
__global__ __launch_bounds__(128) void combine_kernel(const uint16_t* __restrict__ o, int64_t ldo,
                                                      const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ s, int64_t lds, int T_s, int K,
                                                      int H, uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t t = blockIdx.x;
  const int c = blockIdx.y * 1024 + threadIdx.x * 8;
  if (c >= H) return;
  const bool shared = s != nullptr && t < T_s;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int k = 0; k < K; ++k) {
    const int32_t r = token_row[t * K + k];
    if (r < 0) continue;
    const float wk = w[t * K + k];
    const i32x4 raw = *reinterpret_cast<const i32x4*>(o + (int64_t)r * ldo + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(wk, bf16_to_f32((uint32_t)raw[i] & 0xffffu), acc[2 * i]);
      acc[2 * i + 1] = fmaf(wk, bf16_to_f32((uint32_t)raw[i] >> 16), acc[2 * i + 1]);
    }
  }
  if (shared) {
    const i32x4 raw = *reinterpret_cast<const i32x4*>(s + t * lds + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32((uint32_t)raw[i] & 0xffffu);
      acc[2 * i + 1] += bf16_to_f32((uint32_t)raw[i] >> 16);
    }
  }
  i32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = (int)pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<i32x4*>(y + t * ldy + c) = out;
}

hipError_t launch_combine(const uint16_t* o, int64_t ldo, const int32_t* token_row, const float* w,
                          const uint16_t* s, int64_t lds, int T_s, int T, int K, int H, uint16_t* y, int64_t ldy,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)ceil_div(H, 1024));
  combine_kernel<<<grid, 128, 0, stream>>>(o, ldo, token_row, w, s, lds, T_s, K, H, y, ldy);
  return hipGetLastError();
}

}  // namespace dmoe
