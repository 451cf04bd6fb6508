// Grouped expert GEMMs for few rows per expert (decode): weight streaming.
//
// Same operation as the tile kernel in gemm.hip (gate/up with fused SwiGLU, or
// down; FP8 block-scale promotion per 128-wide K slice; Transformers docs
// "Dots3Note" and PR #47844), organised for the case where each expert sees a
// handful of rows and the weights are read once from HBM.
#include "gemm_common.h"

namespace dmoe {

// ---------------------------------------------------------------------------
// Weight-streaming kernel for few rows per expert (decode). Each wave owns 16
// output columns of one expert over the whole K: its lanes load the weight
// rows straight from HBM into MFMA B-operand registers (32 contiguous bytes per
// lane per 128-byte stage, so a wave reads full 128-byte lines of 16 rows), with
// a kRing-deep register prefetch ring; the few A rows come from L2. Up to 16*R
// rows of an expert are held at once; more rows loop (re-streaming the
// weights), which only happens when the host's per-expert estimate is low.
// Grid: (ceil(N_pad / 64), E_loc); experts without rows exit at once.
// ---------------------------------------------------------------------------
constexpr int kRing = 4;

template <int DT, bool GATEUP, int R>
__global__ __launch_bounds__(256) void gemm_stream_kernel(const TileArgs p, int n_cols) {
  const int e = blockIdx.y;
  const GroupView gv = group_view(p, e);
  const int row_beg = gv.row_beg, row_end = gv.row_end;
  if (row_beg >= row_end) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  if (n0 >= n_cols) return;
  const int64_t wcol = g4 * 32;
  const uint8_t* wg = gv.w0 + (int64_t)(n0 + r16) * p.ldw_b + wcol;
  const uint8_t* wu = GATEUP ? gv.w1 + (int64_t)(n0 + r16) * p.ldw_b + wcol : nullptr;
  const int nblk = n0 >> 7;
  const float* sw0 = DT == DMOE_FP8_E4M3 ? gv.s0 + (int64_t)nblk * p.nKb : nullptr;
  const float* sw1 = (DT == DMOE_FP8_E4M3 && GATEUP) ? gv.s1 + (int64_t)nblk * p.nKb : nullptr;
  constexpr int NM = GATEUP ? 2 : 1;  // weight matrices per wave

  for (int m0 = row_beg; m0 < row_end; m0 += 16 * R) {
    // The weight fragment is the MFMA's first operand: lane (r16, g4) ends up
    // with output row m0 + 16 i + r16 and columns n0 + 4 g4 .. n0 + 4 g4 + 3.
    const uint8_t* arow[R];
    bool aok[R];
    const float* asc[R];  // this lane's row of A scales
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int m = m0 + 16 * i + r16;
      aok[i] = m < row_end;
      const int64_t src = aok[i] ? a_row(p, gv, m) : 0;
      arow[i] = p.a + src * p.lda_b + wcol;
      asc[i] = DT == DMOE_FP8_E4M3 ? p.a_scales + src * p.ldas : nullptr;
    }
    f32x4 acc[NM][R];
#pragma unroll
    for (int t = 0; t < NM; ++t)
#pragma unroll
      for (int i = 0; i < R; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 rb[kRing][NM][2];
    i32x4 ra[kRing][R][2];
    auto issue = [&](int slot, int s) {
      const int64_t off = (int64_t)s * kKB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        rb[slot][0][h] = *reinterpret_cast<const i32x4*>(wg + off + 16 * h);
        if (GATEUP) rb[slot][NM - 1][h] = *reinterpret_cast<const i32x4*>(wu + off + 16 * h);
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ra[slot][i][h] = aok[i] ? *reinterpret_cast<const i32x4*>(arow[i] + off + 16 * h) : i32x4{0, 0, 0, 0};
    };
    auto compute = [&](int slot, int s) {
      if constexpr (DT == DMOE_FP8_E4M3 && GATEUP) {
        // exact products: E4M3 -> BF16 (exact), four BF16 MFMAs per 128-wide slice
        const float w0s = sw0[s];
        const float w1s = sw1[s];
        i32x4 b16[NM][4];
#pragma unroll
        for (int t = 0; t < NM; ++t) {
          e4m3x16_to_bf16(rb[slot][t][0], b16[t][0], b16[t][1]);
          e4m3x16_to_bf16(rb[slot][t][1], b16[t][2], b16[t][3]);
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
          i32x4 a16[4];
          e4m3x16_to_bf16(ra[slot][i][0], a16[0], a16[1]);
          e4m3x16_to_bf16(ra[slot][i][1], a16[2], a16[3]);
          const float sa = aok[i] ? asc[i][s] : 0.f;
#pragma unroll
          for (int t = 0; t < NM; ++t) {
            f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
              part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b16[t][k4]),
                                                             __builtin_bit_cast(bf16x8, a16[k4]), part, 0, 0, 0);
            const float saw = sa * (t == 0 ? w0s : w1s);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t][i][q] = fmaf(part[q], saw, acc[t][i][q]);
          }
        }
      } else if constexpr (DT == DMOE_FP8_E4M3) {
        const float w0s = sw0[s];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const i32x8 fa = i32x8{ra[slot][i][0][0], ra[slot][i][0][1], ra[slot][i][0][2], ra[slot][i][0][3],
                                 ra[slot][i][1][0], ra[slot][i][1][1], ra[slot][i][1][2], ra[slot][i][1][3]};
          const float saw = (aok[i] ? asc[i][s] : 0.f) * w0s;
          const i32x8 fb = i32x8{rb[slot][0][0][0], rb[slot][0][0][1], rb[slot][0][0][2], rb[slot][0][0][3],
                                 rb[slot][0][1][0], rb[slot][0][1][1], rb[slot][0][1][2], rb[slot][0][1][3]};
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb, fa, f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                               0, 0, 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[0][i][q] = fmaf(part[q], saw, acc[0][i][q]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const bf16x8 alo = __builtin_bit_cast(bf16x8, ra[slot][i][0]);
          const bf16x8 ahi = __builtin_bit_cast(bf16x8, ra[slot][i][1]);
#pragma unroll
          for (int t = 0; t < NM; ++t) {
            acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rb[slot][t][0]), alo,
                                                                acc[t][i], 0, 0, 0);
            acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rb[slot][t][1]), ahi,
                                                                acc[t][i], 0, 0, 0);
          }
        }
      }
    };

#pragma unroll
    for (int u = 0; u < kRing; ++u)
      if (u < p.stages) issue(u, u);
    for (int s0 = 0; s0 < p.stages; s0 += kRing) {
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
        const int s = s0 + u;
        if (s < p.stages) {
          compute(u, s);
          if (s + kRing < p.stages) issue(u, s + kRing);
        }
      }
    }

    const bool wide = (p.ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (!aok[i]) continue;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = GATEUP ? silu(acc[0][i][q]) * acc[NM - 1][i][q] : acc[0][i][q];
      const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
      uint16_t* o = p.out + (int64_t)(m0 + 16 * i + r16) * p.ldo + n0 + 4 * g4;
      if (wide) {
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
      } else {
        o[0] = (uint16_t)lo;
        o[1] = (uint16_t)(lo >> 16);
        o[2] = (uint16_t)hi;
        o[3] = (uint16_t)(hi >> 16);
      }
    }
  }
}

// The extra group is cut into chunks of p.x_chunk rows, one grid row each.
hipError_t launch_gemm_stream(const TileArgs& p, int dtype, bool gateup, int rows_per_expert, int n_pad,
                              int E_loc, hipStream_t stream) {
  const int R = rows_per_expert <= 16 ? 1 : 2;
  if (p.x_chunk != 16 * R) return hipErrorInvalidValue;
  const int xchunks = (int)ceil_div(p.x_rows, p.x_chunk);
  const dim3 grid((unsigned)(n_pad / 64), (unsigned)(E_loc + xchunks));
#define DMOE_STREAM(DTV, GU)                                                                         \
  do {                                                                                               \
    if (R == 1) gemm_stream_kernel<DTV, GU, 1><<<grid, 256, 0, stream>>>(p, n_pad);                  \
    else gemm_stream_kernel<DTV, GU, 2><<<grid, 256, 0, stream>>>(p, n_pad);                         \
  } while (0)
  if (dtype == DMOE_FP8_E4M3) {
    if (gateup) DMOE_STREAM(DMOE_FP8_E4M3, true);
    else DMOE_STREAM(DMOE_FP8_E4M3, false);
  } else {
    if (gateup) DMOE_STREAM(DMOE_BF16, true);
    else DMOE_STREAM(DMOE_BF16, false);
  }
#undef DMOE_STREAM
  return hipGetLastError();
}

}  // namespace dmoe
