// Grouped expert GEMMs for few rows per expert (decode): weight streaming
// through LDS.
//
// Same operation as the tile kernel in gemm.hip (gate/up with fused SwiGLU, or
// down; FP8 block-scale promotion per 128-wide K slice; Transformers documentation
// "Dots 3 Note Preview" and PR #47844), organised for the case where each expert sees a
// handful of rows and the weights are read once from HBM.
#include "gemm_common.h"

namespace dmoe {

// ---------------------------------------------------------------------------
// Weight-streaming kernel for few rows per expert (decode). A workgroup
// owns WR weight rows of one group: down, 64 rows = 64 columns of o, wave w
// multiplying columns 16 w .. 16 w + 15; gate/up, WR = 2 CW rows (CW gate rows,
// then the CW up rows of the same columns of h). With CW = 64 every wave
// multiplies the gate and the up rows of its 16 columns; with CW = 32 (the
// default) waves 0, 1 multiply the gate rows and waves 2, 3 the up rows of
// columns 16 (w & 1) .. + 15, and the up accumulators reach the gate waves
// through LDS for the SwiGLU epilogue. Narrower workgroups halve the work per
// workgroup, so the last partial round of workgroups (all do the same
// weight traffic) costs half as much. Every 128-byte K stage of the rows, of
// the group's (up to 16 R) A rows and of their FP8 scales moves global -> LDS
// with direct loads (each instruction covers 8 whole 128-byte lines) through a
// ring of kRingBF16 or kRingFP8 stages (a 128-byte BF16 stage holds half the K
// of an FP8 one). Grid: (N_pad / CW, chunks + E_loc).
// ---------------------------------------------------------------------------
#ifndef DMOE_STAGE_RING_BF16
#define DMOE_STAGE_RING_BF16 6
#endif
#ifndef DMOE_STAGE_RING_FP8
#define DMOE_STAGE_RING_FP8 4
#endif
#ifndef DMOE_STREAM_GATEUP_CW
#define DMOE_STREAM_GATEUP_CW 32
#endif
constexpr int kRingBF16 = DMOE_STAGE_RING_BF16, kRingFP8 = DMOE_STAGE_RING_FP8;
constexpr int kGateUpCW = DMOE_STREAM_GATEUP_CW;
static_assert(kGateUpCW == 32 || kGateUpCW == 64, "gate/up column block");

template <int DT, bool GATEUP, int R>
__global__ __launch_bounds__(256) void gemm_stage_kernel(const TileArgs p, int n_cols) {
  constexpr bool kFP8 = DT == DMOE_FP8_E4M3;
  constexpr int CW = GATEUP ? kGateUpCW : 64;  // output columns per workgroup
  constexpr int WR = GATEUP ? 2 * CW : 64;     // weight rows per workgroup
  constexpr bool kSplit = GATEUP && CW == 32;  // gate and up rows on different waves
  constexpr int AR = 16 * R;              // A rows per pass
  constexpr int kRows = WR + AR;
  constexpr int NS = kFP8 ? kRingFP8 : kRingBF16;
  constexpr int kCopiesA = 1 + (kFP8 ? 1 : 0);  // A-row (+ scale) copies per wave per stage
  constexpr int kCopies = WR / 32 + kCopiesA;    // direct copies per wave per stage
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS][kRows * 128];
  __shared__ __attribute__((aligned(256))) float lsa[NS][32];
  __shared__ float lsw[2][kMaxSlices];
  __shared__ f32x4 xup[kSplit ? 2 * R * 64 : 1];  // up accumulators of waves 2, 3
  asm volatile("" ::"v"(&ring[0][0]), "v"(&lsa[0][0]) : "memory");

  // Grid rows 0 .. chunks-1 are the extra group's row chunks, the rest the
  // routed experts: the chunks, which all read the same weights, are dispatched
  // first and together, and the last, partly filled round of workgroups is
  // left to routed experts.
  const int chunks = (int)gridDim.y - p.E_loc;
  const int g = (int)blockIdx.y < chunks ? p.E_loc + (int)blockIdx.y : (int)blockIdx.y - chunks;
  const GroupView gv = group_view(p, g);
  const int row_beg = gv.row_beg, row_end = gv.row_end;
  if (row_beg >= row_end) return;
  const int n0 = blockIdx.x * CW;
  if (n0 >= n_cols) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int S = p.stages;

  // weight block scales of the workgroup's 64 columns (one 128-row block)
  if constexpr (kFP8) {
    for (int i = tid; i < (GATEUP ? 2 : 1) * p.nKb; i += 256) {
      const int w = i / p.nKb, sl = i - w * p.nKb;
      lsw[w][sl] = (w == 0 ? gv.s0 : gv.s1)[(int64_t)(n0 >> 7) * p.nKb + sl];
    }
  }
  __syncthreads();

  // weight copies: copy i of wave w fills LDS rows 8 (4 i + w) .. + 7
  const uint8_t* srcB[WR / 32];
#pragma unroll
  for (int i = 0; i < WR / 32; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    const uint8_t* base = (GATEUP && row >= CW) ? gv.w1 : gv.w0;
    srcB[i] = base + (int64_t)(n0 + row % CW) * p.ldw_b + 16 * swz(row, lane & 7);
  }

  // A routed expert whose rows fit one pass reads its weights exactly once:
  // stream them with the non-temporal policy. The shared expert's row chunks
  // and multi-pass experts read the same weights again and keep the default.
  const bool read_once = g < p.E_loc && row_end - row_beg <= AR;

  const int S0 = min(NS - 1, S);  // stages issued ahead of the ring loop
  for (int m0 = row_beg; m0 < row_end; m0 += AR) {
    // Weight copies of stage s; they need no row index.
    auto issue_w = [&](int s) {
      uint8_t* st = ring[s % NS];
      const int64_t off = (int64_t)s * 128;
#pragma unroll
      for (int i = 0; i < WR / 32; ++i) {
        if (read_once) lds_copy16_nt(srcB[i] + off, st + (8 * (4 * i + wave)) * 128);
        else lds_copy16(srcB[i] + off, st + (8 * (4 * i + wave)) * 128);
      }
    };
    // The first stages' weight copies go out before the A rows' token indices
    // are loaded, so the ring fill waits for one memory round trip instead of
    // two in a row (token index, then weights).
    for (int s = 0; s < S0; ++s) issue_w(s);

    // A copy of wave w: rows (AR / 4) w .. + AR / 4 - 1 (R = 1: lanes 0..31)
    const int arow_l = (AR / 4) * wave + (lane >> 3);
    const bool a_lane = lane < 2 * AR;  // 8 lanes per row, AR / 4 rows per wave
    const int am = m0 + arow_l;
    const int64_t a_src = a_row(p, gv, am < row_end ? am : m0);
    const uint8_t* srcA = p.a + a_src * p.lda_b + 16 * swz(WR + arow_l, lane & 7);
    // scale copy of wave w: rows 8 w + lane (lanes 0..7)
    const int srow_l = 8 * wave + lane;
    const int sm = m0 + srow_l;
    const float* srcS = kFP8 ? p.a_scales + a_row(p, gv, (lane < 8 && sm < row_end) ? sm : m0) * p.ldas : nullptr;

    // A-row and activation-scale copies of stage s (kCopiesA per wave)
    auto issue_a = [&](int s) {
      uint8_t* st = ring[s % NS];
      const int64_t off = (int64_t)s * 128;
      if (a_lane) lds_copy16(srcA + off, st + (WR + (AR / 4) * wave) * 128);
      if (kFP8 && lane < 8) lds_copy4(srcS + s, &lsa[s % NS][8 * wave]);
    };

    // weight fragments per wave: gate and up (CW = 64), or one of them
    constexpr int NM = (GATEUP && !kSplit) ? 2 : 1;
    f32x4 acc[NM][R];
#pragma unroll
    for (int t = 0; t < NM; ++t)
#pragma unroll
      for (int i = 0; i < R; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int s) {
      const uint8_t* st = ring[s % NS];
      // weight fragments of this wave's 16 columns (first MFMA operand), A fragments (second)
      i32x4 fb[NM][2], fa[R][2];
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const int row = 64 * t + 16 * wave + r16;  // kSplit: rows 16 wave .. (gate, then up)
        fb[t][0] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4));
        fb[t][1] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4 + 1));
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int row = WR + 16 * i + r16;
        fa[i][0] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4));
        fa[i][1] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4 + 1));
      }
      if constexpr (kFP8 && GATEUP) {
        // exact products: E4M3 -> BF16 (exact), four BF16 MFMAs per 128-wide slice
        i32x4 b16[NM][4];
#pragma unroll
        for (int t = 0; t < NM; ++t) {
          e4m3x16_to_bf16(fb[t][0], b16[t][0], b16[t][1]);
          e4m3x16_to_bf16(fb[t][1], b16[t][2], b16[t][3]);
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
          i32x4 a16[4];
          e4m3x16_to_bf16(fa[i][0], a16[0], a16[1]);
          e4m3x16_to_bf16(fa[i][1], a16[2], a16[3]);
          const float sa = lsa[s % NS][16 * i + r16];
#pragma unroll
          for (int t = 0; t < NM; ++t) {
            f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
              part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b16[t][k4]),
                                                             __builtin_bit_cast(bf16x8, a16[k4]), part, 0, 0, 0);
            const float saw = sa * lsw[kSplit ? wave >> 1 : t][s];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t][i][q] = fmaf(part[q], saw, acc[t][i][q]);
          }
        }
      } else if constexpr (kFP8) {
        const i32x8 b8 = i32x8{fb[0][0][0], fb[0][0][1], fb[0][0][2], fb[0][0][3],
                               fb[0][1][0], fb[0][1][1], fb[0][1][2], fb[0][1][3]};
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const i32x8 a8 = i32x8{fa[i][0][0], fa[i][0][1], fa[i][0][2], fa[i][0][3],
                                 fa[i][1][0], fa[i][1][1], fa[i][1][2], fa[i][1][3]};
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                               0, 0, 0, 0, 0);
          const float saw = lsa[s % NS][16 * i + r16] * lsw[0][s];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[0][i][q] = fmaf(part[q], saw, acc[0][i][q]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int t = 0; t < NM; ++t) {
            acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb[t][0]),
                                                                __builtin_bit_cast(bf16x8, fa[i][0]), acc[t][i], 0, 0, 0);
            acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb[t][1]),
                                                                __builtin_bit_cast(bf16x8, fa[i][1]), acc[t][i], 0, 0, 0);
          }
      }
    };

    // ---- NS-stage ring: stage s lives in buffer s % NS ----
    // Issue order per wave: W(0 .. S0-1), A(0 .. S0-1), then W(s) A(s) for
    // s = S0, S0+1, ... So stage s < NS - 1 is complete once at most the
    // A copies of stages s+1 .. NS-2 and the s+1 stages issued in the loop
    // are in flight; (NS - 2) kCopiesA + kCopies is the smallest of those
    // counts (s = 0), conservative for 0 < s < NS - 1.
    for (int s = 0; s < S0; ++s) issue_a(s);
    for (int s = 0; s < S; ++s) {
      if (s + NS - 1 < S) {
        issue_w(s + NS - 1);
        issue_a(s + NS - 1);
        if (s < NS - 1) wait_vmcnt<(NS - 2) * kCopiesA + kCopies>();
        else wait_vmcnt<kCopies * (NS - 1)>();  // at most the NS-1 younger stages in flight
      } else {
        wait_vmcnt<0>();
      }
      stage_barrier();  // every wave's copies of stage s have landed in LDS
      compute(s);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
      stage_barrier();  // buffer s % NS may be refilled
    }

    // ---- epilogue: lane (r16, g4) holds row m0 + 16 i + r16, columns n0 + 16 wave' + 4 g4 + q
    // (wave' = wave, or wave & 1 when the gate and up rows sit on different waves) ----
    f32x4 up[R];
    if constexpr (kSplit) {
      // the previous pass's readers of xup finished before the stage barriers of this pass
      if (wave >= 2) {
#pragma unroll
        for (int i = 0; i < R; ++i) xup[((wave - 2) * R + i) * 64 + lane] = acc[0][i];
      }
      __syncthreads();
      if (wave >= 2) continue;
#pragma unroll
      for (int i = 0; i < R; ++i) up[i] = xup[(wave * R + i) * 64 + lane];
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) up[i] = acc[NM - 1][i];
    }
    const bool wide = (p.ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int m = m0 + 16 * i + r16;
      if (m >= row_end) continue;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = GATEUP ? silu(acc[0][i][q]) * up[i][q] : acc[0][i][q];
      const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
      uint16_t* o = p.out + (int64_t)m * p.ldo + n0 + 16 * (kSplit ? wave & 1 : wave) + 4 * g4;
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
  const int cw = gateup ? kGateUpCW : 64;
  const dim3 grid((unsigned)(n_pad / cw), (unsigned)(E_loc + xchunks));
#define DMOE_STREAM(DTV, GU)                                                                         \
  do {                                                                                               \
    if (R == 1) gemm_stage_kernel<DTV, GU, 1><<<grid, 256, 0, stream>>>(p, n_pad);                   \
    else gemm_stage_kernel<DTV, GU, 2><<<grid, 256, 0, stream>>>(p, n_pad);                          \
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
