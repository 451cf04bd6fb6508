// Grouped expert GEMMs: gate/up with fused SwiGLU, and down.
//
// Expert FFN: hidden_act silu over gate_proj/up_proj, then down_proj, no bias
// (Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig hidden_act, mlp_bias);
// 256 routed experts of width 1536 on hidden 5120 (model card
// "dots-studio/dots3-note-prev", Model Overview table). FP8: E4M3 weights
// with one FP32 scale per 128x128 block and dynamic activation scales per 1x128
// slice (Transformers PR #47844, implementation list), so every 128-wide K
// slice's integer-grid product is scaled by a_scale * w_scale before it is
// added to the FP32 accumulator. Dimensions that are not multiples of 128 use
// zero-padded weights and activations (PR #47844, validation list).
//
// Work decomposition: a schedule kernel turns the per-expert row offsets into
// a list of (expert, first row) tiles of kBM rows; the GEMM grid is sized from
// the host-known bound (max_rows / kBM + E_loc tiles) and surplus workgroups
// exit on the device. A workgroup owns kBM rows x (32 * NT) weight rows and
// walks K in 128-byte stages (128 FP8 or 64 BF16 elements) through an LDS ring.
#include <type_traits>

#include "gemm_common.h"

namespace dmoe {

// Tiles past `cap` (only possible when the caller's max_rows understates the
// real row count) are dropped rather than written past the workspace. The
// extra group's tiles (group index E_loc) follow the routed ones.
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ offsets, int E_loc, int bm,
                                                        int x_rows, int x_row0, int cap, int2* __restrict__ tiles,
                                                        int32_t* __restrict__ ntiles) {
  __shared__ int32_t start[1025];
  __shared__ int32_t partial[1024];
  const int t = threadIdx.x;
  // per-thread contiguous chunk of experts
  const int chunk = (E_loc + blockDim.x - 1) / blockDim.x;
  const int b = min(E_loc, t * chunk), e = min(E_loc, b + chunk);
  int32_t s = 0;
  for (int i = b; i < e; ++i) {
    const int32_t n = (offsets[i + 1] - offsets[i] + bm - 1) / bm;
    start[i] = n;
    s += n;
  }
  partial[t] = s;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const int32_t add = t >= off ? partial[t - off] : 0;
    __syncthreads();
    partial[t] += add;
    __syncthreads();
  }
  int32_t run = partial[t] - s;
  for (int i = b; i < e; ++i) {
    const int32_t n = start[i];
    const int32_t r0 = offsets[i];
    for (int k = 0; k < n && run + k < cap; ++k) tiles[run + k] = make_int2(i, r0 + k * bm);
    run += n;
  }
  const int32_t routed = partial[blockDim.x - 1];
  const int32_t nx = (x_rows + bm - 1) / bm;
  for (int k = t; k < nx; k += blockDim.x)
    if (routed + k < cap) tiles[routed + k] = make_int2(E_loc, x_row0 + k * bm);
  if (t == (int)blockDim.x - 1) *ntiles = min(routed + nx, cap);
}


// Tile kernel. A workgroup (2 x WN waves) owns kBM = 128 rows of one group and
// 16 * NT * WN weight rows (gate/up: 8 * NT * WN gate + as many up rows, i.e.
// 8 * NT * WN columns of h; down: 16 * NT * WN columns of o). Wave (wm, wn),
// wm in {0, 1}, wn in [0, WN), computes 16 * MT rows x 16 * NT weight rows as
// MT x NT MFMA tiles of 16x16, rows [16 MT wm, 16 MT wm + 16 MT): MT = 4 covers
// the 128 rows, and the last tile of a group runs with MT = ceil(rows / 32) so
// that short tiles cost MFMA work in proportion to their rows. WN = 2 (256
// threads, two workgroups per CU) or WN = 4 (512 threads, one workgroup per CU
// sharing each A stage over twice the weight rows). Operands move global -> LDS
// with direct (asynchronous, register-free) loads through an NS-stage ring; a
// stage is 128 bytes of every A and weight row (one 128-wide FP8 scale slice,
// or 64 BF16 elements) plus the A rows' activation scales. LDS rows are 128
// bytes with 16-byte units XOR-swizzled (swz in gemm_common.h) so that the
// fragment reads are free of bank conflicts. Grid: 1-D, tile-major, column
// block fastest.

// Build-time tuning knobs; the defaults are the measured best on gfx950 (the
// alternatives stay buildable for re-measurement): ring depth NS (2 with two
// workgroups per CU), waves per SIMD, an XCD-contiguous work order, column
// tiles per wave NT, column waves WN (and the ring depth used with WN = 4), and
// the ceil(rows / 32) row subtiles for short tiles.
#ifndef DMOE_TILE_NS
#define DMOE_TILE_NS 2
#endif
#ifndef DMOE_TILE_WAVES_PER_EU
#define DMOE_TILE_WAVES_PER_EU 2
#endif
#ifndef DMOE_TILE_XCD_REMAP
#define DMOE_TILE_XCD_REMAP 0
#endif
#ifndef DMOE_TILE_NT_GATEUP
#define DMOE_TILE_NT_GATEUP 4
#endif
#ifndef DMOE_TILE_NT_DOWN
#define DMOE_TILE_NT_DOWN 4
#endif
#ifndef DMOE_TILE_WN_GATEUP
#define DMOE_TILE_WN_GATEUP 2
#endif
#ifndef DMOE_TILE_WN_DOWN
#define DMOE_TILE_WN_DOWN 2
#endif
#ifndef DMOE_TILE_NS_WIDE
#define DMOE_TILE_NS_WIDE 3
#endif
#ifndef DMOE_TILE_MT_FINE
#define DMOE_TILE_MT_FINE 1
#endif

template <int MODE, bool GATEUP, int NS, int NT, int WN>
__global__ __launch_bounds__(128 * WN, NT == 4 ? DMOE_TILE_WAVES_PER_EU : 1) void gemm_tile_kernel(
    const TileArgs p, int nNB, int n_valid) {
  constexpr bool kScaled = MODE != kModeBF16;
  constexpr int kThreads = 128 * WN, kWaves = 2 * WN;
  constexpr int NH = NT / 2;               // gate/up: NH gate subtiles, then NH up subtiles per wave
  constexpr int kRowsB = 16 * NT * WN;     // weight rows per workgroup
  constexpr int kHalfB = kRowsB / 2;       // gate/up: gate rows, then as many up rows
  constexpr int kRows = kBM + kRowsB;      // A rows, then weight rows
  constexpr int kInstA = kBM / (8 * kWaves), kInstB = kRowsB / (8 * kWaves);  // direct copies per wave per stage
  static_assert(kInstA * 8 * kWaves == kBM && kInstB * 8 * kWaves == kRowsB, "copy split");
  static_assert(!GATEUP || kHalfB <= 128, "gate/up: one weight scale block per workgroup");
  static_assert(NS >= 2 && NS <= 4, "pipeline depth");
  // One LDS variable per stage so that each stage is a distinct object.
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kRows * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kRows * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[NS > 2 ? kRows * 128 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[NS > 3 ? kRows * 128 : 16];
  __shared__ __attribute__((aligned(256))) float lsa0[kBM];
  __shared__ __attribute__((aligned(256))) float lsa1[kBM];
  __shared__ __attribute__((aligned(256))) float lsa2[NS > 2 ? kBM : 4];
  __shared__ __attribute__((aligned(256))) float lsa3[NS > 3 ? kBM : 4];
  auto stage_ptr = [&](auto uc) -> uint8_t* {
    constexpr int u = decltype(uc)::value;
    if constexpr (u == 0) return lds0;
    else if constexpr (u == 1) return lds1;
    else if constexpr (u == 2) return lds2;
    else return lds3;
  };
  auto scale_ptr = [&](auto uc) -> float* {
    constexpr int u = decltype(uc)::value;
    if constexpr (u == 0) return lsa0;
    else if constexpr (u == 1) return lsa1;
    else if constexpr (u == 2) return lsa2;
    else return lsa3;
  };

  // The direct copies write LDS from asm that sees only integer M0 bases; hand
  // the buffers' addresses to an asm statement once so that the compiler
  // treats them as escaped and every later memory-clobbering asm (the copies,
  // the barriers) as a possible writer of them.
  asm volatile("" ::"v"(lds0), "v"(lds1), "v"(lds2), "v"(lds3), "v"(lsa0), "v"(lsa1), "v"(lsa2), "v"(lsa3)
               : "memory");

#if DMOE_TILE_XCD_REMAP
  // Workgroups are dealt to the 8 XCDs round robin (XCD = blockIdx % 8); give
  // each XCD one contiguous range of the real work items (tile-major, column
  // block fastest) so that a tile's A rows and an expert's weights are fetched
  // into one XCD's L2 instead of all eight. The grid is a multiple of 8.
  const int nitems = *p.ntiles * nNB;
  const int per_xcd = (nitems + 7) >> 3;
  const int L = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || L >= nitems) return;
  const int tile = L / nNB, nb = L - tile * nNB;
#else
  const int L = blockIdx.x;
  const int tile = L / nNB, nb = L - tile * nNB;
  if (tile >= *p.ntiles) return;
#endif
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const GroupView gv = group_view(p, e);
  const int m_end = gv.row_end;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g4 = lane >> 4;
  // first h (gate/up) or o (down) column of the workgroup and of this wave
  const int ncol0 = nb * (GATEUP ? kHalfB : kRowsB);
  const int wcol0 = ncol0 + wn * 16 * (GATEUP ? NH : NT);
  const bool active = GATEUP || wcol0 < n_valid;  // down: waves past N only help with the copies

  // Direct-copy sources: copy i of this wave fills LDS rows 8*(kWaves*i+wave) .. +7,
  // lane -> row 8*(kWaves*i+wave) + lane/8, 16-byte position lane%8.
  int64_t srcA[kInstA];
  const uint8_t* srcB[kInstB];
#pragma unroll
  for (int i = 0; i < kInstA; ++i) {
    const int row = 8 * (kWaves * i + wave) + (lane >> 3);
    const int m = m0 + row;
    const int64_t arow = a_row(p, gv, m < m_end ? m : m0);  // rows past the group reuse a valid row
    srcA[i] = arow * p.lda_b + 16 * swz(row, lane & 7);
  }
#pragma unroll
  for (int i = 0; i < kInstB; ++i) {
    const int row = 8 * (kWaves * i + wave) + (lane >> 3);
    int64_t wrow;
    const uint8_t* base;
    if (GATEUP) {
      wrow = ncol0 + (row % kHalfB);
      base = row < kHalfB ? gv.w0 : gv.w1;
    } else {
      wrow = ncol0 + row < n_valid ? ncol0 + row : 0;  // rows past N (inactive waves) reread row 0
      base = gv.w0;
    }
    srcB[i] = base + wrow * p.ldw_b + 16 * swz(row, lane & 7);
  }
  int64_t srcS = 0;  // waves 0 and 1 copy the activation scales of rows 64*wave + lane
  if (kScaled && wave < 2) {
    const int m = m0 + 64 * wave + lane;
    srcS = a_row(p, gv, m < m_end ? m : m0) * p.ldas;
  }
  // Weight block scales staged in LDS before the pipeline starts: gate/up: the
  // 128-row block of the gate and of the up rows; down: the block of each
  // column-wave's 16*NT columns.
  constexpr int kScaleSets = GATEUP ? 2 : WN;
  __shared__ float lsw[kScaleSets][kMaxSlices];
  if constexpr (kScaled) {
    for (int i = tid; i < kScaleSets * p.nKb; i += kThreads) {
      const int w = i / p.nKb, sl = i - w * p.nKb;
      if (GATEUP) {
        lsw[w][sl] = (w == 0 ? gv.s0 : gv.s1)[(int64_t)(ncol0 >> 7) * p.nKb + sl];
      } else {
        const int col = ncol0 + w * 16 * NT;
        lsw[w][sl] = col < n_valid ? gv.s0[(int64_t)(col >> 7) * p.nKb + sl] : 0.f;
      }
    }
  }
  __syncthreads();

  // Copies address their source as a wave-uniform base (SGPRs) plus a 32-bit
  // per-lane byte offset: advancing a stage is a scalar add. Every offset
  // fits in 32 bits because each operand spans less than 4 GiB (checked by the
  // entry points; a caller-supplied row_token must stay within that span).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t aoff[kInstA], boff[kInstB];
#pragma unroll
  for (int i = 0; i < kInstA; ++i) aoff[i] = (uint32_t)srcA[i];
  const uint8_t* bb0 = uniform_ptr(GATEUP ? gv.w0 + (int64_t)ncol0 * p.ldw_b : gv.w0);
  const uint8_t* bb1 = uniform_ptr(GATEUP ? gv.w1 + (int64_t)ncol0 * p.ldw_b : gv.w0);
  static_assert(!GATEUP || kHalfB % (8 * kWaves) == 0, "a copy covers gate rows or up rows only");
#pragma unroll
  for (int i = 0; i < kInstB; ++i)
    boff[i] = (uint32_t)(srcB[i] - ((GATEUP && 8 * kWaves * i >= kHalfB) ? bb1 : bb0));
  const uint32_t soff = (uint32_t)(srcS * 4);
  auto issue = [&](auto uc, int s) {
    const uint32_t st = (uint32_t)(uintptr_t)stage_ptr(uc);
    const int64_t off = (int64_t)s * 128;
#pragma unroll
    for (int i = 0; i < kInstA; ++i) lds_copy16_s(p.a + off, aoff[i], st + (8 * kWaves * i + 8 * wave_u) * 128);
#pragma unroll
    for (int i = 0; i < kInstB; ++i)
      lds_copy16_s(((GATEUP && 8 * kWaves * i >= kHalfB) ? bb1 : bb0) + off, boff[i],
                   st + (kBM + 8 * kWaves * i + 8 * wave_u) * 128);
    if (kScaled && wave < 2)
      lds_copy4_s(p.a_scales + s, soff, (uint32_t)(uintptr_t)scale_ptr(uc) + 256 * wave_u);
  };

  // A tile of r < 128 rows (the last tile of a group) runs with MT =
  // ceil(r / 32) row subtiles per wave (wave rows 16 MT wm .. 16 MT wm + 16 MT - 1)
  // instead of 4; the copies are the same.
  auto run = [&](auto mtc) {
    constexpr int MT = decltype(mtc)::value;
    f32x4 acc[MT][NT];
  #pragma unroll
    for (int i = 0; i < MT; ++i)
  #pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // weight rows (within the weight region) of this lane's subtiles; the
    // weight fragment is the first MFMA operand, the A fragment the second
    auto brow = [&](int j) -> int {
      if (GATEUP) return (j < NH ? 0 : kHalfB) + wn * 16 * NH + 16 * (j % NH) + r16;
      return wn * 16 * NT + 16 * j + r16;
    };

    auto compute = [&](auto uc, int s) {
      const uint8_t* st = stage_ptr(uc);
      const float* lsa = scale_ptr(uc);
      i32x4 fa[MT][2];
  #pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = 16 * MT * wm + 16 * i + r16;
        fa[i][0] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4));
        fa[i][1] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4 + 1));
      }
      // a_scale * w_scale of this stage's slice for the lane's row of each
      // subtile (index 0: gate or down weights, 1: up weights)
      float saw[GATEUP ? 2 : 1][MT];
      if constexpr (kScaled) {
        const float w0s = GATEUP ? lsw[0][s] : lsw[wn][s];
        const float w1s = GATEUP ? lsw[1][s] : 0.f;
  #pragma unroll
        for (int i = 0; i < MT; ++i) {
          const float a = lsa[16 * MT * wm + 16 * i + r16];
          saw[0][i] = a * w0s;
          if constexpr (GATEUP) saw[GATEUP ? 1 : 0][i] = a * w1s;
        }
      }
      if constexpr (MODE == kModeFP8X) {
        // exact products: codes -> BF16, four 16x16x32 MFMAs per 128-wide slice,
        // software-pipelined over the column tiles: tile j + 1's weight fragment is
        // converted and tile j - 1's sums promoted between tile j's MFMAs, so that
        // the VALU work never waits on a matrix-core result just issued (measured:
        // prefill gate/up 2.60 -> 2.55 ms)
        i32x4 a16[MT][4];
  #pragma unroll
        for (int i = 0; i < MT; ++i) {
          e4m3x16_to_bf16(fa[i][0], a16[i][0], a16[i][1]);
          e4m3x16_to_bf16(fa[i][1], a16[i][2], a16[i][3]);
        }
        auto bconv = [&](int j, i32x4 (&b16)[4]) {
          const int bj = brow(j);
          const uint8_t* bp = st + (kBM + bj) * 128;
          e4m3x16_to_bf16(*reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4)), b16[0], b16[1]);
          e4m3x16_to_bf16(*reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4 + 1)), b16[2], b16[3]);
        };
        auto promote = [&](int j, const f32x4 (&sums)[MT]) {
          const int wsel = (GATEUP && j >= NH) ? 1 : 0;
  #pragma unroll
          for (int i = 0; i < MT; ++i)
  #pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sums[i][r], saw[wsel][i], acc[i][j][r]);
        };
        i32x4 bcur[4], bnext[4];
        bconv(0, bcur);
        f32x4 prev[MT];
  #pragma unroll
        for (int j = 0; j < NT; ++j) {
          if (j + 1 < NT) bconv(j + 1, bnext);
          f32x4 cur[MT];
  #pragma unroll
          for (int i = 0; i < MT; ++i) {
            cur[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
              cur[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bcur[k4]),
                                                               __builtin_bit_cast(bf16x8, a16[i][k4]), cur[i], 0, 0, 0);
          }
          if (j > 0) promote(j - 1, prev);
  #pragma unroll
          for (int i = 0; i < MT; ++i) prev[i] = cur[i];
          if (j + 1 < NT) {
  #pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) bcur[k4] = bnext[k4];
          }
        }
        promote(NT - 1, prev);
      } else if constexpr (MODE == kModeFP8) {
  #pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int bj = brow(j);
          const uint8_t* bp = st + (kBM + bj) * 128;
          const i32x4 b0 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4));
          const i32x4 b1 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4 + 1));
          const i32x8 b8 = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          const int wsel = (GATEUP && j >= NH) ? 1 : 0;
  #pragma unroll
          for (int i = 0; i < MT; ++i) {
            const i32x8 a8 = i32x8{fa[i][0][0], fa[i][0][1], fa[i][0][2], fa[i][0][3],
                                   fa[i][1][0], fa[i][1][1], fa[i][1][2], fa[i][1][3]};
            const f32x4 pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                               0, 0, 0, 0);
  #pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(pr[r], saw[wsel][i], acc[i][j][r]);
          }
        }
      } else {
  #pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int bj = brow(j);
          const uint8_t* bp = st + (kBM + bj) * 128;
          const i32x4 b0 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4));
          const i32x4 b1 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4 + 1));
  #pragma unroll
          for (int i = 0; i < MT; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b0),
                                                                __builtin_bit_cast(bf16x8, fa[i][0]), acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b1),
                                                                __builtin_bit_cast(bf16x8, fa[i][1]), acc[i][j], 0, 0, 0);
          }
        }
      }
    };

    // ---- NS-stage pipeline: stage s lives in buffer s % NS ----
    constexpr int kCopies = kInstA + kInstB;  // per wave per stage, plus one scale copy on waves 0 and 1
    const int S = p.stages;
    const bool scale_wave = kScaled && wave < 2;
    // Two schedules. One barrier per stage (gate/up and BF16 down): the ring
    // starts full (stages 0 .. NS-1) and stage s + NS - 1 is issued once every
    // wave has passed the barrier of stage s, i.e. is done with stage s - 1,
    // whose buffer it refills. Two barriers per stage (FP8 down, whose stages
    // hold little MFMA work and wait on first-touch weight reads): stage
    // s + NS - 1 is issued before the wait for stage s, right after the barrier
    // that releases buffer (s - 1) % NS, which keeps one more stage's latency
    // covered; measured faster there, slower for the others.
    constexpr bool kOneBarrier = GATEUP || MODE == kModeBF16;
    if constexpr (!kOneBarrier) {
      static_for<0, NS - 1>([&](auto uc) {
        if (decltype(uc)::value < S) issue(uc, decltype(uc)::value);
      });
      for (int s0 = 0; s0 < S; s0 += NS) {
        static_for<0, NS>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          const int s = s0 + u;
          if (s < S) {
            if (s + NS - 1 < S) {
              issue(std::integral_constant<int, (u + NS - 1) % NS>{}, s + NS - 1);
              // stage s is complete once at most the NS-1 younger stages are in flight
              if (scale_wave) wait_vmcnt<(kCopies + 1) * (NS - 1)>();
              else wait_vmcnt<kCopies * (NS - 1)>();
            } else {
              wait_vmcnt<0>();
            }
            stage_barrier();  // every wave's copies of stage s have landed in LDS
            if (active) compute(uc, s);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
            stage_barrier();  // buffer u may be refilled
          }
        });
      }
    } else {
      static_for<0, NS>([&](auto uc) {
        if (decltype(uc)::value < S) issue(uc, decltype(uc)::value);
      });
      for (int s0 = 0; s0 < S; s0 += NS) {
        static_for<0, NS>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          const int s = s0 + u;
          if (s < S) {
            // stage s is complete once at most the stages issued after it are in flight:
            // s+1 .. s+NS-1 at s = 0 (the full ring), s+1 .. s+NS-2 afterwards
            const int younger = min(S - 1, s == 0 ? NS - 1 : s + NS - 2) - s;
            if (younger >= NS - 1) {
              if (scale_wave) wait_vmcnt<(kCopies + 1) * (NS - 1)>();
              else wait_vmcnt<kCopies * (NS - 1)>();
            } else if (NS > 2 && younger >= NS - 2) {
              if (scale_wave) wait_vmcnt<(kCopies + 1) * (NS > 2 ? NS - 2 : 0)>();
              else wait_vmcnt<kCopies * (NS > 2 ? NS - 2 : 0)>();
            } else {
              wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage s-1 are done
            // one barrier per stage: every wave's copies of stage s have landed, and every wave is done
            // with buffer (s-1) % NS, which the copies of stage s+NS-1 refill
            stage_barrier();
            if (s > 0 && s + NS - 1 < S) issue(std::integral_constant<int, (u + NS - 1) % NS>{}, s + NS - 1);
            if (active) compute(uc, s);
          }
        });
      }
    }

    if (!active) return;
    // ---- epilogue: the weight fragment is the MFMA's first operand, so lane
    // (r16, g4) holds row 16 i + r16 and the 4 consecutive columns 16 j + 4 g4 + r
    // of each 16x16 tile: one 8-byte store per tile when the output allows it.
    const bool wide = (p.ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
  #pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + 16 * MT * wm + 16 * i + r16;
      if (m >= m_end) continue;
      uint16_t* orow = p.out + (int64_t)m * p.ldo + wcol0 + 4 * g4;
  #pragma unroll
      for (int j = 0; j < (GATEUP ? NH : NT); ++j) {
        float v[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = GATEUP ? silu(acc[i][j][r]) * acc[i][j + NH][r] : acc[i][j][r];
        const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
        if (wide) {
          *reinterpret_cast<uint2*>(orow + 16 * j) = make_uint2(lo, hi);
        } else {
          orow[16 * j] = (uint16_t)lo;
          orow[16 * j + 1] = (uint16_t)(lo >> 16);
          orow[16 * j + 2] = (uint16_t)hi;
          orow[16 * j + 3] = (uint16_t)(hi >> 16);
        }
      }
    }
  };
#if DMOE_TILE_MT_FINE
  const int rows = m_end - m0;
  if (rows <= 32) run(std::integral_constant<int, 1>{});
  else if (rows <= 64) run(std::integral_constant<int, 2>{});
  else if (rows <= 96) run(std::integral_constant<int, 3>{});
  else run(std::integral_constant<int, 4>{});
#else
  if (m_end - m0 <= 64) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 4>{});
#endif
}

__global__ void fill_offsets_kernel(int32_t* offsets, int rows) {
  offsets[0] = 0;
  offsets[1] = rows;
}

hipError_t launch_fill_offsets(int32_t* offsets, int rows, hipStream_t stream) {
  fill_offsets_kernel<<<1, 1, 0, stream>>>(offsets, rows);
  return hipGetLastError();
}

// Which tile kernel a launch uses, and so which of the two schedules in the
// GEMM workspace: the wide kernel (gemm_wide.hip, 256-row tiles) for BF16
// operands and the FP8 down projection; this file's kernel (128-row tiles,
// two workgroups per CU) for the FP8 gate/up projection with exact products,
// where the two independent workgroups per CU overlap one's E4M3 -> BF16
// conversions with the other's matrix-core work (measured faster there: prefill
// gate/up 2.58 vs 2.88 ms). FP8 gate/up moves to the wide kernel, with h
// quantised in its epilogue, when the host bound on rows per expert reaches
// DMOE_WIDE_GU (0: never): with many rows per expert its 256-row tiles halve
// the bytes staged per FLOP and the saved quantise launch pays (EP share, 4096
// rows per expert: layer 5.25 -> 5.02 ms; dense FFN 1.48 -> 1.43 ms; vision,
// 512 rows per expert: 0.813 -> 0.801 ms; prefill's 256 break even).
#ifndef DMOE_WIDE_GU
#define DMOE_WIDE_GU 512
#endif
// The GEMM workspace holds two tile schedules, one per tile height:
// [tiles of 128 rows][count] [tiles of 256 rows][count].
static int tile_cap(int bm, int max_rows, int E_loc, int extra_rows) {
  return (int)(ceil_div(max_rows, bm) + E_loc + ceil_div(extra_rows, bm));
}
static int64_t sched_bytes(int bm, int max_rows, int E_loc, int extra_rows) {
  return round_up((int64_t)tile_cap(bm, max_rows, E_loc, extra_rows) * 8, 256) + 256;
}

// The wide kernel also needs enough rows per expert to fill its 256-row tiles
// (at least 128 on average; fewer, as in the non-divisible workload's 44-90,
// leave most of each tile empty) and enough work items to fill the CUs several
// times over (a dense 4096-row layer's down projection has only 340).
static bool use_wide(int dtype, bool gateup, int max_rows, int E_loc, int extra_rows, int64_t npad) {
  if (gateup && dtype == DMOE_FP8_E4M3 && (DMOE_WIDE_GU <= 0 || ceil_div(max_rows, E_loc) < DMOE_WIDE_GU))
    return false;
  const int64_t col_blocks = gateup ? npad / 128 : ceil_div(npad, 256);
  const int64_t items = (int64_t)tile_cap(kWideBM, max_rows, E_loc, extra_rows) * col_blocks;
  return ceil_div(max_rows, E_loc) >= 128 && items >= 1024;
}

size_t gemm_ws_bytes(int max_rows, int E_loc, int extra_rows) {
  return (size_t)(sched_bytes(kBM, max_rows, E_loc, extra_rows) + sched_bytes(kWideBM, max_rows, E_loc, extra_rows));
}

struct Sched {
  int2* tiles;
  int32_t* count;
  int cap;
};
static Sched sched_of(void* ws, bool wide, int max_rows, int E_loc, int extra_rows) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  if (wide) b += sched_bytes(kBM, max_rows, E_loc, extra_rows);
  const int bm = wide ? kWideBM : kBM;
  const int cap = tile_cap(bm, max_rows, E_loc, extra_rows);
  return Sched{reinterpret_cast<int2*>(b), reinterpret_cast<int32_t*>(b + round_up((int64_t)cap * 8, 256)), cap};
}

hipError_t launch_schedule(const int32_t* offsets, int E_loc, int max_rows, int extra_rows, int extra_row0,
                           void* ws, hipStream_t stream) {
  for (int w = 0; w < 2; ++w) {
    const Sched s = sched_of(ws, w == 1, max_rows, E_loc, extra_rows);
    schedule_kernel<<<1, 1024, 0, stream>>>(offsets, E_loc, w ? kWideBM : kBM, extra_rows, extra_row0, s.cap,
                                            s.tiles, s.count);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool gemm_uses_stream(int max_rows, int E_loc) { return ceil_div(max_rows, E_loc) <= 32; }

const char* gemm_gateup_kernel_name(int dtype, int max_rows, int E_loc, int extra_rows, int N) {
  if (gemm_uses_stream(max_rows, E_loc)) return "gemm_stage_kernel";
  return use_wide(dtype, true, max_rows, E_loc, extra_rows, round_up(N, 128)) ? "gemm_wide_kernel"
                                                                               : "gemm_tile_kernel";
}

const char* gemm_down_kernel_name(int dtype, int max_rows, int E_loc, int extra_rows, int N) {
  if (gemm_uses_stream(max_rows, E_loc)) return "gemm_stage_kernel";
  return use_wide(dtype, false, max_rows, E_loc, extra_rows, round_up(N, 128)) ? "gemm_wide_kernel"
                                                                                : "gemm_tile_kernel";
}

bool gemm_fuses_h_quant(int max_rows, int E_loc, int extra_rows, int N) {
  return DMOE_WIDE_GU > 0 && !gemm_uses_stream(max_rows, E_loc) &&
         use_wide(DMOE_FP8_E4M3, true, max_rows, E_loc, extra_rows, round_up(N, 128));
}

static hipError_t launch_gemm(const GemmArgs& g, bool gateup, hipStream_t stream) {
  const bool wide = use_wide(g.dtype, gateup, g.max_rows, g.E_loc, g.x_rows, round_up(g.N, 128));
  const Sched sch = sched_of(g.ws, wide, g.max_rows, g.E_loc, g.x_rows);
  const int cap = sch.cap;
  const int64_t per_expert = ceil_div(g.max_rows, g.E_loc);
  const bool use_stream = gemm_uses_stream(g.max_rows, g.E_loc);
  if (!g.scheduled && !use_stream) {
    const hipError_t e = launch_schedule(g.offsets, g.E_loc, g.max_rows, g.x_rows, g.x_row0, g.ws, stream);
    if (e != hipSuccess) return e;
  }
  const int es = g.dtype == DMOE_FP8_E4M3 ? 1 : 2;
  const int64_t kpad = round_up(g.K, 128);
  const int64_t npad = round_up(g.N, 128);
  TileArgs p;
  p.a = static_cast<const uint8_t*>(g.a);
  p.lda_b = g.lda * es;
  p.a_scales = g.a_scales;
  p.ldas = g.ldas;
  p.row_token = g.row_token;
  p.offsets = g.offsets;
  p.tiles = sch.tiles;
  p.ntiles = sch.count;
  p.w0 = static_cast<const uint8_t*>(g.w0);
  p.w1 = static_cast<const uint8_t*>(g.w1);
  p.ldw_b = g.ldw * es;
  p.w_expert_b = npad * g.ldw * es;  // gate/up: F_pad rows; down: H rows (H % 128 == 0)
  p.ws0 = g.ws0;
  p.ws1 = g.ws1;
  p.nNb = (int)ceil_div(g.N, 128);
  p.nKb = (int)ceil_div(g.K, 128);
  p.stages = (int)(kpad * es / kKB);  // 128-byte stages (the stream kernel and most tile modes)
  p.out = g.out;
  p.ldo = g.ldo;
  p.E_loc = g.E_loc;
  p.x_rows = g.x_rows;
  p.x_row0 = g.x_row0;
  p.x_a_base = g.x_a_base;
  p.xw0 = static_cast<const uint8_t*>(g.xw0);
  p.xw1 = static_cast<const uint8_t*>(g.xw1);
  p.xws0 = g.xws0;
  p.xws1 = g.xws1;
  p.x_chunk = 0;
  p.out_q = g.out_q;
  p.out_s = g.out_s;
  p.ld_s = g.ld_s;
  // only the wide kernel quantises h in its epilogue (gemm_fuses_h_quant decides both)
  if (g.out_q && (use_stream || !wide || !gateup || g.dtype != DMOE_FP8_E4M3)) return hipErrorInvalidValue;
  // Few rows per expert on average: stream the weights (the tile schedule is not used).
  if (use_stream) {
    p.x_chunk = per_expert <= 16 ? 16 : 32;
    return launch_gemm_stream(p, g.dtype, gateup, (int)per_expert, (int)npad, g.E_loc, stream);
  }
  if (wide) return launch_gemm_wide(p, g.dtype, gateup, (int)npad, cap, stream);
  // tile kernel: 128-byte stages for every mode (FP8: one 128-wide slice, BF16: 64 elements)
  constexpr int NT_GU = DMOE_TILE_NT_GATEUP, NT_DN = DMOE_TILE_NT_DOWN;
  constexpr int WN_GU = DMOE_TILE_WN_GATEUP, WN_DN = DMOE_TILE_WN_DOWN;
  constexpr int NS_GU = WN_GU == 2 ? DMOE_TILE_NS : DMOE_TILE_NS_WIDE;
  constexpr int NS_DN = WN_DN == 2 ? DMOE_TILE_NS : DMOE_TILE_NS_WIDE;
  // weight rows per workgroup: gate/up 8 NT WN gate + as many up rows (npad is a multiple of 128,
  // and 8 NT WN divides 128); down 16 NT WN (a partial last block leaves waves idle)
  const int nNB = gateup ? (int)(npad / (8 * NT_GU * WN_GU)) : (int)ceil_div(npad, 16 * NT_DN * WN_DN);
  const unsigned grid = (unsigned)round_up((int64_t)cap * nNB, 8);
  const int nv = (int)npad;
  const unsigned thr = 128 * (gateup ? WN_GU : WN_DN);
  if (g.dtype == DMOE_FP8_E4M3) {
    if (gateup) gemm_tile_kernel<kModeFP8X, true, NS_GU, NT_GU, WN_GU><<<grid, thr, 0, stream>>>(p, nNB, nv);
    else gemm_tile_kernel<kModeFP8, false, NS_DN, NT_DN, WN_DN><<<grid, thr, 0, stream>>>(p, nNB, nv);
  } else {
    if (gateup) gemm_tile_kernel<kModeBF16, true, NS_GU, NT_GU, WN_GU><<<grid, thr, 0, stream>>>(p, nNB, nv);
    else gemm_tile_kernel<kModeBF16, false, NS_DN, NT_DN, WN_DN><<<grid, thr, 0, stream>>>(p, nNB, nv);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_gateup(const GemmArgs& g, hipStream_t stream) { return launch_gemm(g, true, stream); }
hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t stream) { return launch_gemm(g, false, stream); }

}  // namespace dmoe
