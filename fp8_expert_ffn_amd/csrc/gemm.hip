// Grouped expert GEMMs: gate/up with fused SwiGLU, and down.
//
// Expert FFN: hidden_act silu over gate_proj/up_proj, then down_proj, no bias
// (Transformers docs "Dots3Note", Dots3NoteTextConfig hidden_act, mlp_bias);
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
// exit on the device. A workgroup owns kBM rows x kBNB weight rows and walks K
// in 128-byte stages (128 FP8 or 64 BF16 elements) through two LDS buffers.
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kBM = 64;             // rows per tile
constexpr int kBNB = 128;           // weight rows per tile (gate/up: 64 gate + 64 up)
constexpr int kKB = 128;            // K bytes per stage
constexpr int kPitch = kKB + 16;    // LDS row pitch in bytes (padding spreads the banks)

struct TileArgs {
  const uint8_t* a;
  int64_t lda_b;  // bytes
  const float* a_scales;
  int64_t ldas;
  const int32_t* row_token;
  const int32_t* offsets;
  const int2* tiles;
  const int32_t* ntiles;
  const uint8_t* w0;
  const uint8_t* w1;
  int64_t ldw_b;           // bytes
  int64_t w_expert_b;      // bytes between experts
  const float* ws0;
  const float* ws1;
  int nNb, nKb;            // 128-blocks along N (weight rows) and K
  int stages;              // K stages of kKB bytes
  uint16_t* out;
  int64_t ldo;
};

// Tiles past `cap` (only possible when the caller's max_rows understates the
// real row count) are dropped rather than written past the workspace.
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ offsets, int E_loc, int bm,
                                                        int cap, int2* __restrict__ tiles,
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
  if (t == (int)blockDim.x - 1) *ntiles = min(partial[t], cap);
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

// Operand modes of the tile kernel. Every mode keeps 128-byte K rows in LDS.
//  kModeBF16: BF16 operands, 64 K per stage, BF16 MFMA.
//  kModeFP8X: E4M3 operands converted exactly to BF16 on the way into LDS,
//             64 K per stage (two stages per 128-wide scale slice), BF16 MFMA:
//             every product and the FP32 accumulation of a slice are exact to
//             FP32 rounding.
//  kModeFP8:  E4M3 operands in LDS, 128 K per stage (one scale slice), FP8 MFMA
//             (the matrix core's own accumulation precision within a slice).
constexpr int kModeBF16 = 0, kModeFP8X = 1, kModeFP8 = 2;

__device__ __forceinline__ void e4m3x16_to_bf16(const i32x4 src, i32x4& lo, i32x4& hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  int out[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = (uint32_t)src[w];
    out[2 * w] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false));
    out[2 * w + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true));
  }
  lo = i32x4{out[0], out[1], out[2], out[3]};
  hi = i32x4{out[4], out[5], out[6], out[7]};
}

template <int MODE, bool GATEUP>
__global__ __launch_bounds__(256) void gemm_tile_kernel(const TileArgs p) {
  constexpr bool kScaled = MODE != kModeBF16;
  // global bytes per row per stage, and 16-byte chunks per row
  constexpr int kSrcRow = MODE == kModeFP8X ? 64 : 128;
  constexpr int kCpr = kSrcRow / 16;
  constexpr int kChunksA = kBM * kCpr / 256;   // per thread
  constexpr int kChunksB = kBNB * kCpr / 256;
  constexpr int kStagesPerSlice = MODE == kModeFP8X ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kBNB * kPitch];
  __shared__ float sSa[2][kBM];

  const int tile = blockIdx.x;
  if (tile >= *p.ntiles) return;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int m_end = p.offsets[e + 1];
  const int nb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- global source pointers for this thread's chunks ----
  const uint8_t* srcA[kChunksA];
  bool okA[kChunksA];
#pragma unroll
  for (int i = 0; i < kChunksA; ++i) {
    const int c = tid + 256 * i;
    const int m = m0 + c / kCpr;
    okA[i] = m < m_end;
    int64_t src = m;
    if (okA[i] && p.row_token) src = p.row_token[m];
    srcA[i] = p.a + (okA[i] ? src : 0) * p.lda_b + (c % kCpr) * 16;
  }
  const uint8_t* srcB[kChunksB];
#pragma unroll
  for (int i = 0; i < kChunksB; ++i) {
    const int c = tid + 256 * i;
    const int br = c / kCpr;
    const uint8_t* base;
    int64_t row;
    if (GATEUP) {
      base = br < 64 ? p.w0 : p.w1;
      row = (int64_t)nb * 64 + (br & 63);
    } else {
      base = p.w0;
      row = (int64_t)nb * 128 + br;
    }
    srcB[i] = base + e * p.w_expert_b + row * p.ldw_b + (c % kCpr) * 16;
  }
  int64_t saRow = -1;
  if (kScaled && tid < kBM) {
    const int m = m0 + tid;
    if (m < m_end) saRow = p.row_token ? p.row_token[m] : m;
  }
  const int nblk = GATEUP ? (nb >> 1) : nb;  // 128-row weight block of this tile
  const float* sw0 = kScaled ? p.ws0 + ((int64_t)e * p.nNb + nblk) * p.nKb : nullptr;
  const float* sw1 = (kScaled && GATEUP) ? p.ws1 + ((int64_t)e * p.nNb + nblk) * p.nKb : nullptr;

  i32x4 ra[kChunksA], rb[kChunksB];
  float rsa = 0.f;
  auto load_stage = [&](int s) {
    const int64_t off = (int64_t)s * kSrcRow;
#pragma unroll
    for (int i = 0; i < kChunksA; ++i)
      ra[i] = okA[i] ? *reinterpret_cast<const i32x4*>(srcA[i] + off) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) rb[i] = *reinterpret_cast<const i32x4*>(srcB[i] + off);
    if (kScaled && tid < kBM) rsa = saRow >= 0 ? p.a_scales[saRow * p.ldas + s / kStagesPerSlice] : 0.f;
  };
  auto store_chunk = [&](uint8_t* base, int c, const i32x4 v) {
    if constexpr (MODE == kModeFP8X) {
      i32x4 lo, hi;
      e4m3x16_to_bf16(v, lo, hi);
      uint8_t* d = base + (c / kCpr) * kPitch + (c % kCpr) * 32;
      *reinterpret_cast<i32x4*>(d) = lo;
      *reinterpret_cast<i32x4*>(d + 16) = hi;
    } else {
      *reinterpret_cast<i32x4*>(base + (c / kCpr) * kPitch + (c % kCpr) * 16) = v;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) store_chunk(sA[buf], tid + 256 * i, ra[i]);
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) store_chunk(sB[buf], tid + 256 * i, rb[i]);
    if (kScaled && tid < kBM) sSa[buf][tid] = rsa;
  };

  f32x4 acc[2][4], part[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r16 = lane & 15, g4 = lane >> 4;
  int browj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    browj[j] = GATEUP ? ((j < 2 ? 0 : 64) + 32 * wn + 16 * (j & 1)) : (64 * wn + 16 * j);

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < p.stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < p.stages) load_stage(s + 1);
    // ---- fragments: 32 bytes of one 128-byte LDS row per lane ----
    i32x4 fa[2][2], fb[4][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint8_t* ptr = &sA[buf][(32 * wm + 16 * i + r16) * kPitch + g4 * 32];
      fa[i][0] = *reinterpret_cast<const i32x4*>(ptr);
      fa[i][1] = *reinterpret_cast<const i32x4*>(ptr + 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* ptr = &sB[buf][(browj[j] + r16) * kPitch + g4 * 32];
      fb[j][0] = *reinterpret_cast<const i32x4*>(ptr);
      fb[j][1] = *reinterpret_cast<const i32x4*>(ptr + 16);
    }
    if constexpr (MODE == kModeFP8) {
      const float w0s = sw0[s];
      const float w1s = GATEUP ? sw1[s] : w0s;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float sa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sa[r] = sSa[buf][32 * wm + 16 * i + 4 * g4 + r];
        const i32x8 a8 = i32x8{fa[i][0][0], fa[i][0][1], fa[i][0][2], fa[i][0][3],
                               fa[i][1][0], fa[i][1][1], fa[i][1][2], fa[i][1][3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i32x8 b8 = i32x8{fb[j][0][0], fb[j][0][1], fb[j][0][2], fb[j][0][3],
                                 fb[j][1][0], fb[j][1][1], fb[j][1][2], fb[j][1][3]};
          const f32x4 pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                             0, 0, 0, 0);
          const float ws = (GATEUP && j >= 2) ? w1s : w0s;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(pr[r], sa[r] * ws, acc[i][j][r]);
        }
      }
    } else {
      f32x4(&dst)[2][4] = MODE == kModeBF16 ? acc : part;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8 alo = __builtin_bit_cast(bf16x8, fa[i][0]);
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, fa[i][1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, __builtin_bit_cast(bf16x8, fb[j][0]), dst[i][j],
                                                              0, 0, 0);
          dst[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, __builtin_bit_cast(bf16x8, fb[j][1]), dst[i][j],
                                                              0, 0, 0);
        }
      }
      if constexpr (MODE == kModeFP8X) {
        if ((s & 1) == 1) {  // end of a 128-wide slice: promote with the block scales
          const int sl = s >> 1;
          const float w0s = sw0[sl];
          const float w1s = GATEUP ? sw1[sl] : w0s;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            float sa[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) sa[r] = sSa[buf][32 * wm + 16 * i + 4 * g4 + r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float ws = (GATEUP && j >= 2) ? w1s : w0s;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[i][j][r] = fmaf(part[i][j][r], sa[r] * ws, acc[i][j][r]);
                part[i][j][r] = 0.f;
              }
            }
          }
        }
      }
    }
    if (s + 1 < p.stages) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*g4 + r, column r16 of each 16x16 tile ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 32 * wm + 16 * i + 4 * g4 + r;
      if (m >= m_end) continue;
      uint16_t* orow = p.out + (int64_t)m * p.ldo;
      if (GATEUP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nb * 64 + 32 * wn + 16 * j + r16;
          const float h = silu(acc[i][j][r]) * acc[i][j + 2][r];
          orow[col] = (uint16_t)f32_to_bf16(h);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nb * 128 + 64 * wn + 16 * j + r16;
          orow[col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming variant for few rows per expert (decode). Each wave owns 16
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
  const int row_beg = p.offsets[e], row_end = p.offsets[e + 1];
  if (row_beg >= row_end) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  if (n0 >= n_cols) return;
  const int64_t wcol = g4 * 32;
  const uint8_t* wg = p.w0 + e * p.w_expert_b + (int64_t)(n0 + r16) * p.ldw_b + wcol;
  const uint8_t* wu = GATEUP ? p.w1 + e * p.w_expert_b + (int64_t)(n0 + r16) * p.ldw_b + wcol : nullptr;
  const int nblk = n0 >> 7;
  const float* sw0 = DT == DMOE_FP8_E4M3 ? p.ws0 + ((int64_t)e * p.nNb + nblk) * p.nKb : nullptr;
  const float* sw1 = (DT == DMOE_FP8_E4M3 && GATEUP) ? p.ws1 + ((int64_t)e * p.nNb + nblk) * p.nKb : nullptr;
  constexpr int NM = GATEUP ? 2 : 1;  // weight matrices per wave

  for (int m0 = row_beg; m0 < row_end; m0 += 16 * R) {
    const uint8_t* arow[R];
    bool aok[R];
    int64_t srow[R][4];  // source rows of the 4 output rows this lane holds, for the A scales
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int m = m0 + 16 * i + r16;
      aok[i] = m < row_end;
      const int64_t src = aok[i] ? (p.row_token ? p.row_token[m] : m) : 0;
      arow[i] = p.a + src * p.lda_b + wcol;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mq = m0 + 16 * i + 4 * g4 + q;
        srow[i][q] = mq < row_end ? (p.row_token ? p.row_token[mq] : mq) : -1;
      }
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
          float sa[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) sa[q] = srow[i][q] >= 0 ? p.a_scales[srow[i][q] * p.ldas + s] : 0.f;
#pragma unroll
          for (int t = 0; t < NM; ++t) {
            f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
              part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a16[k4]),
                                                             __builtin_bit_cast(bf16x8, b16[t][k4]), part, 0, 0, 0);
            const float ws = t == 0 ? w0s : w1s;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t][i][q] = fmaf(part[q], sa[q] * ws, acc[t][i][q]);
          }
        }
      } else if constexpr (DT == DMOE_FP8_E4M3) {
        const float w0s = sw0[s];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const i32x8 fa = i32x8{ra[slot][i][0][0], ra[slot][i][0][1], ra[slot][i][0][2], ra[slot][i][0][3],
                                 ra[slot][i][1][0], ra[slot][i][1][1], ra[slot][i][1][2], ra[slot][i][1][3]};
          float sa[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) sa[q] = srow[i][q] >= 0 ? p.a_scales[srow[i][q] * p.ldas + s] : 0.f;
          const i32x8 fb = i32x8{rb[slot][0][0][0], rb[slot][0][0][1], rb[slot][0][0][2], rb[slot][0][0][3],
                                 rb[slot][0][1][0], rb[slot][0][1][1], rb[slot][0][1][2], rb[slot][0][1][3]};
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                               0, 0, 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[0][i][q] = fmaf(part[q], sa[q] * w0s, acc[0][i][q]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const bf16x8 alo = __builtin_bit_cast(bf16x8, ra[slot][i][0]);
          const bf16x8 ahi = __builtin_bit_cast(bf16x8, ra[slot][i][1]);
#pragma unroll
          for (int t = 0; t < NM; ++t) {
            acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, __builtin_bit_cast(bf16x8, rb[slot][t][0]),
                                                                acc[t][i], 0, 0, 0);
            acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, __builtin_bit_cast(bf16x8, rb[slot][t][1]),
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

#pragma unroll
    for (int i = 0; i < R; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + 16 * i + 4 * g4 + q;
        if (m >= row_end) continue;
        const float v = GATEUP ? silu(acc[0][i][q]) * acc[NM - 1][i][q] : acc[0][i][q];
        p.out[(int64_t)m * p.ldo + n0 + r16] = (uint16_t)f32_to_bf16(v);
      }
    }
  }
}

__global__ void fill_offsets_kernel(int32_t* offsets, int rows) {
  offsets[0] = 0;
  offsets[1] = rows;
}

hipError_t launch_fill_offsets(int32_t* offsets, int rows, hipStream_t stream) {
  fill_offsets_kernel<<<1, 1, 0, stream>>>(offsets, rows);
  return hipGetLastError();
}

static int tile_cap(int max_rows, int E_loc) { return (int)ceil_div(max_rows, kBM) + E_loc; }

size_t gemm_ws_bytes(int max_rows, int E_loc) {
  return (size_t)round_up((int64_t)tile_cap(max_rows, E_loc) * 8, 256) + 256;
}

static int2* sched_tiles(void* ws) { return static_cast<int2*>(ws); }
static int32_t* sched_count(void* ws, int cap) {
  return reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + round_up((int64_t)cap * 8, 256));
}

hipError_t launch_schedule(const int32_t* offsets, int E_loc, int max_rows, void* ws, hipStream_t stream) {
  const int cap = tile_cap(max_rows, E_loc);
  schedule_kernel<<<1, 1024, 0, stream>>>(offsets, E_loc, kBM, cap, sched_tiles(ws), sched_count(ws, cap));
  return hipGetLastError();
}

static hipError_t launch_gemm(const GemmArgs& g, bool gateup, hipStream_t stream) {
  const int cap = tile_cap(g.max_rows, g.E_loc);
  if (!g.scheduled) {
    const hipError_t e = launch_schedule(g.offsets, g.E_loc, g.max_rows, g.ws, stream);
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
  p.tiles = sched_tiles(g.ws);
  p.ntiles = sched_count(g.ws, cap);
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
  // Few rows per expert on average: stream the weights (the tile schedule is not used).
  const int64_t per_expert = ceil_div(g.max_rows, g.E_loc);
  if (per_expert <= 32) {
    const dim3 sgrid((unsigned)(npad / 64), (unsigned)g.E_loc);
    const int ncols = (int)npad;
#define DMOE_STREAM(DTV, GU)                                                                         \
  do {                                                                                               \
    if (per_expert <= 16) gemm_stream_kernel<DTV, GU, 1><<<sgrid, 256, 0, stream>>>(p, ncols);       \
    else gemm_stream_kernel<DTV, GU, 2><<<sgrid, 256, 0, stream>>>(p, ncols);                        \
  } while (0)
    if (g.dtype == DMOE_FP8_E4M3) {
      if (gateup) DMOE_STREAM(DMOE_FP8_E4M3, true);
      else DMOE_STREAM(DMOE_FP8_E4M3, false);
    } else {
      if (gateup) DMOE_STREAM(DMOE_BF16, true);
      else DMOE_STREAM(DMOE_BF16, false);
    }
#undef DMOE_STREAM
    return hipGetLastError();
  }
  // the tile kernel's exact FP8 gate/up mode stages 64 K elements (128 bytes once converted)
  if (g.dtype == DMOE_FP8_E4M3 && gateup) p.stages = (int)(kpad / 64);
  const dim3 grid(cap, gateup ? (unsigned)(npad / 64) : (unsigned)(npad / 128));
  if (g.dtype == DMOE_FP8_E4M3) {
    if (gateup) gemm_tile_kernel<kModeFP8X, true><<<grid, 256, 0, stream>>>(p);
    else gemm_tile_kernel<kModeFP8, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (gateup) gemm_tile_kernel<kModeBF16, true><<<grid, 256, 0, stream>>>(p);
    else gemm_tile_kernel<kModeBF16, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_gateup(const GemmArgs& g, hipStream_t stream) { return launch_gemm(g, true, stream); }
hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t stream) { return launch_gemm(g, false, stream); }

}  // namespace dmoe
