// Wide tile kernel for the grouped expert GEMMs with many rows per expert
// (prefill chunks, an EP rank's share, verify batches of thousands of tokens).
//
// Same operation as the other GEMM kernels: gate/up with fused SwiGLU or down,
// FP8 block-scale promotion per 128-wide K slice (Transformers PR #47844,
// implementation list: E4M3 weights in 128x128 blocks, dynamically quantised
// activations; expert form from Transformers documentation "Dots 3 Note
// Preview", Dots3NoteTextConfig hidden_act, mlp_bias).
//
// One 512-thread workgroup per CU owns up to kWBM = 256 rows of one group and
// kWBN = 256 weight rows: gate/up takes 128 gate rows and the matching 128 up
// rows, i.e. one whole 128-column slice of h, so the FP8 path can quantise h
// in the epilogue (the slice's amax is complete inside the workgroup); down
// takes 256 columns of o. Every K stage (128 bytes of each A and weight row:
// one FP8 scale slice, or 64 BF16 elements) moves global -> LDS with direct
// loads through a 2-stage ring (2 x 64 KB). Bytes staged per FLOP are half
// those of a 128 x 128 tile, which is what the global -> LDS path of a CU can
// sustain at the matrix cores' FP8 rate.
//
// Waves: 8 = 4 (rows) x 2 (weight rows); wave (wm, wn) computes 16 MT rows x
// 128 weight rows as MT x 8 MFMA tiles of 16 x 16, MT = ceil(rows / 64) (a
// tile of r < 256 rows costs MFMA work in proportion to ceil(r / 64)). The
// weight fragment is the MFMA's first operand, so each lane ends with one row
// and four consecutive output columns per 16 x 16 tile.
#include "gemm_common.h"
#include "quant_common.h"

namespace dmoe {

constexpr int kWBM = 256;  // rows per tile
constexpr int kWBN = 256;  // weight rows per workgroup
constexpr int kWThreads = 512;
constexpr int kWWaves = kWThreads / 64;

#ifndef DMOE_WIDE_XCD_REMAP
#define DMOE_WIDE_XCD_REMAP 1
#endif
__device__ __forceinline__ float bf16r(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// Epilogue of the FP8 gate/up launch in the layer: h = silu(g) * u goes to LDS
// (FP32, [256 rows][128 columns], 16-byte units XOR-swizzled by row), then two
// threads per row round it to BF16 and quantise the row's 128-column slice with
// the activation rule (amax over the BF16 values, s = f32(amax / 448), codes by
// round-to-nearest-even), as dmoe_quant_act does for a BF16 h, and write the
// codes as 64-byte runs.
template <int MT>
__device__ __forceinline__ void quantise_h_epilogue(const TileArgs& p, const f32x4 (&acc)[MT][8], float* hx, int m0,
                                                    int m_end, int ncol0, int wm, int wn, int r16, int g4) {
  auto unit = [&](int row, int u) -> f32x4* { return reinterpret_cast<f32x4*>(hx + row * 128) + (u ^ (row & 31)); };
  __builtin_amdgcn_s_waitcnt(0xc07f);
  stage_barrier();  // every wave is done reading the ring
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = 16 * MT * wm + 16 * i + r16;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = silu(acc[i][jj][r]) * acc[i][jj + 4][r];
      *unit(row, 16 * wn + 4 * jj + g4) = v;
    }
  }
  __syncthreads();
  const int row = (int)(threadIdx.x >> 1), half = (int)(threadIdx.x & 1);
  const bool valid = m0 + row < m_end;
  float v[64];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const f32x4 t = *unit(row, 16 * half + k);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[4 * k + r] = t[r];
  }
  float mx = 0.f;
#pragma unroll
  for (int k = 0; k < 64; ++k) mx = fmaxf(mx, fabsf(v[k]));
  mx = fmaxf(mx, __shfl_xor(mx, 1));  // the row's other half
  if (!valid) return;
  const int m = m0 + row;
  const float s = div_rn(bf16r(mx), 448.f);
  uint8_t* qrow = p.out_q + (int64_t)m * p.ldo + ncol0 + 64 * half;
  const ScaleDiv d = make_scale_div(s != 0.f ? s : 1.f);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float* q = v + 16 * b + 4 * t;
      w[t] = s != 0.f ? e4m3x4_hw(scale_div(d, bf16r(q[0])), scale_div(d, bf16r(q[1])), scale_div(d, bf16r(q[2])),
                                  scale_div(d, bf16r(q[3])))
                      : 0u;
    }
    *reinterpret_cast<uint4*>(qrow + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (half == 0) p.out_s[(int64_t)m * p.ld_s + (ncol0 >> 7)] = s;
}

template <int MODE, bool GATEUP, bool QH>
__global__ __launch_bounds__(kWThreads, 1) void gemm_wide_kernel(const TileArgs p, int nNB, int n_valid) {
  constexpr bool kScaled = MODE != kModeBF16;
  constexpr int kRows = kWBM + kWBN;  // LDS rows per stage: A rows, then weight rows
  constexpr int kInstB = kWBN / (8 * kWWaves);  // weight-row copies per wave per stage (4)
  static_assert(kInstB * 8 * kWWaves == kWBN, "copy split");
  static_assert(!QH || (GATEUP && MODE != kModeBF16), "h quantisation belongs to the FP8 gate/up epilogue");
  static_assert(GATEUP || MODE != kModeFP8X, "the exact-product mode serves gate/up only");
  static_assert(!GATEUP || MODE != kModeFP8, "FP8 gate/up takes exact products (BF16 matrix cores)");
  // the 2-stage ring; after the K loop the FP8 gate/up epilogue reuses it for h
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kRows * 128];
  __shared__ __attribute__((aligned(256))) float lsa0[kWBM];
  __shared__ __attribute__((aligned(256))) float lsa1[kWBM];
  __shared__ float lsw[2][kMaxSlices];
  asm volatile("" ::"v"(lds), "v"(lsa0), "v"(lsa1) : "memory");

  // ---- work item: (tile, column block); XCD-contiguous ranges keep a tile's
  // column blocks (which share its A rows) and an expert's tiles (which share
  // its weights) in one XCD's L2
  const int nitems = *p.ntiles * nNB;
#if DMOE_WIDE_XCD_REMAP
  const int per_xcd = (nitems + 7) >> 3;
  const int k8 = (int)(blockIdx.x >> 3);
  const int L = (int)(blockIdx.x & 7) * per_xcd + k8;
  if (k8 >= per_xcd || L >= nitems) return;
#else
  const int L = blockIdx.x;
  if (L >= nitems) return;
#endif
  const int tile = L / nNB, nb = L - tile * nNB;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const GroupView gv = group_view(p, e);
  const int m_end = min(gv.row_end, m0 + kWBM);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // first weight row of the workgroup (gate/up: of the gate rows and of the up rows)
  const int ncol0 = nb * (GATEUP ? kWBN / 2 : kWBN);
  const bool active = GATEUP || ncol0 + 128 * wn < n_valid;  // down: waves past N only copy

  // weight block scales of this workgroup, staged once
  if constexpr (kScaled) {
    for (int i = tid; i < 2 * p.nKb; i += kWThreads) {
      const int w = i / p.nKb, sl = i - w * p.nKb;
      if (GATEUP) {
        lsw[w][sl] = (w == 0 ? gv.s0 : gv.s1)[(int64_t)(ncol0 >> 7) * p.nKb + sl];
      } else {
        const int col = ncol0 + 128 * w;
        lsw[w][sl] = col < n_valid ? gv.s0[(int64_t)(col >> 7) * p.nKb + sl] : 0.f;
      }
    }
  }

  // weight-row copy sources: copy i of this wave fills B rows 8 (8 i + wave) + lane / 8
  const uint8_t* bb0 = uniform_ptr(gv.w0 + (GATEUP ? (int64_t)ncol0 * p.ldw_b : 0));
  const uint8_t* bb1 = uniform_ptr(GATEUP ? gv.w1 + (int64_t)ncol0 * p.ldw_b : gv.w0);
  uint32_t boff[kInstB];
#pragma unroll
  for (int i = 0; i < kInstB; ++i) {
    const int row = 8 * (kWWaves * i + wave) + (lane >> 3);
    int64_t wrow;
    if (GATEUP) wrow = row % (kWBN / 2);
    else wrow = ncol0 + row < n_valid ? ncol0 + row : 0;  // rows past N reread row 0
    boff[i] = (uint32_t)(wrow * p.ldw_b + 16 * swz(row, lane & 7));
  }

  auto run = [&](auto mtc) {
    constexpr int MT = decltype(mtc)::value;  // row tiles of 16 per wave; the tile has <= 64 MT rows
    constexpr int kInstA = MT;                // A-row copies per wave per stage (64 MT rows)
    constexpr int kCopies = kInstA + kInstB;
    uint32_t aoff[kInstA];
#pragma unroll
    for (int i = 0; i < kInstA; ++i) {
      const int row = 8 * (kWWaves * i + wave) + (lane >> 3);
      const int m = m0 + row;
      const int64_t arow = a_row(p, gv, m < m_end ? m : m0);  // rows past the tile reuse a valid row
      aoff[i] = (uint32_t)(arow * p.lda_b + 16 * swz(row, lane & 7));
    }
    const int S = p.stages;
    // activation scales: waves 0 .. MT-1 copy the scales of rows 64 wave + lane
    const bool scale_wave = kScaled && wave < MT;
    uint32_t soff = 0;
    if (scale_wave) {
      const int m = m0 + 64 * wave + lane;
      soff = (uint32_t)(a_row(p, gv, m < m_end ? m : m0) * p.ldas * 4);
    }
    auto stage_ptr = [&](int u) -> uint8_t* { return lds + u * (kRows * 128); };
    auto scale_ptr = [&](int u) -> float* { return u ? lsa1 : lsa0; };
    auto issue = [&](int u, int s) {
      const uint32_t st = (uint32_t)(uintptr_t)stage_ptr(u);
      const int64_t off = (int64_t)s * 128;
#pragma unroll
      for (int i = 0; i < kInstA; ++i) lds_copy16_s(p.a + off, aoff[i], st + (8 * kWWaves * i + 8 * wave_u) * 128);
#pragma unroll
      for (int i = 0; i < kInstB; ++i)
        lds_copy16_s(((GATEUP && i >= kInstB / 2) ? bb1 : bb0) + off, boff[i],
                     st + (kWBM + 8 * kWWaves * i + 8 * wave_u) * 128);
      if (scale_wave) lds_copy4_s(p.a_scales + s, soff, (uint32_t)(uintptr_t)scale_ptr(u) + 256 * wave_u);
    };

    f32x4 acc[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B row (within the weight region) of this lane's column tile j: gate/up:
    // tiles 0-3 gate rows, 4-7 the matching up rows; down: 16 consecutive columns each
    auto brow = [&](int j) -> int {
      if (GATEUP) return (j < 4 ? 0 : kWBN / 2) + 64 * wn + 16 * (j & 3) + r16;
      return 128 * wn + 16 * j + r16;
    };

    auto compute = [&](int u, int s) {
      const uint8_t* st = stage_ptr(u);
      const float* lsa = scale_ptr(u);
      i32x4 fa[MT][2];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = 16 * MT * wm + 16 * i + r16;
        fa[i][0] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4));
        fa[i][1] = *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4 + 1));
      }
      float saw[2][MT];  // a_scale * w_scale per row tile: [0] gate / down, [1] up
      if constexpr (kScaled) {
        const float w0s = GATEUP ? lsw[0][s] : lsw[wn][s];
        const float w1s = GATEUP ? lsw[1][s] : 0.f;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const float a = lsa[16 * MT * wm + 16 * i + r16];
          saw[0][i] = a * w0s;
          saw[1][i] = a * w1s;
        }
      }
      if constexpr (MODE == kModeFP8X) {
        // Waves 4-7 (one of the two waves of each SIMD) issue at a raised priority
        // over the exact-product block: the stage barrier otherwise keeps a SIMD's
        // two waves in step, converting at the same time and multiplying at the
        // same time; with one ahead, one converts while the other multiplies
        // (measured: EP share gate/up 3.62 -> 3.36 ms, dense FFN 1.07 -> 1.02 ms).
        if (wave_u >= 4) __builtin_amdgcn_s_setprio(3);
        i32x4 a16[MT][4];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          e4m3x16_to_bf16(fa[i][0], a16[i][0], a16[i][1]);
          e4m3x16_to_bf16(fa[i][1], a16[i][2], a16[i][3]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int bj = brow(j);
          const uint8_t* bp = st + (kWBM + bj) * 128;
          const i32x4 b0 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4));
          const i32x4 b1 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4 + 1));
          i32x4 b16[4];
          e4m3x16_to_bf16(b0, b16[0], b16[1]);
          e4m3x16_to_bf16(b1, b16[2], b16[3]);
          const int wsel = (GATEUP && j >= 4) ? 1 : 0;
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
              part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b16[k4]),
                                                             __builtin_bit_cast(bf16x8, a16[i][k4]), part, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[r], saw[wsel][i], acc[i][j][r]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      } else if constexpr (MODE == kModeFP8) {
        // Software pipeline over the column tiles: the MT products of tile j
        // are issued before the promotion of tile j - 1's products, so the
        // promotion FMAs never wait on a matrix-core result just issued and
        // they overlap the next MFMAs.
        auto bfrag = [&](int j) -> i32x8 {
          const int bj = brow(j);
          const uint8_t* bp = st + (kWBM + bj) * 128;
          const i32x4 b0 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4));
          const i32x4 b1 = *reinterpret_cast<const i32x4*>(bp + 16 * swz(bj, 2 * g4 + 1));
          return i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        };
        i32x8 a8[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
          a8[i] = i32x8{fa[i][0][0], fa[i][0][1], fa[i][0][2], fa[i][0][3],
                        fa[i][1][0], fa[i][1][1], fa[i][1][2], fa[i][1][3]};
        f32x4 prev[MT];
        i32x8 bnext = bfrag(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const i32x8 b8 = bnext;
          if (j + 1 < 8) bnext = bfrag(j + 1);
          f32x4 cur[MT];
#pragma unroll
          for (int i = 0; i < MT; ++i)
            cur[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8[i], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                      0, 0, 0);
          if (j > 0) {
            const int wsel = (GATEUP && j - 1 >= 4) ? 1 : 0;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][j - 1][r] = fmaf(prev[i][r], saw[wsel][i], acc[i][j - 1][r]);
          }
#pragma unroll
          for (int i = 0; i < MT; ++i) prev[i] = cur[i];
        }
        {
          const int wsel = GATEUP ? 1 : 0;
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][7][r] = fmaf(prev[i][r], saw[wsel][i], acc[i][7][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int bj = brow(j);
          const uint8_t* bp = st + (kWBM + bj) * 128;
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

    // ---- 2-stage ring, one barrier per stage: stage s + 1 is issued once
    // every wave has passed the barrier of stage s (so is done with stage s - 1,
    // whose buffer it refills) and lands while stage s is computed.
    __syncthreads();  // weight scales staged
    issue(0, 0);
    if (S > 1) issue(1, 1);
    for (int s = 0; s < S; ++s) {
      const int u = s & 1;
      // stage s has landed once at most the copies issued after it (stage 1, at s = 0) are in flight
      if (s == 0 && S > 1) {
        if (scale_wave) wait_vmcnt<kCopies + 1>();
        else wait_vmcnt<kCopies>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads of stage s - 1 are done
      stage_barrier();
      if (s > 0 && s + 1 < S) issue(u ^ 1, s + 1);
      if (active) compute(u, s);
    }

    // ---- epilogue
    if constexpr (GATEUP) {
      // h columns of this lane: ncol0 + 64 wn + 16 jj + 4 g4 + r (jj = 0..3)
      const int hcol0 = ncol0 + 64 * wn + 4 * g4;
      if constexpr (QH) {
        quantise_h_epilogue<MT>(p, acc, reinterpret_cast<float*>(lds), m0, m_end, ncol0, wm, wn, r16, g4);
      } else {
        const bool wide = (p.ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const int m = m0 + 16 * MT * wm + 16 * i + r16;
          if (m >= m_end) continue;
          uint16_t* orow = p.out + (int64_t)m * p.ldo + hcol0;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = silu(acc[i][jj][r]) * acc[i][jj + 4][r];
            const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
            if (wide) {
              *reinterpret_cast<uint2*>(orow + 16 * jj) = make_uint2(lo, hi);
            } else {
              orow[16 * jj] = (uint16_t)lo;
              orow[16 * jj + 1] = (uint16_t)(lo >> 16);
              orow[16 * jj + 2] = (uint16_t)hi;
              orow[16 * jj + 3] = (uint16_t)(hi >> 16);
            }
          }
        }
      }
    } else {
      if (!active) return;
      const bool wide = (p.ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
      const int ocol0 = ncol0 + 128 * wn + 4 * g4;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * MT * wm + 16 * i + r16;
        if (m >= m_end) continue;
        uint16_t* orow = p.out + (int64_t)m * p.ldo + ocol0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]), hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
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
    }
  };
  const int rows = m_end - m0;
  if (rows <= 64) run(std::integral_constant<int, 1>{});
  else if (rows <= 128) run(std::integral_constant<int, 2>{});
  else if (rows <= 192) run(std::integral_constant<int, 3>{});
  else run(std::integral_constant<int, 4>{});
}

int wide_tile_rows() { return kWBM; }

hipError_t launch_gemm_wide(const TileArgs& p, int dtype, bool gateup, int npad, int cap, hipStream_t stream) {
  const int nNB = gateup ? npad / (kWBN / 2) : (int)ceil_div(npad, kWBN);
  const unsigned grid = (unsigned)round_up((int64_t)cap * nNB, 8);
  const bool qh = p.out_q != nullptr;
  if (dtype == DMOE_FP8_E4M3) {
    if (gateup) {
      if (qh) gemm_wide_kernel<kModeFP8X, true, true><<<grid, kWThreads, 0, stream>>>(p, nNB, npad);
      else gemm_wide_kernel<kModeFP8X, true, false><<<grid, kWThreads, 0, stream>>>(p, nNB, npad);
    } else {
      gemm_wide_kernel<kModeFP8, false, false><<<grid, kWThreads, 0, stream>>>(p, nNB, npad);
    }
  } else {
    if (gateup) gemm_wide_kernel<kModeBF16, true, false><<<grid, kWThreads, 0, stream>>>(p, nNB, npad);
    else gemm_wide_kernel<kModeBF16, false, false><<<grid, kWThreads, 0, stream>>>(p, nNB, npad);
  }
  return hipGetLastError();
}

}  // namespace dmoe
