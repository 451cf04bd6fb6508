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

template <int DT, bool GATEUP>
__global__ __launch_bounds__(256) void gemm_tile_kernel(const TileArgs p) {
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

  // ---- global source pointers for this thread's LDS chunks ----
  const uint8_t* srcA[2];
  bool okA[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int m = m0 + (c >> 3);
    okA[i] = m < m_end;
    int64_t src = m;
    if (okA[i] && p.row_token) src = p.row_token[m];
    srcA[i] = p.a + (okA[i] ? src : 0) * p.lda_b + (c & 7) * 16;
  }
  const uint8_t* srcB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int br = c >> 3;
    const uint8_t* base;
    int64_t row;
    if (GATEUP) {
      base = br < 64 ? p.w0 : p.w1;
      row = (int64_t)nb * 64 + (br & 63);
    } else {
      base = p.w0;
      row = (int64_t)nb * 128 + br;
    }
    srcB[i] = base + e * p.w_expert_b + row * p.ldw_b + (c & 7) * 16;
  }
  // FP8 scales
  int64_t saRow = -1;
  if (DT == DMOE_FP8_E4M3 && tid < kBM) {
    const int m = m0 + tid;
    if (m < m_end) saRow = p.row_token ? p.row_token[m] : m;
  }
  const int nblk = GATEUP ? (nb >> 1) : nb;  // 128-row weight block of this tile
  const float* sw0 = DT == DMOE_FP8_E4M3 ? p.ws0 + ((int64_t)e * p.nNb + nblk) * p.nKb : nullptr;
  const float* sw1 = (DT == DMOE_FP8_E4M3 && GATEUP) ? p.ws1 + ((int64_t)e * p.nNb + nblk) * p.nKb : nullptr;

  i32x4 ra[2], rb[4];
  float rsa = 0.f;
  auto load_stage = [&](int s) {
    const int64_t off = (int64_t)s * kKB;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra[i] = okA[i] ? *reinterpret_cast<const i32x4*>(srcA[i] + off) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const i32x4*>(srcB[i] + off);
    if (DT == DMOE_FP8_E4M3 && tid < kBM) rsa = saRow >= 0 ? p.a_scales[saRow * p.ldas + s] : 0.f;
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<i32x4*>(&sA[buf][(c >> 3) * kPitch + (c & 7) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<i32x4*>(&sB[buf][(c >> 3) * kPitch + (c & 7) * 16]) = rb[i];
    }
    if (DT == DMOE_FP8_E4M3 && tid < kBM) sSa[buf][tid] = rsa;
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    // ---- compute on buf ----
    i32x8 fa[2], fb[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint8_t* ptr = &sA[buf][(32 * wm + 16 * i + r16) * kPitch + g4 * 32];
      const i32x4 lo = *reinterpret_cast<const i32x4*>(ptr);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(ptr + 16);
      fa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* ptr = &sB[buf][(browj[j] + r16) * kPitch + g4 * 32];
      const i32x4 lo = *reinterpret_cast<const i32x4*>(ptr);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(ptr + 16);
      fb[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    if constexpr (DT == DMOE_FP8_E4M3) {
      const float w0s = sw0[s];
      const float w1s = GATEUP ? sw1[s] : w0s;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float sa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sa[r] = sSa[buf][32 * wm + 16 * i + 4 * g4 + r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              fa[i], fb[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          const float ws = (GATEUP && j >= 2) ? w1s : w0s;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[r], sa[r] * ws, acc[i][j][r]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8 alo = __builtin_bit_cast(bf16x8, i32x4{fa[i][0], fa[i][1], fa[i][2], fa[i][3]});
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, i32x4{fa[i][4], fa[i][5], fa[i][6], fa[i][7]});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 blo = __builtin_bit_cast(bf16x8, i32x4{fb[j][0], fb[j][1], fb[j][2], fb[j][3]});
          const bf16x8 bhi = __builtin_bit_cast(bf16x8, i32x4{fb[j][4], fb[j][5], fb[j][6], fb[j][7]});
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, blo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi, acc[i][j], 0, 0, 0);
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
  p.stages = (int)(kpad * es / kKB);
  p.out = g.out;
  p.ldo = g.ldo;
  const dim3 grid(cap, gateup ? (unsigned)(npad / 64) : (unsigned)(npad / 128));
  if (g.dtype == DMOE_FP8_E4M3) {
    if (gateup) gemm_tile_kernel<DMOE_FP8_E4M3, true><<<grid, 256, 0, stream>>>(p);
    else gemm_tile_kernel<DMOE_FP8_E4M3, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (gateup) gemm_tile_kernel<DMOE_BF16, true><<<grid, 256, 0, stream>>>(p);
    else gemm_tile_kernel<DMOE_BF16, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_gateup(const GemmArgs& g, hipStream_t stream) { return launch_gemm(g, true, stream); }
hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t stream) { return launch_gemm(g, false, stream); }

}  // namespace dmoe
