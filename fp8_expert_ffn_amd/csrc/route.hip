// Router: FP32 logits on matrix cores, then top-K selection (optionally
// group-limited) and softmax weights, one wavefront per token.
//
// FP32 routing: Transformers PR #47844, implementation list. Top-K with
// renormalised weights: Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig
// (num_experts_per_tok, norm_topk_prob, routed_scaling_factor, n_group,
// topk_group); the softmax scoring is the reading of the docs' "post-softmax"
// router_logits entry.
#include "gemm_common.h"

namespace dmoe {

// ---------------------------------------------------------------------------
// Router logits L = f32(x) . W_r^T.
//
// x is BF16 (8 significant bits). Each FP32 router weight is split exactly as
// w = hi + mid + lo with three BF16 values (truncation: hi keeps the top 8
// significand bits, mid the next 8, lo the last 8), so every product x*part is
// exact in FP32 and the three BF16 MFMAs sum exactly the products of the FP32
// definition, with FP32 accumulation.
//
// Wave tile: (16*TT tokens) x (16*EE experts); the NW waves of a workgroup split
// H into NW ranges and their partial tiles are added in wave order through LDS
// (fixed order: deterministic). Rows past T or E read row 0 (their sums are
// never stored), so every load is unconditional and a wave can have the loads
// of PF K-steps in flight at once (few tokens: the kernel waits on W_r reads).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split3_bf16(const float (&w)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = __float_as_uint(w[i]);
    const float h = __uint_as_float(b & 0xffff0000u);
    const float r1 = w[i] - h;  // exact
    const float m = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
    const float r2 = r1 - m;  // exact, fits in 8 significant bits
    hi[i] = __builtin_bit_cast(__bf16, (uint16_t)(b >> 16));
    mid[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(m) >> 16));
    lo[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(r2) >> 16));
  }
}

// NW waves split H into NW equal ranges (H % (32 NW PF) == 0). With
// gridDim.z = KS > 1 workgroup z covers only the z-th of KS equal K ranges
// (H % (32 NW PF KS) == 0) and stores its partial sums as plane z of `logits`
// ([KS][T][E]); the planes are added in plane order by the route kernels.
template <int TT, int EE, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void router_logits_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                const float* __restrict__ w_r, int T, int H, int E,
                                                                float* __restrict__ logits) {
  __shared__ f32x4 red[NW - 1][TT * EE][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16 * TT;
  const int e0 = blockIdx.y * 16 * EE;
  const int r16 = lane & 15;
  const int kg = (lane >> 4) * 8;
  const int kq = H / (NW * (int)gridDim.z);
  const int kbeg = (int)blockIdx.z * (H / (int)gridDim.z) + wave * kq;
  logits += (int64_t)blockIdx.z * T * E;

  const uint16_t* xrow[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int t = t0 + 16 * i + r16;
    xrow[i] = x + (int64_t)(t < T ? t : 0) * ldx + kg;
  }
  int64_t wrow[EE];
#pragma unroll
  for (int j = 0; j < EE; ++j) {
    const int e = e0 + 16 * j + r16;
    wrow[j] = (int64_t)(e < E ? e : 0) * H + kg;
  }

  f32x4 acc[TT][EE];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < EE; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg; k0 < kbeg + kq; k0 += 32 * PF) {
    bf16x8 a[PF][TT];
    f32x4 wv[PF][EE][2];
#pragma unroll
    for (int pf = 0; pf < PF; ++pf) {
      const int k = k0 + 32 * pf;
#pragma unroll
      for (int i = 0; i < TT; ++i) a[pf][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(xrow[i] + k));
#pragma unroll
      for (int j = 0; j < EE; ++j) {
        wv[pf][j][0] = *reinterpret_cast<const f32x4*>(w_r + wrow[j] + k);
        wv[pf][j][1] = *reinterpret_cast<const f32x4*>(w_r + wrow[j] + k + 4);
      }
    }
#pragma unroll
    for (int pf = 0; pf < PF; ++pf) {
#pragma unroll
      for (int j = 0; j < EE; ++j) {
        const float w[8] = {wv[pf][j][0][0], wv[pf][j][0][1], wv[pf][j][0][2], wv[pf][j][0][3],
                            wv[pf][j][1][0], wv[pf][j][1][1], wv[pf][j][1][2], wv[pf][j][1][3]};
        bf16x8 hi, mid, lo;
        split3_bf16(w, hi, mid, lo);
#pragma unroll
        for (int i = 0; i < TT; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[pf][i], hi, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[pf][i], mid, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[pf][i], lo, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
      for (int j = 0; j < EE; ++j) red[wave - 1][i * EE + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
#pragma unroll
    for (int j = 0; j < EE; ++j) {
      f32x4 s = acc[i][j];
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) s += red[w][i * EE + j][lane];  // fixed wave order: deterministic
      const int e = e0 + 16 * j + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * i + (lane >> 4) * 4 + r;
        if (t < T && e < E) logits[(int64_t)t * E + e] = s[r];
      }
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, int64_t ldx, const float* w_r, int T, int H, int E,
                                float* logits, hipStream_t stream) {
  if (T <= 256) {
    // few tokens: the weight read dominates; 16 waves per workgroup, each with up to 5 K-steps of loads in flight
    dim3 grid((T + 15) / 16, (E + 15) / 16);
    if (H % 2560 == 0)
      router_logits_kernel<1, 1, 16, 5><<<grid, 1024, 0, stream>>>(x, ldx, w_r, T, H, E, logits);
    else if (H % 512 == 0)
      router_logits_kernel<1, 1, 16, 1><<<grid, 1024, 0, stream>>>(x, ldx, w_r, T, H, E, logits);
    else
      router_logits_kernel<1, 1, 4, 1><<<grid, 256, 0, stream>>>(x, ldx, w_r, T, H, E, logits);
  } else {
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    router_logits_kernel<4, 4, 4, 1><<<grid, 256, 0, stream>>>(x, ldx, w_r, T, H, E, logits);
  }
  return hipGetLastError();
}

int router_nparts(int T, int H) { return (T <= 256 && H % 1024 == 0) ? 4 : 1; }

hipError_t launch_router_logits_parts(const uint16_t* x, int64_t ldx, const float* w_r, int T, int H, int E,
                                      float* parts, hipStream_t stream) {
  // Few tokens: 4 K ranges x (16-token, 16-expert) tiles give 4x the
  // workgroups of the single-plane launch, each with 8 waves whose loads of
  // up to 5 K-steps are all in flight at once.
  const int ks = router_nparts(T, H);
  if (ks != 4) return hipErrorInvalidValue;
  dim3 grid((T + 15) / 16, (E + 15) / 16, ks);
  if (H % 5120 == 0)
    router_logits_kernel<1, 1, 8, 5><<<grid, 512, 0, stream>>>(x, ldx, w_r, T, H, E, parts);
  else
    router_logits_kernel<1, 1, 8, 1><<<grid, 512, 0, stream>>>(x, ldx, w_r, T, H, E, parts);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router logits for many tokens as a tiled GEMM. W_r is split once per call
// into its three BF16 parts (router_split_kernel: row e of `wsplit` holds hi,
// then mid, then lo of W_r row e, H values each), so the GEMM itself is pure
// BF16 matrix-core work: L = x.hi^T + x.mid^T + x.lo^T with FP32 accumulation,
// three MFMAs per 32-wide K block as in router_logits_kernel.
//
// Workgroup tile: 64 tokens x 64 experts, 4 waves; wave (wm, wn) computes
// tokens 32 wm .. +31 x experts 32 wn .. +31 as 2 x 2 MFMA tiles (the weight
// fragment first, so each lane ends with one token and 4 consecutive experts).
// Each stage is 64 K: 128 bytes of the 64 x rows and of the 3 x 64 weight rows
// (part-major), moved global -> LDS with direct loads through a 2-stage ring
// (32 KB per stage: two workgroups share a CU), one barrier per stage.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w_r, int E, int H,
                                                           uint16_t* __restrict__ wsplit) {
  const int64_t n8 = (int64_t)E * H / 8;  // groups of 8 consecutive values (H % 8 == 0: one row each)
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < n8; g += (int64_t)gridDim.x * 256) {
    const int64_t i = g * 8;
    const int e = (int)(i / H), h = (int)(i - (int64_t)e * H);
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(w_r + i);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(w_r + i + 4);
    const float w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    bf16x8 hi, mid, lo;
    split3_bf16(w, hi, mid, lo);
    uint16_t* row = wsplit + (int64_t)e * 3 * H + h;
    *reinterpret_cast<bf16x8*>(row) = hi;
    *reinterpret_cast<bf16x8*>(row + H) = mid;
    *reinterpret_cast<bf16x8*>(row + 2 * H) = lo;
  }
}

__global__ __launch_bounds__(256, 2) void router_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                             const uint16_t* __restrict__ wsplit, int T, int H, int E,
                                                             float* __restrict__ logits) {
  constexpr int kX = 64, kW = 3 * 64, kRows = kX + kW;  // 128-byte LDS rows per stage
  constexpr int kInst = kRows / 32;                     // direct copies per wave per stage (8 rows each)
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kRows * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kRows * 128];
  asm volatile("" ::"v"(lds0), "v"(lds1) : "memory");
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int S = H / 64;

  // copy i of wave w fills LDS rows 8 (4 i + w) .. + 7: x rows first, then the
  // weight rows part by part (LDS row 64 + 64 p + k holds part p of expert e0 + k)
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(wsplit);
  uint32_t off[kInst];
#pragma unroll
  for (int i = 0; i < kInst; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    const int c = 16 * swz(row, lane & 7);
    if (row < kX) {
      const int t = t0 + row < T ? t0 + row : 0;
      off[i] = (uint32_t)((int64_t)t * ldx * 2 + c);
    } else {
      const int pr = row - kX, part = pr / 64, k = pr % 64;
      const int e = e0 + k < E ? e0 + k : 0;
      off[i] = (uint32_t)(((int64_t)e * 3 + part) * H * 2 + c);
    }
  }
  auto issue = [&](uint8_t* st, int s) {
    const int64_t o = (int64_t)s * 128;
#pragma unroll
    for (int i = 0; i < kInst; ++i)
      lds_copy16_s((8 * 4 * i < kX ? xb : wb) + o, off[i], (uint32_t)(uintptr_t)st + (8 * 4 * i + 8 * wave_u) * 128);
  };
  static_assert(kX % 32 == 0, "a copy covers x rows or weight rows only");

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const uint8_t* st, int row, int kb) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(st + row * 128 + 16 * swz(row, 2 * g4 + kb)));
  };
  auto compute = [&](const uint8_t* st) {
    bf16x8 fx[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) fx[i][kb] = frag(st, 32 * wm + 16 * i + r16, kb);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 fw[3][2];
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) fw[part][kb] = frag(st, kX + 64 * part + 32 * wn + 16 * j + r16, kb);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int part = 0; part < 3; ++part)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[part][kb], fx[i][kb], acc[i][j], 0, 0, 0);
    }
  };

  // 2-stage ring, full at start; stage s + 1 is issued once every wave has
  // passed the barrier of stage s (done with stage s - 1, whose buffer it refills)
  issue(lds0, 0);
  if (S > 1) issue(lds1, 1);
  for (int s = 0; s < S; ++s) {
    if (s == 0 && S > 1) wait_vmcnt<kInst>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage s-1 are done
    stage_barrier();
    if (s > 0 && s + 1 < S) issue((s & 1) ? lds0 : lds1, s + 1);
    compute((s & 1) ? lds1 : lds0);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 32 * wm + 16 * i + r16;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + 32 * wn + 16 * j + 4 * g4;
      float* out = logits + (int64_t)t * E + e;
      if ((E & 3) == 0 && e + 3 < E) {
        *reinterpret_cast<f32x4*>(out) = acc[i][j];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e + q < E) out[q] = acc[i][j][q];
      }
    }
  }
}

size_t router_split_bytes(int E, int H) { return (size_t)E * 3 * H * 2; }

hipError_t launch_router_logits_split(const uint16_t* x, int64_t ldx, const float* w_r, int T, int H, int E,
                                      uint16_t* wsplit, float* logits, hipStream_t stream) {
  const int64_t n8 = (int64_t)E * H / 8;
  const unsigned sgrid = (unsigned)std::min<int64_t>(ceil_div(n8, 256), 2048);
  router_split_kernel<<<sgrid, 256, 0, stream>>>(w_r, E, H, wsplit);
  dim3 grid((unsigned)ceil_div(T, 64), (unsigned)ceil_div(E, 64));
  router_gemm_kernel<<<grid, 256, 0, stream>>>(x, ldx, wsplit, T, H, E, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-K selection: one wavefront per token; lane l holds experts l, l+64, ...
// Each logit becomes a 64-bit key (order-preserving image of the FP32 value
// in the high word, ~expert in the low word), so the maximum key is the
// largest value with the lowest index among equals. K rounds of a wave-wide
// maximum pick the slots in rank order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t route_key(float v, uint32_t e) {
  if (v == 0.f) v = 0.f;  // -0.0 -> +0.0
  const uint32_t b = __float_as_uint(v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~e;
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  const uint32_t b = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(b);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = shfl_xor_u64(v, off);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += shfl_xor_f64(v, off);
  return v;
}

// Group-limited selection (n_group > 1): the experts form n_group groups of
// E / n_group consecutive experts; a group's score is its best key (largest
// logit, lower expert first), the topk_group best groups are kept (equal best
// logits: the lower expert, hence the lower group) and the keys of every other
// group's experts are cleared, so the K rounds below choose only among kept
// experts.
template <int VPL>
__device__ __forceinline__ void keep_best_groups(uint64_t (&key)[VPL], int lane, int E, int n_group, int topk_group) {
  const int gs = E / n_group;
  uint64_t gkey = 0;  // lane g < n_group: best key of group g
  for (int g = 0; g < n_group; ++g) {
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && e / gs == g && key[i] > m) m = key[i];
    }
    m = wave_max_u64(m);
    if (lane == g) gkey = m;
  }
  uint64_t kept = 0;  // bit g: group g kept (n_group <= 64)
  for (int r = 0; r < topk_group; ++r) {
    const uint64_t best = wave_max_u64(gkey);
    const int g = (int)(~(uint32_t)best) / gs;
    kept |= 1ull << g;
    if (lane == g) gkey = 0;
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E && !((kept >> (e / gs)) & 1ull)) key[i] = 0ull;
  }
}

// The logit of (t, e): element t * E + e of plane 0, plus that of planes
// 1 .. NP - 1 in plane order (NP > 1: partial sums of the router's K ranges).
// NP is a compile-time count so that the NP loads are issued together.
template <int NP>
__device__ __forceinline__ float logit_at(const LogitSrc& s, int64_t i) {
  float v[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) v[c] = s.p[c * s.plane + i];
  float r = v[0];
#pragma unroll
  for (int c = 1; c < NP; ++c) r += v[c];
  return r;
}

// Routing options (Dots3NoteTextConfig n_group, topk_group, norm_topk_prob,
// routed_scaling_factor).
struct RouteOpts {
  int n_group, topk_group;
  bool renormalize;
  float scaling;
};

template <int VPL, int NP>
__global__ __launch_bounds__(256) void route_kernel(const LogitSrc src, int T, int E, int K, RouteOpts opt,
                                                    int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t row = (int64_t)t * E;
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0ull;  // 0 sorts below every finite key
    if (e < E) {
      const float v = logit_at<NP>(src, row + e);
      if (src.out) src.out[row + e] = v;
      key[i] = route_key(v, (uint32_t)e);
    }
  }
  if (opt.n_group > 1) keep_best_groups(key, lane, E, opt.n_group, opt.topk_group);
  uint64_t mine = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (key[i] == best) key[i] = 0ull;
    if (lane == k) mine = best;
  }
  // Weights: exp(l_k - l_max) over the selected set (renormalised) or over all
  // E experts, in double, times the scaling factor, rounded once. Slot 0 holds
  // the largest logit of all experts (its group always has the best score).
  const float v = key_value(mine);
  const float vmax = __shfl(v, 0);
  const double ex = lane < K ? exp((double)v - (double)vmax) : 0.0;
  double sum;
  if (opt.renormalize) {
    sum = wave_sum_f64(ex);
  } else {
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) part += exp((double)logit_at<NP>(src, row + e) - (double)vmax);
    }
    sum = wave_sum_f64(part);
  }
  if (lane < K) {
    ids[(int64_t)t * K + lane] = (int32_t)(~(uint32_t)mine);
    wts[(int64_t)t * K + lane] = (float)(ex / sum * (double)opt.scaling);
  }
}

// ---------------------------------------------------------------------------
// Sigmoid scoring with a selection-only correction bias (the bias-balanced
// routers the Transformers documentation "Dots 3 Note Preview" names in its aux_loss entry: DeepSeek-V3 and
// its derivatives). s = f32(1 / (1 + exp(-l))) evaluated in double; the key
// of expert e is f32(s + bias[e]); a group's score is f32(b1 + b2), its two
// largest biased scores; weights come from the unbiased s.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_score(float l) { return (float)(1.0 / (1.0 + exp(-(double)l))); }

template <int VPL, int NP>
__global__ __launch_bounds__(256) void route_sigmoid_kernel(const LogitSrc src, const float* __restrict__ bias,
                                                            int T, int E, int K, RouteOpts opt,
                                                            int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t row = (int64_t)t * E;
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float l = logit_at<NP>(src, row + e);
      if (src.out) src.out[row + e] = l;
      const float b = sigmoid_score(l) + (bias ? bias[e] : 0.f);
      key[i] = route_key(b, (uint32_t)e);
    } else {
      key[i] = 0ull;
    }
  }
  if (opt.n_group > 1) {
    const int gs = E / opt.n_group;
    uint64_t gkey = 0;  // lane g: key of group g's score
    for (int g = 0; g < opt.n_group; ++g) {
      uint64_t m1 = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && e / gs == g && key[i] > m1) m1 = key[i];
      }
      m1 = wave_max_u64(m1);
      float score = key_value(m1);
      if (gs > 1) {
        uint64_t m2 = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          const int e = lane + 64 * i;
          if (e < E && e / gs == g && key[i] != m1 && key[i] > m2) m2 = key[i];
        }
        m2 = wave_max_u64(m2);
        score = score + key_value(m2);
      }
      if (lane == g) gkey = route_key(score, (uint32_t)g);
    }
    uint64_t kept = 0;
    for (int r = 0; r < opt.topk_group; ++r) {
      const uint64_t best = wave_max_u64(gkey);
      const int g = (int)(~(uint32_t)best);
      kept |= 1ull << g;
      if (lane == g) gkey = 0;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((kept >> (e / gs)) & 1ull)) key[i] = 0ull;
    }
  }
  uint64_t mine = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (key[i] == best) key[i] = 0ull;
    if (lane == k) mine = best;
  }
  const int e = (int)(~(uint32_t)mine);
  const double s = lane < K ? (double)sigmoid_score(logit_at<NP>(src, row + e)) : 0.0;
  const double sum = opt.renormalize ? wave_sum_f64(s) : 1.0;
  if (lane < K) {
    ids[(int64_t)t * K + lane] = e;
    wts[(int64_t)t * K + lane] = (float)(s / sum * (double)opt.scaling);
  }
}

hipError_t launch_route_sigmoid(const LogitSrc& logits, const float* bias, int T, int E, int K, int n_group,
                                int topk_group, bool renormalize, float scaling, int32_t* ids, float* w,
                                hipStream_t stream) {
  const dim3 grid((T + 3) / 4);
  const int vpl = (E + 63) / 64;
  const RouteOpts opt{n_group, topk_group, renormalize, scaling};
  auto go = [&](auto npc) {
    constexpr int NP = decltype(npc)::value;
    if (vpl <= 1) route_sigmoid_kernel<1, NP><<<grid, 256, 0, stream>>>(logits, bias, T, E, K, opt, ids, w);
    else if (vpl <= 2) route_sigmoid_kernel<2, NP><<<grid, 256, 0, stream>>>(logits, bias, T, E, K, opt, ids, w);
    else if (vpl <= 4) route_sigmoid_kernel<4, NP><<<grid, 256, 0, stream>>>(logits, bias, T, E, K, opt, ids, w);
    else if (vpl <= 8) route_sigmoid_kernel<8, NP><<<grid, 256, 0, stream>>>(logits, bias, T, E, K, opt, ids, w);
    else route_sigmoid_kernel<16, NP><<<grid, 256, 0, stream>>>(logits, bias, T, E, K, opt, ids, w);
  };
  if (logits.n == 1) go(std::integral_constant<int, 1>{});
  else if (logits.n == 4) go(std::integral_constant<int, 4>{});
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_route(const LogitSrc& logits, int T, int E, int K, int n_group, int topk_group, bool renormalize,
                        float scaling, int32_t* ids, float* w, hipStream_t stream) {
  const dim3 grid((T + 3) / 4);
  const int vpl = (E + 63) / 64;
  const RouteOpts opt{n_group, topk_group, renormalize, scaling};
  auto go = [&](auto npc) {
    constexpr int NP = decltype(npc)::value;
    if (vpl <= 1) route_kernel<1, NP><<<grid, 256, 0, stream>>>(logits, T, E, K, opt, ids, w);
    else if (vpl <= 2) route_kernel<2, NP><<<grid, 256, 0, stream>>>(logits, T, E, K, opt, ids, w);
    else if (vpl <= 4) route_kernel<4, NP><<<grid, 256, 0, stream>>>(logits, T, E, K, opt, ids, w);
    else if (vpl <= 8) route_kernel<8, NP><<<grid, 256, 0, stream>>>(logits, T, E, K, opt, ids, w);
    else route_kernel<16, NP><<<grid, 256, 0, stream>>>(logits, T, E, K, opt, ids, w);
  };
  if (logits.n == 1) go(std::integral_constant<int, 1>{});
  else if (logits.n == 4) go(std::integral_constant<int, 4>{});
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dmoe
