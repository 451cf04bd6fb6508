// Shared pieces of the grouped expert GEMM kernels (gemm.hip: tile kernel for
// many rows per expert; gemm_stream.hip: weight-streaming kernel for few).
#pragma once

#include <type_traits>

#include "dmoe_internal.h"

namespace dmoe {

constexpr int kBM = 128;            // rows per tile
constexpr int kKB = 128;            // K bytes per stage
constexpr int kWideBM = 256;        // rows per tile of the wide kernel (gemm_wide.hip)
constexpr int kMaxSlices = 128;     // FP8 tile kernel: at most 128 scale slices along K (K <= 16384)

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
  int E_loc;
  int x_rows, x_row0, x_a_base;  // extra (shared-expert) group, see GemmArgs
  int x_chunk;                   // > 0: group indices >= E_loc are consecutive chunks of x_chunk rows
  const uint8_t* xw0;
  const uint8_t* xw1;
  const float* xws0;
  const float* xws1;
  // FP8 gate/up in the layer: h quantised in the epilogue (1x128 rule) into
  // codes out_q [rows, ldo] and scales out_s [rows, ld_s]; nullptr: BF16 h in out
  uint8_t* out_q;
  float* out_s;
  int64_t ld_s;
};

// Weights, scales and rows of group g: a routed expert (g < E_loc) or the extra group.
struct GroupView {
  const uint8_t* w0;
  const uint8_t* w1;
  const float* s0;  // block scales of this group, [nNb][nKb]
  const float* s1;
  int row_beg, row_end;
  bool gather;  // A row = row_token[r]; otherwise A row = r - a_base
  int a_base;
};

__device__ __forceinline__ GroupView group_view(const TileArgs& p, int g) {
  GroupView v;
  if (g < p.E_loc) {
    v.w0 = p.w0 + g * p.w_expert_b;
    v.w1 = p.w1 ? p.w1 + g * p.w_expert_b : nullptr;
    v.s0 = p.ws0 ? p.ws0 + (int64_t)g * p.nNb * p.nKb : nullptr;
    v.s1 = p.ws1 ? p.ws1 + (int64_t)g * p.nNb * p.nKb : nullptr;
    v.row_beg = p.offsets[g];
    v.row_end = p.offsets[g + 1];
    v.gather = p.row_token != nullptr;
    v.a_base = 0;
  } else {
    v.w0 = p.xw0;
    v.w1 = p.xw1;
    v.s0 = p.xws0;
    v.s1 = p.xws1;
    v.row_beg = p.x_row0 + (p.x_chunk > 0 ? (g - p.E_loc) * p.x_chunk : 0);
    v.row_end = p.x_chunk > 0 ? min(p.x_row0 + p.x_rows, v.row_beg + p.x_chunk) : p.x_row0 + p.x_rows;
    v.gather = false;
    v.a_base = p.x_a_base;
  }
  return v;
}

__device__ __forceinline__ int64_t a_row(const TileArgs& p, const GroupView& v, int r) {
  return v.gather ? (int64_t)p.row_token[r] : (int64_t)(r - v.a_base);
}

// Operand modes of the tile kernels. Every mode moves 128-byte K rows through LDS.
//  kModeBF16: BF16 operands, 64 K per stage, BF16 MFMA.
//  kModeFP8X: E4M3 operands, 128 K per stage (one scale slice); fragments are
//             converted exactly to BF16 after the LDS read and multiplied on
//             BF16 matrix cores: every product is exact and the slice's sum is
//             accumulated in FP32 before the a_scale * w_scale promotion.
//  kModeFP8:  E4M3 operands, 128 K per stage (one scale slice), FP8 MFMA
//             (the matrix core's own accumulation precision within a slice).
constexpr int kModeBF16 = 0, kModeFP8X = 1, kModeFP8 = 2;

// Wave-uniform copy of a pointer (lets the compiler use scalar loads through it).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

__device__ __forceinline__ void e4m3x16_to_bf16(const i32x4 src, i32x4& lo, i32x4& hi) {
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

// LDS rows are 128 bytes; their 16-byte units are XOR-swizzled by a row-dependent
// constant. A fragment read (ds_read_b128) has lanes 16 g4 + r16 read row
// base + r16 (base a multiple of 16), unit 2 g4 + h. Measured on gfx950, a
// 128-bit read is conflict-free when the 32 lanes served together touch 32
// distinct 16-byte units modulo 512 bytes, i.e. distinct (row & 3, unit) pairs;
// XOR by (row & 7) ^ ((row >> 3) & 1) gives the 8 (row >> 2, g4 & 1) combinations
// of each row & 3 distinct units (about 1.85x the LDS read rate of XOR by
// (row >> 1) & 7 on that pattern).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Asynchronous global -> LDS copies of 16 (or 4) bytes per lane: lane l writes
// LDS bytes [base + 16 l, +16) (resp. [base + 4 l, +4)); base is wave-uniform
// and is passed in M0 (an input operand bound to that register, so the
// compiler sets M0 itself and knows it is read). Issued from asm so that the
// compiler's wait insertion, which cannot tell the pipeline's LDS buffers
// apart, does not make every LDS read wait for every copy in flight; the
// pipeline waits on vmcnt itself. The instruction writes no register, so
// nothing of it is live after issue.
__device__ __forceinline__ void lds_copy16(const void* gptr, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}
// Weights that one launch reads once: the non-temporal policy (nt) marks the
// lines for early eviction, so a stream of several GB does not push reused
// data (activation rows, other workgroups' stages) out of L2 and the
// memory-side cache. Measured on the decode launches: 6.15 -> 6.78 TB/s.
__device__ __forceinline__ void lds_copy16_nt(const void* gptr, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void lds_copy4(const void* gptr, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}

// The same copies with the global address split into a wave-uniform 64-bit base
// (SGPRs) and a per-lane 32-bit byte offset, so that moving to the next stage
// is a scalar add and the per-lane offsets stay in place.
__device__ __forceinline__ void lds_copy16_s(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void lds_copy16_s_nt(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void lds_copy4_s(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// half would wait for every outstanding global load, including the younger
// pipeline stages). Callers order memory with explicit s_waitcnt first; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

hipError_t launch_gemm_wide(const TileArgs& p, int dtype, bool gateup, int npad, int cap, hipStream_t stream);
hipError_t launch_gemm_stream(const TileArgs& p, int dtype, bool gateup, int rows_per_expert, int n_pad,
                              int E_loc, hipStream_t stream);

}  // namespace dmoe
