// Expert-contiguous permutation of the routed (token, slot) pairs.
//
// The pages fix only the routing (Transformers documentation "Dots 3 Note Preview",
// Dots3NoteTextConfig num_experts_per_tok) and the EP8 deployment whose
// grouped expert GEMMs need each expert's rows contiguous (SGLang cookbook
// "Dots3-Note", Deployment: DP8 attention x TP8 x EP8, MoE runner). The order
// is a stable counting sort over the flat pair index p = t*K + k, so rows are
// ordered by (local expert, token) and the result is unique.
//
// Pairs are cut into blocks of kPermutePairs. Inside a block each local
// expert gets a kPermutePairs-bit LDS mask of the pairs routed to it; the
// rank of a pair among its expert's pairs in the block is a popcount of the
// mask bits below it. Masks are built with atomic OR, which is order
// independent, so the result is the same on every run.
//   count:   per-block, per-expert counts
//   scan:    exclusive prefix over blocks (per expert) and over experts (offsets)
//   scatter: rows = offsets[e] + block prefix + in-block rank
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kMaskWords = kPermutePairs / 32;

__device__ __forceinline__ void build_masks(const int32_t* __restrict__ ids, int64_t pbeg, int np, int e0,
                                            int E_loc, uint32_t* mask) {
  for (int i = threadIdx.x; i < E_loc * kMaskWords; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  for (int pl = threadIdx.x; pl < np; pl += blockDim.x) {
    const int e = ids[pbeg + pl] - e0;
    if ((unsigned)e < (unsigned)E_loc) atomicOr(&mask[e * kMaskWords + (pl >> 5)], 1u << (pl & 31));
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ ids, int64_t npairs,
                                                            int e0, int E_loc, int32_t* __restrict__ counts) {
  extern __shared__ uint32_t mask[];
  const int64_t pbeg = (int64_t)blockIdx.x * kPermutePairs;
  const int np = (int)min<int64_t>(kPermutePairs, npairs - pbeg);
  build_masks(ids, pbeg, np, e0, E_loc, mask);
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) c += __popc(mask[e * kMaskWords + w]);
    counts[(int64_t)blockIdx.x * E_loc + e] = c;
  }
}

// Exclusive scan of n ints in LDS by one workgroup of blockDim.x threads.
__device__ void block_exclusive_scan(int32_t* v, int n, int32_t* partial, int32_t* total) {
  const int nt = blockDim.x, t = threadIdx.x;
  const int chunk = (n + nt - 1) / nt;
  const int b = min(n, t * chunk), e = min(n, b + chunk);
  int32_t s = 0;
  for (int i = b; i < e; ++i) s += v[i];
  partial[t] = s;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {  // inclusive Hillis-Steele over the per-thread sums
    const int32_t add = t >= off ? partial[t - off] : 0;
    __syncthreads();
    partial[t] += add;
    __syncthreads();
  }
  int32_t run = partial[t] - s;
  for (int i = b; i < e; ++i) {
    const int32_t x = v[i];
    v[i] = run;
    run += x;
  }
  if (t == nt - 1) *total = partial[t];
  __syncthreads();
}

// One workgroup: prefix over blocks for every expert, then offsets over experts.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ counts, int nblocks, int E_loc,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[1024];
  __shared__ int32_t partial[1024];
  __shared__ int32_t total;
  // a thread walks one expert's column of counts, 16 independent loads in flight per step
  constexpr int kChunk = 16;
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) {
    int32_t run = 0;
    for (int b0 = 0; b0 < nblocks; b0 += kChunk) {
      int32_t c[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) c[j] = b0 + j < nblocks ? counts[(int64_t)(b0 + j) * E_loc + e] : 0;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (b0 + j < nblocks) counts[(int64_t)(b0 + j) * E_loc + e] = run;
        run += c[j];
      }
    }
    tot[e] = run;
  }
  __syncthreads();
  block_exclusive_scan(tot, E_loc, partial, &total);
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) offsets[e] = tot[e];
  if (threadIdx.x == 0) offsets[E_loc] = total;
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t* __restrict__ ids, int64_t npairs,
                                                              int K, int e0, int E_loc,
                                                              const int32_t* __restrict__ block_base,
                                                              const int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ row_slot,
                                                              int32_t* __restrict__ token_row) {
  extern __shared__ uint32_t mask[];
  const int64_t pbeg = (int64_t)blockIdx.x * kPermutePairs;
  const int np = (int)min<int64_t>(kPermutePairs, npairs - pbeg);
  build_masks(ids, pbeg, np, e0, E_loc, mask);
  for (int pl = threadIdx.x; pl < np; pl += blockDim.x) {
    const int64_t p = pbeg + pl;
    const int e = ids[p] - e0;
    if ((unsigned)e < (unsigned)E_loc) {
      const uint32_t* m = mask + e * kMaskWords;
      const int w = pl >> 5;
      int rank = __popc(m[w] & ((1u << (pl & 31)) - 1u));
      for (int i = 0; i < w; ++i) rank += __popc(m[i]);
      const int32_t row = offsets[e] + block_base[(int64_t)blockIdx.x * E_loc + e] + rank;
      row_token[row] = (int32_t)(p / K);
      row_slot[row] = (int32_t)(p % K);
      token_row[p] = row;
    } else {
      token_row[p] = -1;
    }
  }
}

// All pairs in one block (T*K <= kPermutePairs): masks, counts, offsets and the
// scatter in a single workgroup.
__global__ __launch_bounds__(256) void permute_single_kernel(const int32_t* __restrict__ ids, int npairs, int K,
                                                             int e0, int E_loc, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_token,
                                                             int32_t* __restrict__ row_slot,
                                                             int32_t* __restrict__ token_row) {
  extern __shared__ uint32_t smem[];
  uint32_t* mask = smem;                                          // E_loc * kMaskWords
  int32_t* base = reinterpret_cast<int32_t*>(smem + E_loc * kMaskWords);  // E_loc
  __shared__ int32_t partial[256];
  __shared__ int32_t total;
  build_masks(ids, 0, npairs, e0, E_loc, mask);
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) c += __popc(mask[e * kMaskWords + w]);
    base[e] = c;
  }
  __syncthreads();
  block_exclusive_scan(base, E_loc, partial, &total);
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) offsets[e] = base[e];
  if (threadIdx.x == 0) offsets[E_loc] = total;
  for (int pl = threadIdx.x; pl < npairs; pl += blockDim.x) {
    const int e = ids[pl] - e0;
    if ((unsigned)e < (unsigned)E_loc) {
      const uint32_t* m = mask + e * kMaskWords;
      const int w = pl >> 5;
      int rank = __popc(m[w] & ((1u << (pl & 31)) - 1u));
      for (int i = 0; i < w; ++i) rank += __popc(m[i]);
      const int32_t row = base[e] + rank;
      row_token[row] = pl / K;
      row_slot[row] = pl % K;
      token_row[pl] = row;
    } else {
      token_row[pl] = -1;
    }
  }
}

size_t permute_ws_bytes(int T, int K, int E_loc) {
  const int64_t nb = ceil_div((int64_t)T * K, kPermutePairs);
  return (size_t)round_up(std::max<int64_t>(nb, 1) * E_loc * 4, 256);
}

hipError_t launch_permute(const int32_t* ids, int T, int K, int e0, int E_loc, int32_t* offsets,
                          int32_t* row_token, int32_t* row_slot, int32_t* token_row, void* ws,
                          hipStream_t stream) {
  const int64_t npairs = (int64_t)T * K;
  const int nb = (int)ceil_div(npairs, kPermutePairs);
  int32_t* counts = static_cast<int32_t*>(ws);
  const size_t lds = (size_t)E_loc * kMaskWords * 4;
  if (nb == 1 && E_loc <= 512) {
    permute_single_kernel<<<1, 256, lds + (size_t)E_loc * 4, stream>>>(ids, (int)npairs, K, e0, E_loc, offsets,
                                                                      row_token, row_slot, token_row);
    return hipGetLastError();
  }
  if (nb > 0) permute_count_kernel<<<nb, 256, lds, stream>>>(ids, npairs, e0, E_loc, counts);
  permute_scan_kernel<<<1, 1024, 0, stream>>>(counts, nb, E_loc, offsets);
  if (nb > 0)
    permute_scatter_kernel<<<nb, 256, lds, stream>>>(ids, npairs, K, e0, E_loc, counts, offsets, row_token,
                                                      row_slot, token_row);
  return hipGetLastError();
}

}  // namespace dmoe
