// Internal launchers between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <algorithm>
#include <stdint.h>

#include "../../include/dmoe.h"
#include "dmoe_device.h"

namespace dmoe {

// Sets the calling thread's dmoe_last_error text and returns `code` (api.hip).
dmoe_status set_error(dmoe_status code, const char* fmt, ...);

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline int64_t ceil_div(int64_t v, int64_t m) { return (v + m - 1) / m; }

// route.hip
hipError_t launch_router_logits(const uint16_t* x, int64_t ldx, const float* w_r, int T, int H, int E,
                                float* logits, hipStream_t stream);
// Many tokens: W_r split once into its BF16 parts in `wsplit` (router_split_bytes)
// and a tiled BF16 GEMM; requires H % 64 == 0 and T * ldx * 2 <= 4 GiB.
size_t router_split_bytes(int E, int H);
hipError_t launch_router_logits_split(const uint16_t* x, int64_t ldx, const float* w_r, int T, int H, int E,
                                      uint16_t* wsplit, float* logits, hipStream_t stream);
// Few tokens in dmoe_forward: router_nparts(T, H) > 1 partial planes [n][T][E]
// over equal K ranges, which the route launches add in plane order.
int router_nparts(int T, int H);
hipError_t launch_router_logits_parts(const uint16_t* x, int64_t ldx, const float* w_r, int T, int H, int E,
                                      float* parts, hipStream_t stream);
// Where the route launches read the logits: n planes (1 or 4) of `plane`
// floats from p (n = 1: the logits themselves); out != nullptr: the summed
// logits are stored there.
struct LogitSrc {
  const float* p;
  int n;
  int64_t plane;
  float* out;
};
// n_group <= 1: ungrouped; renormalize: divide by the selected experts' sum (norm_topk_prob)
hipError_t launch_route(const LogitSrc& logits, int T, int E, int K, int n_group, int topk_group, bool renormalize,
                        float scaling, int32_t* ids, float* w, hipStream_t stream);
// sigmoid scoring; bias: per-expert selection bias or nullptr
hipError_t launch_route_sigmoid(const LogitSrc& logits, const float* bias, int T, int E, int K, int n_group,
                                int topk_group, bool renormalize, float scaling, int32_t* ids, float* w,
                                hipStream_t stream);

// permute.hip
constexpr int kPermutePairs = 512;  // (token, slot) pairs per permutation block
size_t permute_ws_bytes(int T, int K, int E_loc);
hipError_t launch_permute(const int32_t* ids, int T, int K, int e0, int E_loc, int32_t* offsets,
                          int32_t* row_token, int32_t* row_slot, int32_t* token_row, void* ws,
                          hipStream_t stream);

// quant.hip
// skip_from (device pointer, may be null): rows [*skip_from, skip_to) are not touched
hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int64_t ldx, uint8_t* q, int64_t ldq,
                            float* scales, int64_t lds, hipStream_t stream, const int32_t* skip_from = nullptr,
                            int skip_to = 0);
hipError_t launch_quant_weight_blocks(const float* w, int rows, int cols, int64_t ldw, uint8_t* q, int64_t ldq,
                                      float* scales, hipStream_t stream);

// gemm.hip
struct GemmArgs {
  int dtype;              // DMOE_BF16 / DMOE_FP8_E4M3
  const void* a;          // activations (BF16 or E4M3 codes)
  int64_t lda;            // elements
  const float* a_scales;  // FP8: per row and 128-column slice
  int64_t ldas;
  const int32_t* row_token;  // gather map for the A rows (NULL: identity)
  const int32_t* offsets;    // [E_loc + 1]
  int E_loc;
  int max_rows;
  const void* w0;  // gate (gate/up) or down weights
  const void* w1;  // up (gate/up only)
  int64_t ldw;     // elements
  const float* ws0;
  const float* ws1;
  int K;           // reduction length (valid): H for gate/up, F for down
  int N;           // valid output columns: F for gate/up, H for down
  uint16_t* out;   // BF16 [rows, ldo]
  int64_t ldo;
  void* ws;               // tile schedule (gemm_ws_bytes)
  bool scheduled = false; // true: ws already holds the schedule for these offsets and max_rows
  // Optional extra group computed in the same launch (the shared expert): rows
  // [x_row0, x_row0 + x_rows) of the output row space, identity token map
  // (A row = row - x_a_base), its own weights and scales (same N and K).
  int x_rows = 0;
  int x_row0 = 0;
  int x_a_base = 0;
  const void* xw0 = nullptr;
  const void* xw1 = nullptr;
  const float* xws0 = nullptr;
  const float* xws1 = nullptr;
  // FP8 gate/up only, when gemm_fuses_h_quant(): quantise h in the epilogue
  // into codes out_q [rows, ldo] and scales out_s [rows, ld_s] instead of
  // writing BF16 h to out
  uint8_t* out_q = nullptr;
  float* out_s = nullptr;
  int64_t ld_s = 0;
};
size_t gemm_ws_bytes(int max_rows, int E_loc, int extra_rows = 0);
hipError_t launch_schedule(const int32_t* offsets, int E_loc, int max_rows, int extra_rows, int extra_row0,
                           void* ws, hipStream_t stream);
// true when launch_gemm_* picks the weight-streaming kernel (it needs no tile schedule)
bool gemm_uses_stream(int max_rows, int E_loc);
// true when the FP8 gate/up launch can quantise h in its epilogue (GemmArgs.out_q)
// true when the FP8 gate/up launch of this shape runs on the wide kernel with h
// quantised in its epilogue (build option DMOE_WIDE_GU); N = output columns (F)
bool gemm_fuses_h_quant(int max_rows, int E_loc, int extra_rows, int N);
// name of the kernel a gate/up launch of this shape runs (the launcher's rule)
const char* gemm_gateup_kernel_name(int dtype, int max_rows, int E_loc, int extra_rows, int N);
const char* gemm_down_kernel_name(int dtype, int max_rows, int E_loc, int extra_rows, int N);
hipError_t launch_gemm_gateup(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t stream);
hipError_t launch_fill_offsets(int32_t* offsets, int rows, hipStream_t stream);

// combine.hip
hipError_t launch_combine(const uint16_t* o, int64_t ldo, const int32_t* token_row, const float* w,
                          const uint16_t* s, int64_t lds, int T_s, int T, int K, int H, uint16_t* y, int64_t ldy,
                          hipStream_t stream);

}  // namespace dmoe
