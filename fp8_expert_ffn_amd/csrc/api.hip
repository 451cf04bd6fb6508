// C-ABI entry points of libdmoe: argument validation on the host, then the
// kernel launches on the caller's stream. Nothing here allocates, frees,
// synchronises or reads device memory.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

#include "dmoe_internal.h"

using namespace dmoe;

namespace {

thread_local char g_err[512] = "";

dmoe_status fail(dmoe_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

dmoe_status ok() {
  g_err[0] = '\0';
  return DMOE_OK;
}

dmoe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQ(cond, code, ...)                  \
  do {                                        \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQ_PTR(p, name) REQ((p) != nullptr, DMOE_ERR_INVALID_ARG, "%s is NULL", name)
#define REQ_AL(p, name) REQ(aligned16(p), DMOE_ERR_ALIGNMENT, "%s is not 16-byte aligned", name)

int dtype_size(int dtype) { return dtype == DMOE_FP8_E4M3 ? 1 : 2; }

dmoe_status check_dtype(int dtype) {
  REQ(dtype == DMOE_BF16 || dtype == DMOE_FP8_E4M3, DMOE_ERR_UNSUPPORTED, "dtype %d is not DMOE_BF16 or DMOE_FP8_E4M3",
      dtype);
  return DMOE_OK;
}

// Pitch requirement: rows start 16-byte aligned.
dmoe_status check_pitch(int64_t ld, int64_t min_ld, int elem, const char* name) {
  REQ(ld >= min_ld, DMOE_ERR_INVALID_ARG, "%s = %lld is below the row width %lld", name, (long long)ld,
      (long long)min_ld);
  REQ((ld * elem) % 16 == 0, DMOE_ERR_ALIGNMENT, "%s = %lld elements is not a multiple of 16 bytes", name,
      (long long)ld);
  return DMOE_OK;
}

#define TRY(expr)                    \
  do {                               \
    dmoe_status st_ = (expr);        \
    if (st_ != DMOE_OK) return st_;  \
  } while (0)

}  // namespace

dmoe_status dmoe::set_error(dmoe_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

extern "C" {

const char* dmoe_last_error(void) { return g_err; }
int32_t dmoe_abi_version(void) { return DMOE_ABI_VERSION; }

// ---------------------------------------------------------------------------
dmoe_status dmoe_router_logits(const uint16_t* x, int64_t ldx, const float* w_r, int32_t T, int32_t H, int32_t E,
                               float* logits, hipStream_t stream) {
  REQ(T >= 0, DMOE_ERR_INVALID_ARG, "T = %d < 0", T);
  REQ(H > 0 && H % 128 == 0, DMOE_ERR_INVALID_ARG, "H = %d must be a positive multiple of 128", H);
  REQ(E >= 1 && E <= 1024, DMOE_ERR_INVALID_ARG, "E = %d outside [1, 1024]", E);
  if (T == 0) return ok();
  REQ_PTR(x, "x");
  REQ_PTR(w_r, "w_r");
  REQ_PTR(logits, "logits");
  REQ_AL(x, "x");
  REQ_AL(w_r, "w_r");
  TRY(check_pitch(ldx, H, 2, "ldx"));
  return hip_status(launch_router_logits(x, ldx, w_r, T, H, E, logits, stream), "router_logits launch");
}

namespace {
// Group-limited routing options; n_group 0 or 1 means ungrouped, topk_group 0 means every group.
dmoe_status check_route_opts(int32_t E, int32_t K, int32_t n_group, int32_t topk_group, float scaling) {
  const int32_t g = n_group <= 1 ? 1 : n_group;
  const int32_t tg = topk_group <= 0 ? g : topk_group;
  REQ(n_group >= 0 && n_group <= 64, DMOE_ERR_INVALID_ARG, "n_group = %d outside [0, 64]", n_group);
  REQ(E % g == 0, DMOE_ERR_INVALID_ARG, "E = %d is not a multiple of n_group = %d", E, g);
  REQ(tg >= 1 && tg <= g, DMOE_ERR_INVALID_ARG, "topk_group = %d outside [1, n_group = %d]", topk_group, g);
  REQ((int64_t)K <= (int64_t)tg * (E / g), DMOE_ERR_INVALID_ARG,
      "K = %d exceeds the %d experts of topk_group = %d groups", K, tg * (E / g), tg);
  REQ(scaling > 0.f && scaling < 3.0e38f, DMOE_ERR_INVALID_ARG, "routed_scaling_factor must be positive and finite");
  return DMOE_OK;
}
}  // namespace

dmoe_status dmoe_route_grouped(const float* logits, int32_t T, int32_t E, int32_t K, int32_t n_group,
                               int32_t topk_group, int32_t renormalize, float routed_scaling_factor,
                               int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  REQ(T >= 0, DMOE_ERR_INVALID_ARG, "T = %d < 0", T);
  REQ(E >= 1 && E <= 1024, DMOE_ERR_INVALID_ARG, "E = %d outside [1, 1024]", E);
  REQ(K >= 1 && K <= E && K <= 64, DMOE_ERR_INVALID_ARG, "K = %d outside [1, min(E, 64)]", K);
  TRY(check_route_opts(E, K, n_group, topk_group, routed_scaling_factor));
  if (T == 0) return ok();
  REQ_PTR(logits, "logits");
  REQ_PTR(topk_ids, "topk_ids");
  REQ_PTR(topk_w, "topk_w");
  const int g = n_group <= 1 ? 1 : n_group;
  return hip_status(launch_route(LogitSrc{logits, 1, 0, nullptr}, T, E, K, g, topk_group <= 0 ? g : topk_group,
                                 renormalize != 0,
                                 routed_scaling_factor, topk_ids, topk_w, stream),
                    "route launch");
}

dmoe_status dmoe_route(const float* logits, int32_t T, int32_t E, int32_t K, int32_t* topk_ids, float* topk_w,
                       hipStream_t stream) {
  return dmoe_route_grouped(logits, T, E, K, 1, 1, 1, 1.0f, topk_ids, topk_w, stream);
}

dmoe_status dmoe_route_sigmoid(const float* logits, const float* score_bias, int32_t T, int32_t E, int32_t K,
                               int32_t n_group, int32_t topk_group, int32_t renormalize, float routed_scaling_factor,
                               int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  REQ(T >= 0, DMOE_ERR_INVALID_ARG, "T = %d < 0", T);
  REQ(E >= 1 && E <= 1024, DMOE_ERR_INVALID_ARG, "E = %d outside [1, 1024]", E);
  REQ(K >= 1 && K <= E && K <= 64, DMOE_ERR_INVALID_ARG, "K = %d outside [1, min(E, 64)]", K);
  TRY(check_route_opts(E, K, n_group, topk_group, routed_scaling_factor));
  if (T == 0) return ok();
  REQ_PTR(logits, "logits");
  REQ_PTR(topk_ids, "topk_ids");
  REQ_PTR(topk_w, "topk_w");
  const int g = n_group <= 1 ? 1 : n_group;
  return hip_status(launch_route_sigmoid(LogitSrc{logits, 1, 0, nullptr}, score_bias, T, E, K, g,
                                         topk_group <= 0 ? g : topk_group,
                                         renormalize != 0, routed_scaling_factor, topk_ids, topk_w, stream),
                    "route launch");
}

size_t dmoe_permute_ws_bytes(int32_t T, int32_t K, int32_t E_loc) {
  if (T < 0 || K < 1 || E_loc < 1) return 0;
  return permute_ws_bytes(T, K, E_loc);
}

dmoe_status dmoe_permute(const int32_t* topk_ids, int32_t T, int32_t K, int32_t e0, int32_t E_loc,
                         int32_t* offsets, int32_t* row_token, int32_t* row_slot, int32_t* token_row, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  REQ(T >= 0, DMOE_ERR_INVALID_ARG, "T = %d < 0", T);
  REQ(K >= 1 && K <= 1024, DMOE_ERR_INVALID_ARG, "K = %d outside [1, 1024]", K);
  REQ(E_loc >= 1 && E_loc <= 1024, DMOE_ERR_INVALID_ARG, "E_loc = %d outside [1, 1024]", E_loc);
  REQ(e0 >= 0, DMOE_ERR_INVALID_ARG, "e0 = %d < 0", e0);
  REQ((int64_t)T * K <= INT32_MAX, DMOE_ERR_INVALID_ARG, "T*K overflows int32");
  REQ_PTR(offsets, "offsets");
  if (T > 0) {
    REQ_PTR(topk_ids, "topk_ids");
    REQ_PTR(row_token, "row_token");
    REQ_PTR(row_slot, "row_slot");
    REQ_PTR(token_row, "token_row");
  }
  REQ(ws != nullptr && ws_bytes >= permute_ws_bytes(T, K, E_loc), DMOE_ERR_WORKSPACE,
      "permute workspace needs %zu bytes, got %zu", permute_ws_bytes(T, K, E_loc), ws_bytes);
  return hip_status(launch_permute(topk_ids, T, K, e0, E_loc, offsets, row_token, row_slot, token_row, ws, stream),
                    "permute launch");
}

dmoe_status dmoe_quant_act(const uint16_t* x, int32_t rows, int32_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                           float* scales, int64_t lds, hipStream_t stream) {
  REQ(rows >= 0 && cols >= 0, DMOE_ERR_INVALID_ARG, "negative size");
  REQ(cols % 8 == 0, DMOE_ERR_INVALID_ARG, "cols = %d is not a multiple of 8", cols);
  if (rows == 0 || cols == 0) return ok();
  REQ_PTR(x, "x");
  REQ_PTR(q, "q");
  REQ_PTR(scales, "scales");
  REQ_AL(x, "x");
  REQ((reinterpret_cast<uintptr_t>(q) & 7u) == 0, DMOE_ERR_ALIGNMENT, "q is not 8-byte aligned");
  TRY(check_pitch(ldx, cols, 2, "ldx"));
  REQ(ldq >= round_up(cols, 128) && ldq % 8 == 0, DMOE_ERR_INVALID_ARG,
      "ldq = %lld must be >= round_up(cols, 128) and a multiple of 8", (long long)ldq);
  REQ(lds >= ceil_div(cols, 128), DMOE_ERR_INVALID_ARG, "lds = %lld below ceil(cols/128)", (long long)lds);
  return hip_status(launch_quant_act(x, rows, cols, ldx, q, ldq, scales, lds, stream), "quant_act launch");
}

dmoe_status dmoe_quant_weight_blocks(const float* w, int32_t rows, int32_t cols, int64_t ldw, uint8_t* q,
                                     int64_t ldq, float* scales, hipStream_t stream) {
  REQ(rows >= 0 && cols >= 0, DMOE_ERR_INVALID_ARG, "negative size");
  REQ(cols % 4 == 0 && ldw % 4 == 0, DMOE_ERR_INVALID_ARG, "cols and ldw must be multiples of 4");
  if (rows == 0 || cols == 0) return ok();
  REQ_PTR(w, "w");
  REQ_PTR(q, "q");
  REQ_PTR(scales, "scales");
  REQ_AL(w, "w");
  REQ_AL(q, "q");
  REQ(ldw >= cols, DMOE_ERR_INVALID_ARG, "ldw below cols");
  REQ(ldq >= round_up(cols, 128) && ldq % 16 == 0, DMOE_ERR_INVALID_ARG,
      "ldq = %lld must be >= round_up(cols, 128) and a multiple of 16", (long long)ldq);
  return hip_status(launch_quant_weight_blocks(w, rows, cols, ldw, q, ldq, scales, stream), "quant_weight launch");
}

size_t dmoe_gemm_ws_bytes(int32_t max_rows, int32_t E_loc) {
  if (max_rows < 0 || E_loc < 1) return 0;
  return gemm_ws_bytes(max_rows, E_loc);
}

// The tile GEMM addresses every operand as a base plus a 32-bit byte offset.
static bool span_fits(int64_t rows, int64_t ld, int64_t es) { return rows * ld * es <= (int64_t(1) << 32); }

// a_rows: rows of a the call can read (< 0: not known on the host, the
// caller's row_token must stay within 4 GiB of a).
static dmoe_status check_gemm_common(int dtype, const void* a, int64_t lda, const float* a_scales, int64_t ldas,
                                     const int32_t* offsets, int E_loc, int max_rows, int Kdim, int Ndim,
                                     int64_t a_rows, const void* w0, int64_t ldw, const float* ws0, void* ws,
                                     size_t ws_bytes) {
  TRY(check_dtype(dtype));
  REQ(E_loc >= 1 && E_loc <= 1024, DMOE_ERR_INVALID_ARG, "E_loc = %d outside [1, 1024]", E_loc);
  REQ(max_rows >= 0, DMOE_ERR_INVALID_ARG, "max_rows < 0");
  REQ_PTR(offsets, "offsets");
  REQ_PTR(a, "a");
  REQ_PTR(w0, "weights");
  REQ_AL(a, "a");
  REQ_AL(w0, "weights");
  const int es = dtype_size(dtype);
  TRY(check_pitch(lda, round_up(Kdim, 128), es, "lda"));
  TRY(check_pitch(ldw, round_up(Kdim, 128), es, "ldw"));
  if (dtype == DMOE_FP8_E4M3) {
    REQ_PTR(a_scales, "a_scales");
    REQ_PTR(ws0, "weight scales");
    REQ(ldas >= ceil_div(Kdim, 128), DMOE_ERR_INVALID_ARG, "ldas below ceil(K/128)");
    REQ(Kdim <= 16384, DMOE_ERR_UNSUPPORTED, "FP8 reduction length %d above 16384", Kdim);
  }
  REQ(span_fits(round_up(Ndim, 128), ldw, es), DMOE_ERR_UNSUPPORTED, "one expert's weights span 4 GiB or more");
  REQ(a_rows < 0 || (span_fits(a_rows, lda, es) && span_fits(a_rows, ldas, 4)), DMOE_ERR_UNSUPPORTED,
      "the activation operand spans 4 GiB or more");
  REQ(ws != nullptr && ws_bytes >= gemm_ws_bytes(max_rows, E_loc), DMOE_ERR_WORKSPACE,
      "gemm workspace needs %zu bytes, got %zu", gemm_ws_bytes(max_rows, E_loc), ws_bytes);
  return DMOE_OK;
}

dmoe_status dmoe_grouped_gemm_gateup(int32_t dtype, const void* a, int64_t lda, const float* a_scales,
                                     int64_t ldas, const int32_t* row_token, const int32_t* offsets,
                                     int32_t E_loc, int32_t max_rows, const void* w_gate, const void* w_up,
                                     int64_t ldw, const float* w_scales_gate, const float* w_scales_up, int32_t H,
                                     int32_t F, uint16_t* h, int64_t ldh, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  REQ(H > 0 && H % 128 == 0, DMOE_ERR_INVALID_ARG, "H = %d must be a positive multiple of 128", H);
  REQ(F > 0 && F % 8 == 0, DMOE_ERR_INVALID_ARG, "F = %d must be a positive multiple of 8", F);
  TRY(check_gemm_common(dtype, a, lda, a_scales, ldas, offsets, E_loc, max_rows, H, F, row_token ? -1 : max_rows,
                        w_gate, ldw, w_scales_gate, ws, ws_bytes));
  REQ_PTR(w_up, "w_up");
  REQ_AL(w_up, "w_up");
  if (dtype == DMOE_FP8_E4M3) REQ_PTR(w_scales_up, "w_scales_up");
  REQ_PTR(h, "h");
  REQ_AL(h, "h");
  TRY(check_pitch(ldh, round_up(F, 128), 2, "ldh"));
  GemmArgs g{dtype, a, lda, a_scales, ldas, row_token, offsets, E_loc, max_rows, w_gate, w_up, ldw,
             w_scales_gate, w_scales_up, H, F, h, ldh, ws};
  return hip_status(launch_gemm_gateup(g, stream), "gateup launch");
}

dmoe_status dmoe_grouped_gemm_down(int32_t dtype, const void* h, int64_t ldh, const float* h_scales, int64_t ldhs,
                                   const int32_t* offsets, int32_t E_loc, int32_t max_rows, const void* w_down,
                                   int64_t ldw, const float* w_scales_down, int32_t F, int32_t H, uint16_t* o,
                                   int64_t ldo, void* ws, size_t ws_bytes, hipStream_t stream) {
  REQ(H > 0 && H % 128 == 0, DMOE_ERR_INVALID_ARG, "H = %d must be a positive multiple of 128", H);
  REQ(F > 0 && F % 8 == 0, DMOE_ERR_INVALID_ARG, "F = %d must be a positive multiple of 8", F);
  TRY(check_gemm_common(dtype, h, ldh, h_scales, ldhs, offsets, E_loc, max_rows, F, H, max_rows, w_down, ldw,
                        w_scales_down, ws, ws_bytes));
  REQ_PTR(o, "o");
  REQ_AL(o, "o");
  TRY(check_pitch(ldo, H, 2, "ldo"));
  GemmArgs g{dtype, h, ldh, h_scales, ldhs, nullptr, offsets, E_loc, max_rows, w_down, nullptr, ldw,
             w_scales_down, nullptr, F, H, o, ldo, ws};
  return hip_status(launch_gemm_down(g, stream), "down launch");
}

// ---------------------------------------------------------------------------
// Shared expert: one group of T_s rows with the identity row map.
// Workspace: [offsets 256 B][gemm ws][h BF16][h codes][h scales]
// ---------------------------------------------------------------------------
namespace {
struct SharedLayout {
  int64_t offsets, gemm, h, hq, hs, total;
};
SharedLayout shared_layout(int dtype, int T_s, int H, int F_s) {
  (void)H;
  SharedLayout L;
  const int64_t fpad = round_up(F_s, 128);
  L.offsets = 0;
  L.gemm = 256;
  L.h = L.gemm + round_up((int64_t)gemm_ws_bytes(T_s, 1), 256);
  L.hq = L.h + round_up((int64_t)T_s * fpad * 2, 256);
  L.hs = L.hq + (dtype == DMOE_FP8_E4M3 ? round_up((int64_t)T_s * fpad, 256) : 0);
  L.total = L.hs + (dtype == DMOE_FP8_E4M3 ? round_up((int64_t)T_s * ceil_div(F_s, 128) * 4, 256) : 0);
  return L;
}

dmoe_status run_shared(int dtype, const void* a, int64_t lda, const float* a_scales, int64_t ldas, int T_s,
                       const void* wg, const void* wu, const void* wd, int64_t ldw_gu, int64_t ldw_d,
                       const float* sg, const float* su, const float* sd, int H, int F_s, uint16_t* s_out,
                       int64_t lds_out, uint8_t* ws, hipStream_t stream) {
  const SharedLayout L = shared_layout(dtype, T_s, H, F_s);
  int32_t* offs = reinterpret_cast<int32_t*>(ws + L.offsets);
  void* gws = ws + L.gemm;
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  const int64_t fpad = round_up(F_s, 128);
  hipError_t e = launch_fill_offsets(offs, T_s, stream);
  if (e != hipSuccess) return hip_status(e, "shared offsets");
  GemmArgs g1{dtype, a, lda, a_scales, ldas, nullptr, offs, 1, T_s, wg, wu, ldw_gu, sg, su, H, F_s, h, fpad, gws};
  e = launch_gemm_gateup(g1, stream);
  if (e != hipSuccess) return hip_status(e, "shared gateup");
  const void* ha = h;
  const float* hsc = nullptr;
  int64_t ldha = fpad, ldhs = 0;
  if (dtype == DMOE_FP8_E4M3) {
    uint8_t* hq = ws + L.hq;
    float* hs = reinterpret_cast<float*>(ws + L.hs);
    ldhs = ceil_div(F_s, 128);
    e = launch_quant_act(h, T_s, F_s, fpad, hq, fpad, hs, ldhs, stream);
    if (e != hipSuccess) return hip_status(e, "shared h quant");
    ha = hq;
    hsc = hs;
  }
  GemmArgs g2{dtype, ha, ldha, hsc, ldhs, nullptr, offs, 1, T_s, wd, nullptr, ldw_d, sd, nullptr, F_s, H,
              s_out, lds_out, gws};
  return hip_status(launch_gemm_down(g2, stream), "shared down");
}
}  // namespace

size_t dmoe_shared_expert_ws_bytes(int32_t dtype, int32_t T_s, int32_t H, int32_t F_s) {
  if (T_s < 0 || H <= 0 || F_s <= 0) return 0;
  return (size_t)shared_layout(dtype, T_s, H, F_s).total;
}

dmoe_status dmoe_shared_expert(int32_t dtype, const void* a, int64_t lda, const float* a_scales, int64_t ldas,
                               int32_t T_s, const void* w_gate, const void* w_up, const void* w_down,
                               int64_t ldw_gu, int64_t ldw_d, const float* w_scales_gate,
                               const float* w_scales_up, const float* w_scales_down, int32_t H, int32_t F_s,
                               uint16_t* s_out, int64_t lds_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  TRY(check_dtype(dtype));
  REQ(T_s >= 0, DMOE_ERR_INVALID_ARG, "T_s < 0");
  REQ(H > 0 && H % 128 == 0, DMOE_ERR_INVALID_ARG, "H = %d must be a positive multiple of 128", H);
  REQ(F_s > 0 && F_s % 8 == 0, DMOE_ERR_INVALID_ARG, "F_s = %d must be a positive multiple of 8", F_s);
  if (T_s == 0) return ok();
  REQ_PTR(a, "a");
  REQ_PTR(w_gate, "w_gate");
  REQ_PTR(w_up, "w_up");
  REQ_PTR(w_down, "w_down");
  REQ_PTR(s_out, "s_out");
  REQ_AL(a, "a");
  REQ_AL(w_gate, "w_gate");
  REQ_AL(w_up, "w_up");
  REQ_AL(w_down, "w_down");
  REQ_AL(s_out, "s_out");
  const int es = dtype_size(dtype);
  TRY(check_pitch(lda, H, es, "lda"));
  TRY(check_pitch(ldw_gu, H, es, "ldw_gu"));
  TRY(check_pitch(ldw_d, round_up(F_s, 128), es, "ldw_d"));
  TRY(check_pitch(lds_out, H, 2, "lds_out"));
  if (dtype == DMOE_FP8_E4M3) {
    REQ(a_scales && w_scales_gate && w_scales_up && w_scales_down, DMOE_ERR_INVALID_ARG, "FP8 scales missing");
    REQ(ldas >= H / 128, DMOE_ERR_INVALID_ARG, "ldas below H/128");
  }
  REQ(span_fits(T_s, lda, es) && span_fits(T_s, ldas, 4) && span_fits(round_up(F_s, 128), ldw_gu, es) &&
          span_fits(H, ldw_d, es) && span_fits(T_s, round_up(F_s, 128), 2),
      DMOE_ERR_UNSUPPORTED, "an operand spans 4 GiB or more");
  const size_t need = dmoe_shared_expert_ws_bytes(dtype, T_s, H, F_s);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, DMOE_ERR_WORKSPACE,
      "shared expert workspace needs %zu bytes, got %zu", need, ws_bytes);
  return run_shared(dtype, a, lda, a_scales, ldas, T_s, w_gate, w_up, w_down, ldw_gu, ldw_d, w_scales_gate,
                    w_scales_up, w_scales_down, H, F_s, s_out, lds_out, static_cast<uint8_t*>(ws), stream);
}

dmoe_status dmoe_combine(const uint16_t* o, int64_t ldo, const int32_t* token_row, const float* topk_w,
                         const uint16_t* s_out, int64_t lds, int32_t T_s, int32_t T, int32_t K, int32_t H,
                         uint16_t* y, int64_t ldy, hipStream_t stream) {
  REQ(T >= 0 && T_s >= 0, DMOE_ERR_INVALID_ARG, "negative token count");
  REQ(K >= 1 && K <= 64, DMOE_ERR_INVALID_ARG, "K = %d outside [1, 64]", K);
  REQ(H > 0 && H % 8 == 0, DMOE_ERR_INVALID_ARG, "H = %d must be a positive multiple of 8", H);
  if (T == 0) return ok();
  REQ_PTR(o, "o");
  REQ_PTR(token_row, "token_row");
  REQ_PTR(topk_w, "topk_w");
  REQ_PTR(y, "y");
  REQ_AL(o, "o");
  REQ_AL(y, "y");
  TRY(check_pitch(ldo, H, 2, "ldo"));
  TRY(check_pitch(ldy, H, 2, "ldy"));
  if (s_out) {
    REQ_AL(s_out, "s_out");
    TRY(check_pitch(lds, H, 2, "lds"));
  }
  return hip_status(launch_combine(o, ldo, token_row, topk_w, s_out, lds, s_out ? T_s : 0, T, K, H, y, ldy, stream),
                    "combine launch");
}

// ---------------------------------------------------------------------------
// Whole layer.
// ---------------------------------------------------------------------------
namespace {
enum { W_OFFSETS, W_ROW_TOKEN, W_ROW_SLOT, W_TOKEN_ROW, W_XQ, W_XS, W_H, W_HQ, W_HS, W_O, W_S, W_PERM, W_GEMM,
       W_SHARED, W_RSPLIT, W_RPART, W_COUNT };

struct FwdLayout {
  int64_t off[W_COUNT];
  int64_t total;
};

// The shared expert joins the routed GEMM launches as one extra group when its
// width equals the routed width; its rows then follow the T*K routed rows in h and o.
bool fuse_shared(const dmoe_layer_desc* d) { return d->T_s > 0 && d->F_s > 0 && d->F_s == d->F; }

// Many tokens: the router runs as a tiled GEMM over W_r split once into BF16 parts.
bool router_tiled(const dmoe_layer_desc* d) { return !d->logits_given && d->T > 256; }

// Few tokens: the router's K ranges run as separate workgroups and leave
// partial planes that the route launch adds; 1 = logits written directly.
int router_planes(const dmoe_layer_desc* d) {
  return (d->logits_given || router_tiled(d)) ? 1 : router_nparts(d->T, d->H);
}

FwdLayout fwd_layout(const dmoe_layer_desc* d) {
  FwdLayout L;
  const bool fp8 = d->dtype == DMOE_FP8_E4M3;
  const bool shared = d->T_s > 0 && d->F_s > 0;
  const bool fused = fuse_shared(d);
  const int64_t mcap = (int64_t)d->T * d->K;
  const int64_t rows = mcap + (fused ? d->T_s : 0);
  const int64_t fpad = round_up(d->F, 128);
  const int64_t sizes[W_COUNT] = {
      (int64_t)(d->E_loc + 1) * 4,
      mcap * 4,
      mcap * 4,
      mcap * 4,
      fp8 ? (int64_t)d->T * d->H : -1,
      fp8 ? (int64_t)d->T * (d->H / 128) * 4 : -1,
      rows * fpad * 2,
      fp8 ? rows * fpad : -1,
      fp8 ? rows * ceil_div(d->F, 128) * 4 : -1,
      rows * d->H * 2,
      (shared && !fused) ? (int64_t)d->T_s * d->H * 2 : -1,
      (int64_t)permute_ws_bytes(d->T, d->K, d->E_loc),
      (int64_t)gemm_ws_bytes((int)mcap, d->E_loc, fused ? d->T_s : 0),
      (shared && !fused) ? shared_layout(d->dtype, d->T_s, d->H, d->F_s).total : -1,
      router_tiled(d) ? (int64_t)router_split_bytes(d->E, d->H) : -1,
      router_planes(d) > 1 ? (int64_t)router_planes(d) * d->T * d->E * 4 : -1,
  };
  int64_t at = 0;
  for (int i = 0; i < W_COUNT; ++i) {
    if (sizes[i] < 0) {
      L.off[i] = -1;
      continue;
    }
    L.off[i] = at;
    at += round_up(std::max<int64_t>(sizes[i], 1), 256);
  }
  if (fused) L.off[W_S] = L.off[W_O] + mcap * d->H * 2;  // shared rows of o
  L.total = at;
  return L;
}

dmoe_status check_desc(const dmoe_layer_desc* d) {
  REQ(d != nullptr, DMOE_ERR_INVALID_ARG, "desc is NULL");
  TRY(check_dtype(d->dtype));
  REQ(d->T >= 0, DMOE_ERR_INVALID_ARG, "T < 0");
  REQ(d->H > 0 && d->H % 128 == 0, DMOE_ERR_INVALID_ARG, "H = %d must be a positive multiple of 128", d->H);
  REQ(d->F > 0 && d->F % 8 == 0, DMOE_ERR_INVALID_ARG, "F = %d must be a positive multiple of 8", d->F);
  REQ(d->F_s >= 0 && d->F_s % 8 == 0, DMOE_ERR_INVALID_ARG, "F_s = %d must be a multiple of 8", d->F_s);
  REQ(d->E >= 1 && d->E <= 1024, DMOE_ERR_INVALID_ARG, "E = %d outside [1, 1024]", d->E);
  REQ(d->K >= 1 && d->K <= d->E && d->K <= 64, DMOE_ERR_INVALID_ARG, "K = %d outside [1, min(E, 64)]", d->K);
  REQ(d->E_loc >= 1 && d->e0 >= 0 && d->e0 + d->E_loc <= d->E, DMOE_ERR_INVALID_ARG,
      "local experts [%d, %d) not inside [0, %d)", d->e0, d->e0 + d->E_loc, d->E);
  REQ(d->T_s >= 0 && d->T_s <= d->T, DMOE_ERR_INVALID_ARG, "T_s = %d outside [0, T]", d->T_s);
  REQ(d->dtype != DMOE_FP8_E4M3 || (d->H <= 16384 && d->F <= 16384 && d->F_s <= 16384), DMOE_ERR_UNSUPPORTED,
      "FP8 layers support H, F, F_s up to 16384");
  REQ((int64_t)d->T * d->K <= INT32_MAX / 2, DMOE_ERR_INVALID_ARG, "T*K too large");
  TRY(check_route_opts(d->E, d->K, d->n_group, d->topk_group,
                       d->routed_scaling_factor == 0.f ? 1.f : d->routed_scaling_factor));
  REQ(d->scoring == DMOE_SCORING_SOFTMAX || d->scoring == DMOE_SCORING_SIGMOID, DMOE_ERR_INVALID_ARG,
      "scoring = %d is not DMOE_SCORING_SOFTMAX or DMOE_SCORING_SIGMOID", d->scoring);
  return DMOE_OK;
}
}  // namespace

size_t dmoe_forward_ws_bytes(const dmoe_layer_desc* desc) {
  if (check_desc(desc) != DMOE_OK) return 0;
  return (size_t)fwd_layout(desc).total;
}

const char* dmoe_forward_gateup_kernel(const dmoe_layer_desc* desc) {
  if (check_desc(desc) != DMOE_OK) return nullptr;
  const int mcap = desc->T * desc->K;
  return gemm_gateup_kernel_name(desc->dtype, mcap, desc->E_loc, fuse_shared(desc) ? desc->T_s : 0, desc->F);
}

const char* dmoe_forward_down_kernel(const dmoe_layer_desc* desc) {
  if (check_desc(desc) != DMOE_OK) return nullptr;
  const int mcap = desc->T * desc->K;
  return gemm_down_kernel_name(desc->dtype, mcap, desc->E_loc, fuse_shared(desc) ? desc->T_s : 0, desc->H);
}

int64_t dmoe_forward_ws_offset(const dmoe_layer_desc* desc, int32_t which) {
  if (check_desc(desc) != DMOE_OK || which < 0 || which > W_S) return -1;
  return fwd_layout(desc).off[which];
}

static dmoe_status forward_impl(const dmoe_layer_desc* d, const dmoe_layer_ptrs* p, void* ws, size_t ws_bytes,
                                hipStream_t stream, hipEvent_t* ev) {
  TRY(check_desc(d));
  REQ(p != nullptr, DMOE_ERR_INVALID_ARG, "ptrs is NULL");
  if (d->T == 0) return ok();
  const bool fp8 = d->dtype == DMOE_FP8_E4M3;
  const bool shared = d->T_s > 0 && d->F_s > 0;
  const int es = dtype_size(d->dtype);
  const int64_t fpad = round_up(d->F, 128);
  REQ_PTR(p->x, "x");
  REQ_AL(p->x, "x");
  TRY(check_pitch(p->ldx, d->H, 2, "ldx"));
  REQ_PTR(p->logits, "logits");
  if (!d->logits_given) {
    REQ_PTR(p->w_router, "w_router");
    REQ_AL(p->w_router, "w_router");
  }
  REQ(p->w_gate && p->w_up && p->w_down, DMOE_ERR_INVALID_ARG, "routed expert weights are NULL");
  REQ(aligned16(p->w_gate) && aligned16(p->w_up) && aligned16(p->w_down), DMOE_ERR_ALIGNMENT,
      "routed expert weights are not 16-byte aligned");
  TRY(check_pitch(p->ldw_gu, d->H, es, "ldw_gu"));
  TRY(check_pitch(p->ldw_d, fpad, es, "ldw_d"));
  if (fp8) REQ(p->ws_gate && p->ws_up && p->ws_down, DMOE_ERR_INVALID_ARG, "routed expert scales are NULL");
  if (shared) {
    REQ(p->sw_gate && p->sw_up && p->sw_down, DMOE_ERR_INVALID_ARG, "shared expert weights are NULL");
    REQ(aligned16(p->sw_gate) && aligned16(p->sw_up) && aligned16(p->sw_down), DMOE_ERR_ALIGNMENT,
        "shared expert weights are not 16-byte aligned");
    TRY(check_pitch(p->ldsw_gu, d->H, es, "ldsw_gu"));
    TRY(check_pitch(p->ldsw_d, round_up(d->F_s, 128), es, "ldsw_d"));
    if (fp8) REQ(p->sws_gate && p->sws_up && p->sws_down, DMOE_ERR_INVALID_ARG, "shared expert scales are NULL");
  }
  REQ(p->topk_ids && p->topk_w, DMOE_ERR_INVALID_ARG, "topk outputs are NULL");
  REQ_PTR(p->y, "y");
  REQ_AL(p->y, "y");
  TRY(check_pitch(p->ldy, d->H, 2, "ldy"));
  {
    // every GEMM operand within 4 GiB of its base (32-bit offsets in the tile GEMM)
    const int64_t rows = (int64_t)d->T * d->K + d->T_s;
    const int64_t fspad = round_up(d->F_s, 128);
    REQ(span_fits(d->T, fp8 ? d->H : p->ldx, fp8 ? 1 : 2) && (!router_tiled(d) || span_fits(d->T, p->ldx, 2)) &&
            span_fits(rows, fpad, 2) &&
            span_fits(fpad, p->ldw_gu, es) && span_fits(d->H, p->ldw_d, es) &&
            (!shared || (span_fits(fspad, p->ldsw_gu, es) && span_fits(d->H, p->ldsw_d, es))),
        DMOE_ERR_UNSUPPORTED, "an operand spans 4 GiB or more");
  }
  const FwdLayout L = fwd_layout(d);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= (size_t)L.total, DMOE_ERR_WORKSPACE,
      "forward workspace needs %lld bytes, got %zu", (long long)L.total, ws_bytes);

  uint8_t* w8 = static_cast<uint8_t*>(ws);
  auto at = [&](int i) { return w8 + L.off[i]; };
  int32_t* offsets = reinterpret_cast<int32_t*>(at(W_OFFSETS));
  int32_t* row_token = reinterpret_cast<int32_t*>(at(W_ROW_TOKEN));
  int32_t* row_slot = reinterpret_cast<int32_t*>(at(W_ROW_SLOT));
  int32_t* token_row = reinterpret_cast<int32_t*>(at(W_TOKEN_ROW));
  uint16_t* h = reinterpret_cast<uint16_t*>(at(W_H));
  uint16_t* o = reinterpret_cast<uint16_t*>(at(W_O));
  const int mcap = d->T * d->K;
  hipError_t e = hipSuccess;
  int stage = 0;
  // Marks the end of a stage (and the start of the next) when the caller asked for events.
  auto mark = [&]() -> hipError_t {
    const int i = stage++;
    return (ev && ev[i]) ? hipEventRecord(ev[i], stream) : hipSuccess;
  };
#define STEP(call, what)                               \
  do {                                                 \
    e = (call);                                        \
    if (e != hipSuccess) return hip_status(e, what);   \
  } while (0)

  STEP(mark(), "event");
  const int planes = router_planes(d);
  float* rpart = planes > 1 ? reinterpret_cast<float*>(at(W_RPART)) : nullptr;
  if (!d->logits_given) {
    if (router_tiled(d))
      STEP(launch_router_logits_split(p->x, p->ldx, p->w_router, d->T, d->H, d->E,
                                      reinterpret_cast<uint16_t*>(at(W_RSPLIT)), p->logits, stream),
           "router_logits");
    else if (planes > 1)
      STEP(launch_router_logits_parts(p->x, p->ldx, p->w_router, d->T, d->H, d->E, rpart, stream), "router_logits");
    else
      STEP(launch_router_logits(p->x, p->ldx, p->w_router, d->T, d->H, d->E, p->logits, stream), "router_logits");
  }
  STEP(mark(), "event");
  {
    const int g = d->n_group <= 1 ? 1 : d->n_group;
    const int tg = d->topk_group <= 0 ? g : d->topk_group;
    const float sc = d->routed_scaling_factor == 0.f ? 1.f : d->routed_scaling_factor;
    // partial planes: the route launch adds them and stores the logits
    const LogitSrc src = planes > 1 ? LogitSrc{rpart, planes, (int64_t)d->T * d->E, p->logits}
                                    : LogitSrc{p->logits, 1, 0, nullptr};
    if (d->scoring == DMOE_SCORING_SIGMOID)
      STEP(launch_route_sigmoid(src, p->score_bias, d->T, d->E, d->K, g, tg, d->no_renormalize == 0, sc,
                                p->topk_ids, p->topk_w, stream),
           "route");
    else
      STEP(launch_route(src, d->T, d->E, d->K, g, tg, d->no_renormalize == 0, sc, p->topk_ids, p->topk_w, stream),
           "route");
  }
  STEP(mark(), "event");
  STEP(launch_permute(p->topk_ids, d->T, d->K, d->e0, d->E_loc, offsets, row_token, row_slot, token_row,
                      at(W_PERM), stream),
       "permute");
  const bool fused = fuse_shared(d);
  const int xrows = fused ? d->T_s : 0;
  if (!gemm_uses_stream(mcap, d->E_loc))
    STEP(launch_schedule(offsets, d->E_loc, mcap, xrows, mcap, at(W_GEMM), stream), "schedule");
  STEP(mark(), "event");

  const void* a = p->x;
  int64_t lda = p->ldx;
  const float* a_scales = nullptr;
  int64_t ldas = 0;
  if (fp8) {
    uint8_t* xq = at(W_XQ);
    float* xs = reinterpret_cast<float*>(at(W_XS));
    STEP(launch_quant_act(p->x, d->T, d->H, p->ldx, xq, d->H, xs, d->H / 128, stream), "quant x");
    a = xq;
    lda = d->H;
    a_scales = xs;
    ldas = d->H / 128;
  }
  STEP(mark(), "event");
  GemmArgs g1{d->dtype, a, lda, a_scales, ldas, row_token, offsets, d->E_loc, mcap, p->w_gate, p->w_up,
              p->ldw_gu, p->ws_gate, p->ws_up, d->H, d->F, h, fpad, at(W_GEMM), true};
  if (fused) {
    g1.x_rows = xrows;
    g1.x_row0 = mcap;
    g1.x_a_base = mcap;  // shared row mcap + t reads token t
    g1.xw0 = p->sw_gate;
    g1.xw1 = p->sw_up;
    g1.xws0 = p->sws_gate;
    g1.xws1 = p->sws_up;
  }
  // FP8 with the wide tile kernel: h is quantised in the gate/up epilogue
  const bool fused_quant = fp8 && gemm_fuses_h_quant(mcap, d->E_loc, xrows, d->F);
  if (fused_quant) {
    g1.out_q = at(W_HQ);
    g1.out_s = reinterpret_cast<float*>(at(W_HS));
    g1.ld_s = ceil_div(d->F, 128);
  }
  STEP(launch_gemm_gateup(g1, stream), "gateup");
  STEP(mark(), "event");

  const void* ha = h;
  const float* hsc = nullptr;
  int64_t ldhs = 0;
  if (fp8) {
    uint8_t* hq = at(W_HQ);
    float* hs = reinterpret_cast<float*>(at(W_HS));
    ldhs = ceil_div(d->F, 128);
    // rows [M, T*K) were never written by gate/up: skipped (M read on the device)
    if (!fused_quant)
      STEP(launch_quant_act(h, mcap + xrows, d->F, fpad, hq, fpad, hs, ldhs, stream, offsets + d->E_loc, mcap),
           "quant h");
    ha = hq;
    hsc = hs;
  }
  STEP(mark(), "event");
  GemmArgs g2{d->dtype, ha, fpad, hsc, ldhs, nullptr, offsets, d->E_loc, mcap, p->w_down, nullptr, p->ldw_d,
              p->ws_down, nullptr, d->F, d->H, o, d->H, at(W_GEMM), true};
  if (fused) {
    g2.x_rows = xrows;
    g2.x_row0 = mcap;
    g2.x_a_base = 0;  // h rows are already in the unified row space
    g2.xw0 = p->sw_down;
    g2.xws0 = p->sws_down;
  }
  STEP(launch_gemm_down(g2, stream), "down");
  STEP(mark(), "event");

  const uint16_t* s_out = fused ? o + (int64_t)mcap * d->H : nullptr;
  if (shared && !fused) {
    uint16_t* s = reinterpret_cast<uint16_t*>(at(W_S));
    TRY(run_shared(d->dtype, a, lda, a_scales, ldas, d->T_s, p->sw_gate, p->sw_up, p->sw_down, p->ldsw_gu,
                   p->ldsw_d, p->sws_gate, p->sws_up, p->sws_down, d->H, d->F_s, s, d->H, at(W_SHARED), stream));
    s_out = s;
  }
  STEP(mark(), "event");
  STEP(launch_combine(o, d->H, token_row, p->topk_w, s_out, d->H, shared ? d->T_s : 0, d->T, d->K, d->H, p->y,
                      p->ldy, stream),
       "combine");
  STEP(mark(), "event");
#undef STEP
  return ok();
}

dmoe_status dmoe_forward(const dmoe_layer_desc* d, const dmoe_layer_ptrs* p, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  return forward_impl(d, p, ws, ws_bytes, stream, nullptr);
}

dmoe_status dmoe_forward_timed(const dmoe_layer_desc* d, const dmoe_layer_ptrs* p, void* ws, size_t ws_bytes,
                               hipStream_t stream, hipEvent_t* stage_events) {
  return forward_impl(d, p, ws, ws_bytes, stream, stage_events);
}

}  // extern "C"
