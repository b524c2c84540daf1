// C ABI of the S3R library: argument validation, workspace sizing and
// dispatch to the kernels. Every entry point validates all host-side
// arguments before enqueuing anything and returns a status code.

#include <math.h>

#include "../../include/s3r.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxK = 15;
constexpr int kMaxRows = 64;

bool kv_ok(const s3r_paged_kv* kv) {
  return kv != nullptr && kv->k_pages != nullptr && kv->v_pages != nullptr &&
         kv->block_table != nullptr && kv->num_pages >= 1 && kv->max_pages_per_seq >= 1 &&
         kv->num_kv_heads >= 1 && kv->head_dim >= 1 && kv->page_size >= 1 &&
         (kv->dtype == S3R_F32 || kv->dtype == S3R_BF16);
}

s3r_status kv_supported(const s3r_paged_kv* kv) {
  if (kv->page_size != 16) return S3R_ERR_UNSUPPORTED;
  if (kv->head_dim != 64 && kv->head_dim != 128) return S3R_ERR_UNSUPPORTED;
  return S3R_OK;
}

s3r_status from_hip(hipError_t e) { return e == hipSuccess ? S3R_OK : S3R_ERR_HIP; }

long long budget_ll(long long L, long long s_num, long long s_den, long long window) {
  const long long newest = window < L ? window : L;
  const long long frac = (s_num * L + s_den - 1) / s_den;
  long long n = newest > frac ? newest : frac;
  return n < L ? n : L;
}

}  // namespace

extern "C" {

const char* s3r_status_string(s3r_status status) {
  switch (status) {
    case S3R_OK: return "S3R_OK";
    case S3R_ERR_INVALID_ARG: return "S3R_ERR_INVALID_ARG: invalid argument";
    case S3R_ERR_UNSUPPORTED: return "S3R_ERR_UNSUPPORTED: shape or dtype without a kernel";
    case S3R_ERR_WORKSPACE: return "S3R_ERR_WORKSPACE: workspace too small";
    case S3R_ERR_HIP: return "S3R_ERR_HIP: kernel launch failed";
  }
  return "S3R: unknown status";
}

int32_t s3r_version(void) { return 200; }

int32_t s3r_budget(int32_t L, int32_t s_num, int32_t s_den, int32_t window) {
  if (L < 0 || s_den <= 0 || s_num < 0 || s_num > s_den || window < 0) return -1;
  return (int32_t)budget_ll(L, s_num, s_den, window);
}

s3r_status s3r_select(const float* scores, int32_t score_stride, const int32_t* ctx_len, int32_t B,
                      int32_t Hkv, int32_t max_ctx_len, int32_t s_num, int32_t s_den,
                      int32_t window, int32_t* idx, int32_t nsel_cap, int32_t* n_sel, int32_t* order,
                      hipStream_t stream) {
  if (!scores || !ctx_len || !idx || !n_sel) return S3R_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || max_ctx_len < 1 || B > 65535 || Hkv > 65535) return S3R_ERR_INVALID_ARG;
  if (s_den <= 0 || s_num < 0 || s_num > s_den || window < 0) return S3R_ERR_INVALID_ARG;
  if (score_stride < max_ctx_len) return S3R_ERR_INVALID_ARG;
  if (nsel_cap < 1 || nsel_cap < budget_ll(max_ctx_len, s_num, s_den, window)) return S3R_ERR_INVALID_ARG;
  return from_hip(s3r::launch_select(scores, score_stride, ctx_len, B, Hkv, max_ctx_len, s_num,
                                     s_den, window, idx, nsel_cap, n_sel, order, stream));
}

int32_t s3r_select_grouped_capacity(int32_t max_ctx_len, int32_t s_num, int32_t s_den, int32_t window,
                                    int32_t unit) {
  if (max_ctx_len < 1 || s_den <= 0 || s_num < 0 || s_num > s_den || window < 0) return -1;
  if (unit != 1 && unit != 16) return -1;
  return s3r::grouped_select_capacity(max_ctx_len, s_num, s_den, window, unit);
}

size_t s3r_select_grouped_workspace_bytes(int32_t B, int32_t Hkv, int32_t max_ctx_len, int32_t s_num,
                                          int32_t s_den, int32_t window, int32_t unit, int32_t all_heads) {
  if (B < 1 || Hkv < 1 || max_ctx_len < 1 || s_den <= 0 || s_num < 0 || s_num > s_den || window < 0) return 0;
  if (unit != 1 && unit != 16) return 0;
  if (unit == 1 && !all_heads) return 0;  // the plain selection needs none
  return s3r::grouped_select_plan(B, Hkv, max_ctx_len, s_num, s_den, window, unit, all_heads ? 1 : 0).bytes;
}

s3r_status s3r_select_grouped(const float* scores, int32_t score_stride, const int32_t* ctx_len, int32_t B,
                              int32_t Hkv, int32_t max_ctx_len, int32_t s_num, int32_t s_den, int32_t window,
                              int32_t unit, int32_t all_heads, int32_t* idx, int32_t nsel_cap, int32_t* n_sel,
                              int32_t* order, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!scores || !ctx_len || !idx || !n_sel) return S3R_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || max_ctx_len < 1 || B > 65535 || Hkv > 65535) return S3R_ERR_INVALID_ARG;
  if (s_den <= 0 || s_num < 0 || s_num > s_den || window < 0) return S3R_ERR_INVALID_ARG;
  if (unit != 1 && unit != 16) return S3R_ERR_INVALID_ARG;
  if (score_stride < max_ctx_len) return S3R_ERR_INVALID_ARG;
  if (nsel_cap < 1 || nsel_cap < s3r::grouped_select_capacity(max_ctx_len, s_num, s_den, window, unit))
    return S3R_ERR_INVALID_ARG;
  if (unit == 1 && !all_heads)
    return from_hip(s3r::launch_select(scores, score_stride, ctx_len, B, Hkv, max_ctx_len, s_num, s_den,
                                       window, idx, nsel_cap, n_sel, order, stream));
  const size_t need = s3r::grouped_select_plan(B, Hkv, max_ctx_len, s_num, s_den, window, unit,
                                               all_heads ? 1 : 0).bytes;
  if (ws_bytes < need || ws == nullptr) return S3R_ERR_WORKSPACE;
  return from_hip(s3r::launch_select_grouped(scores, score_stride, ctx_len, B, Hkv, max_ctx_len, s_num, s_den,
                                             window, unit, all_heads ? 1 : 0, idx, nsel_cap, n_sel, order, ws,
                                             stream));
}

s3r_status s3r_select_pages(const float* page_scores, int32_t page_stride, const int32_t* ctx_len, int32_t B,
                            int32_t Hkv, int32_t max_ctx_len, int32_t s_num, int32_t s_den, int32_t window,
                            int32_t all_heads, int32_t* idx, int32_t nsel_cap, int32_t* n_sel, int32_t* order,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!page_scores || !ctx_len || !idx || !n_sel) return S3R_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || max_ctx_len < 1 || B > 65535 || Hkv > 65535) return S3R_ERR_INVALID_ARG;
  if (s_den <= 0 || s_num < 0 || s_num > s_den || window < 0) return S3R_ERR_INVALID_ARG;
  if (page_stride < (max_ctx_len + 15) / 16) return S3R_ERR_INVALID_ARG;
  if (nsel_cap < 1 || nsel_cap < s3r::grouped_select_capacity(max_ctx_len, s_num, s_den, window, 16))
    return S3R_ERR_INVALID_ARG;
  const size_t need = s3r::grouped_select_plan(B, Hkv, max_ctx_len, s_num, s_den, window, 16,
                                               all_heads ? 1 : 0).bytes;
  if (ws_bytes < need || ws == nullptr) return S3R_ERR_WORKSPACE;
  return from_hip(s3r::launch_select_pages(page_scores, page_stride, ctx_len, B, Hkv, max_ctx_len, s_num, s_den,
                                           window, all_heads ? 1 : 0, idx, nsel_cap, n_sel, order, ws, stream));
}

size_t s3r_sparse_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim, int32_t max_attend) {
  if (B < 1 || Hq < 1 || head_dim < 1 || max_attend < 1) return 0;
  return s3r::decode_workspace_bytes(B, Hq, head_dim, max_attend);
}

s3r_status s3r_length_order(const int32_t* len, int32_t B, int32_t* order, hipStream_t stream) {
  if (!len || !order || B < 1 || B > 65535) return S3R_ERR_INVALID_ARG;
  return from_hip(s3r::launch_length_order(len, B, order, stream));
}

s3r_status s3r_sparse_decode_attn(const void* q, const s3r_paged_kv* kv, const int32_t* idx,
                                  int32_t nsel_cap, const int32_t* n_sel, const int32_t* sel_len,
                                  const int32_t* cur_len, const int32_t* order, int32_t B, int32_t Hq,
                                  float scale, int32_t max_attend, float* out, float* lse, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (!q || !kv_ok(kv) || !idx || !n_sel || !sel_len || !cur_len || !out) return S3R_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || nsel_cap < 1 || max_attend < 1 || B > 65535) return S3R_ERR_INVALID_ARG;
  if (!isfinite(scale)) return S3R_ERR_INVALID_ARG;
  const int Hkv = kv->num_kv_heads;
  if (Hq % Hkv != 0 || Hkv > 65535) return S3R_ERR_INVALID_ARG;
  s3r_status st = kv_supported(kv);
  if (st != S3R_OK) return st;
  const int G = Hq / Hkv;
  if (!s3r::decode_supported(kv->dtype, kv->head_dim, G)) return S3R_ERR_UNSUPPORTED;
  const size_t need = s3r::decode_workspace_bytes(B, Hq, kv->head_dim, max_attend);
  if (ws_bytes < need || (need > 0 && ws == nullptr)) return S3R_ERR_WORKSPACE;
  return from_hip(s3r::launch_sparse_decode(kv->dtype, kv->head_dim, G, q, kv->k_pages, kv->v_pages,
                                            kv->block_table, kv->max_pages_per_seq, Hkv, idx,
                                            nsel_cap, n_sel, sel_len, cur_len, order, B, scale,
                                            max_attend, out, lse, ws, stream));
}

size_t s3r_verify_workspace_bytes(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                  int32_t dtype, int32_t max_seq_len) {
  if (B < 1 || k < 0 || k > kMaxK || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || head_dim < 1 ||
      max_seq_len < 1)
    return 0;
  return s3r::verify_plan(B, k, Hq, Hkv, head_dim, dtype, max_seq_len, false).bytes;
}

size_t s3r_verify_pages_workspace_bytes(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                        int32_t dtype, int32_t max_seq_len) {
  if (B < 1 || k < 0 || k > kMaxK || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || head_dim < 1 ||
      max_seq_len < 1)
    return 0;
  return s3r::verify_plan(B, k, Hq, Hkv, head_dim, dtype, max_seq_len, true).bytes;
}

// Shared argument checks of the verification entry points (pages: the
// page-score form, whose scores hold one entry per page of 16 positions).
static s3r_status verify_check(const s3r_paged_kv* kv, const int32_t* seq_len, int32_t B, int32_t k,
                               int32_t Hq, int32_t max_seq_len, float* scores, int32_t score_stride,
                               void* ws, size_t ws_bytes, bool pages = false) {
  if (!kv_ok(kv) || !seq_len) return S3R_ERR_INVALID_ARG;
  if (B < 1 || B > 65535 || Hq < 1 || k < 0 || k > kMaxK || max_seq_len < k + 1) return S3R_ERR_INVALID_ARG;
  const int Hkv = kv->num_kv_heads;
  if (Hq % Hkv != 0 || Hkv > 65535) return S3R_ERR_INVALID_ARG;
  if ((long long)kv->max_pages_per_seq * kv->page_size < max_seq_len) return S3R_ERR_INVALID_ARG;
  const int need_stride = pages ? (max_seq_len + 15) / 16 : max_seq_len;
  if (scores != nullptr && score_stride < need_stride) return S3R_ERR_INVALID_ARG;
  s3r_status st = kv_supported(kv);
  if (st != S3R_OK) return st;
  if ((k + 1) * (Hq / Hkv) > kMaxRows) return S3R_ERR_UNSUPPORTED;
  const size_t need = s3r::verify_plan(B, k, Hq, Hkv, kv->head_dim, kv->dtype, max_seq_len, pages).bytes;
  if (ws_bytes < need || ws == nullptr) return S3R_ERR_WORKSPACE;
  return S3R_OK;
}

s3r_status s3r_verify_attn(const void* q, const s3r_paged_kv* kv, const int32_t* seq_len,
                           int32_t B, int32_t k, int32_t Hq, float scale, int32_t max_seq_len,
                           float* out, float* lse, float* scores, int32_t score_stride, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!q || !out || !isfinite(scale)) return S3R_ERR_INVALID_ARG;
  const s3r_status st = verify_check(kv, seq_len, B, k, Hq, max_seq_len, scores, score_stride, ws, ws_bytes);
  if (st != S3R_OK) return st;
  return from_hip(s3r::launch_verify(kv->dtype, kv->head_dim, q, kv->k_pages, kv->v_pages,
                                     kv->block_table, kv->max_pages_per_seq, kv->num_kv_heads, seq_len,
                                     B, k, Hq, scale, max_seq_len, out, lse, scores, score_stride, false,
                                     false, ws, stream));
}

s3r_status s3r_verify_attn_pages(const void* q, const s3r_paged_kv* kv, const int32_t* seq_len, int32_t B,
                                 int32_t k, int32_t Hq, float scale, int32_t max_seq_len, float* out, float* lse,
                                 float* page_scores, int32_t page_stride, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  if (!q || !out || !page_scores || !isfinite(scale)) return S3R_ERR_INVALID_ARG;
  const s3r_status st =
      verify_check(kv, seq_len, B, k, Hq, max_seq_len, page_scores, page_stride, ws, ws_bytes, true);
  if (st != S3R_OK) return st;
  return from_hip(s3r::launch_verify(kv->dtype, kv->head_dim, q, kv->k_pages, kv->v_pages,
                                     kv->block_table, kv->max_pages_per_seq, kv->num_kv_heads, seq_len,
                                     B, k, Hq, scale, max_seq_len, out, lse, page_scores, page_stride, true,
                                     false, ws, stream));
}

s3r_status s3r_verify_attn_deferred(const void* q, const s3r_paged_kv* kv, const int32_t* seq_len,
                                    int32_t B, int32_t k, int32_t Hq, float scale, int32_t max_seq_len,
                                    float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !out || !isfinite(scale)) return S3R_ERR_INVALID_ARG;
  const s3r_status st = verify_check(kv, seq_len, B, k, Hq, max_seq_len, nullptr, 0, ws, ws_bytes);
  if (st != S3R_OK) return st;
  return from_hip(s3r::launch_verify(kv->dtype, kv->head_dim, q, kv->k_pages, kv->v_pages,
                                     kv->block_table, kv->max_pages_per_seq, kv->num_kv_heads, seq_len,
                                     B, k, Hq, scale, max_seq_len, out, lse, nullptr, 0, false, true, ws,
                                     stream));
}

s3r_status s3r_verify_scores(const s3r_paged_kv* kv, const int32_t* seq_len, int32_t B, int32_t k,
                             int32_t Hq, int32_t max_seq_len, float* scores, int32_t score_stride,
                             const void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!scores) return S3R_ERR_INVALID_ARG;
  const s3r_status st = verify_check(kv, seq_len, B, k, Hq, max_seq_len, scores, score_stride,
                                     const_cast<void*>(ws), ws_bytes);
  if (st != S3R_OK) return st;
  return from_hip(s3r::launch_verify_scores(kv->dtype, kv->head_dim, seq_len, B, k, Hq, kv->num_kv_heads,
                                            max_seq_len, scores, score_stride, ws, stream));
}

size_t s3r_spec_sample_workspace_bytes(int32_t B, int32_t k, int32_t V) {
  if (B < 1 || k < 0 || k > kMaxK || V < 1) return 0;
  return s3r::sample_workspace_bytes(B, k, V);
}

s3r_status s3r_spec_sample(const float* target_logits, const float* draft_logits,
                           const int32_t* draft_tokens, const float* uniforms, int32_t B,
                           int32_t k, int32_t V, float temperature, int32_t* tokens,
                           int32_t* n_out, int8_t* accepted, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (!target_logits || !uniforms || !tokens || !n_out) return S3R_ERR_INVALID_ARG;
  if (B < 1 || B > 65535 || V < 1 || k < 0 || k > kMaxK) return S3R_ERR_INVALID_ARG;
  if (k > 0 && (!draft_logits || !draft_tokens)) return S3R_ERR_INVALID_ARG;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return S3R_ERR_INVALID_ARG;
  const size_t need = s3r::sample_workspace_bytes(B, k, V);
  if (ws_bytes < need || ws == nullptr) return S3R_ERR_WORKSPACE;
  return from_hip(s3r::launch_spec_sample(target_logits, draft_logits, draft_tokens, uniforms, B, k,
                                          V, temperature, tokens, n_out, accepted, ws, stream));
}

s3r_status s3r_spec_sample_noalloc(const float* target_logits, const float* draft_logits,
                                   const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t k,
                                   int32_t V, float temperature, int32_t* tokens, int32_t* n_out,
                                   int8_t* accepted, hipStream_t stream) {
  if (!target_logits || !uniforms || !tokens || !n_out) return S3R_ERR_INVALID_ARG;
  if (B < 1 || B > 65535 || V < 1 || k < 0 || k > kMaxK) return S3R_ERR_INVALID_ARG;
  if (k > 0 && (!draft_logits || !draft_tokens)) return S3R_ERR_INVALID_ARG;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return S3R_ERR_INVALID_ARG;
  if (s3r::sample_workspace_bytes(B, k, V) > s3r::kSampleScratchBytes) return S3R_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = s3r::sample_scratch(stream, &ws);
  if (e != hipSuccess) return S3R_ERR_HIP;
  return from_hip(s3r::launch_spec_sample(target_logits, draft_logits, draft_tokens, uniforms, B, k, V,
                                          temperature, tokens, n_out, accepted, ws, stream));
}

size_t s3r_read_pattern_sink_words(int32_t B, int32_t Hkv, int32_t max_len, int32_t draft) {
  if (B < 1 || Hkv < 1 || max_len < 1) return 0;
  return draft ? s3r::read_draft_pattern_words(B, Hkv, max_len) : s3r::read_verify_pattern_words(B, Hkv, max_len);
}

s3r_status s3r_read_verify_pattern(const s3r_paged_kv* kv, const int32_t* seq_len, int32_t B, int32_t max_seq_len,
                                   uint32_t* sink, size_t sink_words, hipStream_t stream) {
  if (!kv_ok(kv) || !seq_len || !sink) return S3R_ERR_INVALID_ARG;
  if (B < 1 || B > 65535 || max_seq_len < 1 || kv->num_kv_heads > 65535) return S3R_ERR_INVALID_ARG;
  if ((long long)kv->max_pages_per_seq * kv->page_size < max_seq_len) return S3R_ERR_INVALID_ARG;
  if (kv->page_size != 16 || kv->head_dim != 128 || kv->dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  if (sink_words < s3r::read_verify_pattern_words(B, kv->num_kv_heads, max_seq_len)) return S3R_ERR_WORKSPACE;
  return from_hip(s3r::launch_read_verify_pattern(kv->k_pages, kv->v_pages, kv->block_table, kv->max_pages_per_seq,
                                                  kv->num_kv_heads, seq_len, B, max_seq_len, sink, stream));
}

s3r_status s3r_read_draft_pattern(const s3r_paged_kv* kv, const int32_t* idx, int32_t nsel_cap,
                                  const int32_t* n_sel, const int32_t* sel_len, const int32_t* cur_len, int32_t B,
                                  int32_t max_attend, uint32_t* sink, size_t sink_words, hipStream_t stream) {
  if (!kv_ok(kv) || !idx || !n_sel || !sel_len || !cur_len || !sink) return S3R_ERR_INVALID_ARG;
  if (B < 1 || B > 65535 || nsel_cap < 1 || max_attend < 1 || kv->num_kv_heads > 65535) return S3R_ERR_INVALID_ARG;
  if (kv->page_size != 16 || kv->head_dim != 128 || kv->dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  if (sink_words < s3r::read_draft_pattern_words(B, kv->num_kv_heads, max_attend)) return S3R_ERR_WORKSPACE;
  return from_hip(s3r::launch_read_draft_pattern(kv->k_pages, kv->v_pages, kv->block_table, kv->max_pages_per_seq,
                                                 kv->num_kv_heads, idx, nsel_cap, n_sel, sel_len, cur_len, B,
                                                 max_attend, sink, stream));
}

s3r_status s3r_kv_append(const void* k_rows, const void* v_rows, const s3r_paged_kv* kv,
                         const int32_t* pos, int32_t B, int32_t n, int32_t max_pos, hipStream_t stream) {
  if (!k_rows || !v_rows || !pos || !kv_ok(kv)) return S3R_ERR_INVALID_ARG;
  if (B < 1 || n < 1 || max_pos < n) return S3R_ERR_INVALID_ARG;
  if ((long long)kv->max_pages_per_seq * kv->page_size < max_pos) return S3R_ERR_INVALID_ARG;
  const s3r_status st = kv_supported(kv);
  if (st != S3R_OK) return st;
  const int row_bytes = kv->head_dim * (kv->dtype == S3R_BF16 ? 2 : 4);
  // The descriptor's pointers are const for the reading calls; this one writes the pages.
  return from_hip(s3r::launch_kv_append(k_rows, v_rows, const_cast<void*>(kv->k_pages),
                                        const_cast<void*>(kv->v_pages), kv->block_table,
                                        kv->max_pages_per_seq, pos, B, n, kv->num_kv_heads, row_bytes,
                                        stream));
}

s3r_status s3r_commit(const int32_t* n_out, const int32_t* tokens, int32_t B, int32_t k, int32_t* ctx_len,
                      int32_t* pending, int32_t* cur_len, int32_t* seq_len, int64_t* verified,
                      hipStream_t stream) {
  if (!n_out || !tokens || !ctx_len) return S3R_ERR_INVALID_ARG;
  if (B < 1 || k < 0 || k > kMaxK) return S3R_ERR_INVALID_ARG;
  return from_hip(s3r::launch_commit(n_out, tokens, B, k, ctx_len, pending, k > 0 ? cur_len : nullptr,
                                     seq_len, reinterpret_cast<long long*>(verified), stream));
}

}  // extern "C"
