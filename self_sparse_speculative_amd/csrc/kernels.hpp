// Internal launcher declarations shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace s3r {

// bfloat16 element that converts to float (generic kernels).
struct BF16Val {
  uint16_t bits;
  __device__ __forceinline__ operator float() const { return __uint_as_float((uint32_t)bits << 16); }
};

constexpr int kDecChunk = 256;         // attended positions per draft split (vector path)
#ifndef S3R_DRAFT_CHUNK
#define S3R_DRAFT_CHUNK 2048
#endif
constexpr int kDecChunkMfma = S3R_DRAFT_CHUNK;  // most attended positions per draft split (bf16 x 128 MFMA path)
#ifndef S3R_DRAFT_WAVES
#define S3R_DRAFT_WAVES 4
#endif
// Waves per draft workgroup (bf16 x 128 MFMA path). With 4, three workgroups
// share a CU (VGPRs and LDS), so the 1024 (sequence, KV head) pairs of a
// 128-sequence batch run in one and a third rounds; 2 or 1 waves (every pair
// resident at once, fewer waves per CU) measured the same at 24K and 4 % /
// 20 % slower on mixed lengths (4K-24K).
constexpr int kDecMfmaWaves = S3R_DRAFT_WAVES;
#ifndef S3R_DRAFT_BALANCE
#define S3R_DRAFT_BALANCE 1
#endif
constexpr bool kDecBalance = S3R_DRAFT_BALANCE != 0;  // equal-size draft splits
#ifndef S3R_VERIFY_CHUNK
#define S3R_VERIFY_CHUNK 4096
#endif
constexpr int kVerChunkMfma = S3R_VERIFY_CHUNK;  // most context positions per verify split (bf16 x 128 path)
#ifndef S3R_VERIFY_BALANCE
#define S3R_VERIFY_BALANCE 1
#endif
constexpr bool kVerBalance = S3R_VERIFY_BALANCE != 0;  // equal-size verify splits per sequence
#ifndef S3R_VERIFY_Q_LDS
#define S3R_VERIFY_Q_LDS 1
#endif
// Verify query fragments read from LDS each subtile instead of held in
// registers, for three row tiles (33-48 rows): the freed VGPRs let two
// workgroups share a CU instead of one (36 rows at 24K: 3.90 -> 3.64 ms).
// At two row tiles the same change spills and is slower (3.39 -> 3.48 ms).
constexpr bool kVerQLds = S3R_VERIFY_Q_LDS != 0;
#ifndef S3R_VERIFY_EARLY_LOADS
#define S3R_VERIFY_EARLY_LOADS 1
#endif
// Verify: a wave issues its next subtile's K loads right after its S MFMAs and
// its V loads right after the V transpose, instead of both at the end.
constexpr bool kVerEarlyLoads = S3R_VERIFY_EARLY_LOADS != 0;
#ifndef S3R_VERIFY_SPLIT_EDGE
#define S3R_VERIFY_SPLIT_EDGE 1
#endif
// Verify: separate code for the subtiles that need the causal mask and those
// that do not (0: one masked form for all).
constexpr bool kVerSplitEdge = S3R_VERIFY_SPLIT_EDGE != 0;
#ifndef S3R_VERIFY_PAGE_BURST
#define S3R_VERIFY_PAGE_BURST 1
#endif
// Verify, page scores, up to two row tiles: a split's page records gathered in
// LDS and written in one burst at its end.
constexpr bool kVerPageBurst = S3R_VERIFY_PAGE_BURST != 0;
#ifndef S3R_VERIFY_POS_BURST
#define S3R_VERIFY_POS_BURST 1
#endif
// Verify, position scores, up to two row tiles: the partials of each group of
// 16 subtiles gathered in LDS and written as one run.
constexpr bool kVerPosBurst = S3R_VERIFY_POS_BURST != 0;

#ifndef S3R_SELECT_SAMPLED
#define S3R_SELECT_SAMPLED 1
#endif
constexpr bool kSelSampled = S3R_SELECT_SAMPLED != 0;  // sampled-threshold path for long rows
constexpr int kVerChunkGeneric = 256;  // context positions per verify split (generic path)
constexpr int kSmpChunks = 64;         // vocabulary chunks of the final draw

hipError_t launch_select(const float* scores, int stride, const int* ctx_len, int B, int Hkv,
                         int max_ctx_len, int s_num, int s_den, int window, int* idx, int nsel_cap,
                         int* n_sel, int* order, hipStream_t stream);

bool decode_supported(int dtype, int D, int G);
size_t decode_workspace_bytes(int B, int Hq, int D, int max_attend);
hipError_t launch_sparse_decode(int dtype, int D, int G, const void* q, const void* kp,
                                const void* vp, const int* bt, int max_pages, int Hkv,
                                const int* idx, int nsel_cap, const int* n_sel, const int* sel_len,
                                const int* cur_len, const int* order, int B, float scale, int max_attend,
                                float* out, float* lse, void* ws, hipStream_t stream);
hipError_t launch_length_order(const int* len, int B, int* order, hipStream_t stream);

struct VerifyPlan {
  int G, R, NT, RP, chunk, nsplit, ntile_cap;
  bool mfma, pages;
  size_t off_part_o, off_part_ml, off_sc_max, off_sc_val, off_tmp, bytes;
};
// pages: the workspace of the page-score form (s3r_verify_attn_pages).
VerifyPlan verify_plan(int B, int k, int Hq, int Hkv, int D, int dtype, int max_seq_len, bool pages);
// Split pass + merge of the output rows. With scores != nullptr the scores
// are written too (pages: one per page of 16 positions); with defer_scores
// the position-score partials stay in ws for a later launch_verify_scores
// (scores must then be nullptr and pages false).
hipError_t launch_verify(int dtype, int D, const void* q, const void* kp, const void* vp,
                         const int* bt, int max_pages, int Hkv, const int* seq_len, int B, int k,
                         int Hq, float scale, int max_seq_len, float* out, float* lse,
                         float* scores, int score_stride, bool pages, bool defer_scores, void* ws,
                         hipStream_t stream);
hipError_t launch_verify_scores(int dtype, int D, const int* seq_len, int B, int k, int Hq, int Hkv,
                                int max_seq_len, float* scores, int score_stride, const void* ws,
                                hipStream_t stream);

size_t sample_workspace_bytes(int B, int k, int V);
// Device address, on the device that runs `stream`, of the sampling step's
// library-owned scratch (kSampleScratchBytes per GPU); looked up once per device.
constexpr size_t kSampleScratchBytes = (size_t)8 << 20;
hipError_t sample_scratch(hipStream_t stream, void** ptr);
hipError_t launch_spec_sample(const float* zt, const float* zd, const int* dtok, const float* u,
                              int B, int k, int V, float temperature, int* tokens, int* n_out,
                              int8_t* accepted, void* ws, hipStream_t stream);

struct GroupedSelectPlan {
  int G, kstride, cap_u;
  size_t off_keys, off_units, off_top, off_wc, off_sel, off_nsel, bytes;
};
GroupedSelectPlan grouped_select_plan(int B, int Hkv, int max_ctx_len, int s_num, int s_den, int window,
                                      int unit, int all_heads);
int grouped_select_capacity(int max_ctx_len, int s_num, int s_den, int window, int unit);
// Whole-page selection from scores given per page (stride >= max_ctx_len / 16).
// order (nullable): the draft steps' dispatch order, written by the last kernel.
hipError_t launch_select_pages(const float* page_scores, int stride, const int* ctx_len, int B, int Hkv,
                               int max_ctx_len, int s_num, int s_den, int window, int all_heads, int* idx,
                               int nsel_cap, int* n_sel, int* order, void* ws, hipStream_t stream);
hipError_t launch_select_grouped(const float* scores, int stride, const int* ctx_len, int B, int Hkv,
                                 int max_ctx_len, int s_num, int s_den, int window, int unit, int all_heads,
                                 int* idx, int nsel_cap, int* n_sel, int* order, void* ws, hipStream_t stream);

// Measurement: the read patterns of the verification and of a draft step.
size_t read_verify_pattern_words(int B, int Hkv, int max_seq_len);
size_t read_draft_pattern_words(int B, int Hkv, int max_attend);
hipError_t launch_read_verify_pattern(const void* kp, const void* vp, const int* bt, int max_pages, int Hkv,
                                      const int* seq_len, int B, int max_seq_len, uint32_t* sink,
                                      hipStream_t stream);
hipError_t launch_read_draft_pattern(const void* kp, const void* vp, const int* bt, int max_pages, int Hkv,
                                     const int* idx, int nsel_cap, const int* n_sel, const int* sel_len,
                                     const int* cur_len, int B, int max_attend, uint32_t* sink,
                                     hipStream_t stream);

hipError_t launch_kv_append(const void* k_rows, const void* v_rows, void* k_pages, void* v_pages,
                            const int* bt, int max_pages, const int* pos, int B, int n, int Hkv,
                            int row_bytes, hipStream_t stream);
hipError_t launch_commit(const int* n_out, const int* tokens, int B, int k, int* ctx_len, int* pending,
                         int* cur_len, int* seq_len, long long* verified, hipStream_t stream);

}  // namespace s3r
