// Multi-round kernels: K/V rows appended into the paged cache, and the round
// commit (lengths, pending token, the next round's draft and verify lengths).
//
// [news] "Long-context RL training stops waiting on autoregressive rollouts...",
// Interpretation: verification recomputes the proposed block against the
// complete cache, so the block's rows replace what the draft steps wrote.
// [explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
// mean?", Jargon "Block efficiency (tau)": a round outputs the accepted drafts
// plus one token, which is what the committed length grows by.
//
// kv_append_kernel: one thread per 16 B of a row (a row is one KV head of one
// position: D elements); consecutive threads cover consecutive bytes of a row,
// then the rows of the same position, so each wave writes whole 256 B-512 B
// rows. The copy is byte-exact in any dtype.
//
// commit_kernel: one workgroup; per sequence L' = L + n_out, the last output
// token becomes pending, the next round's draft steps attend up to L' + j and
// its verification covers L' + k + 1 positions. The verified-token total is a
// fixed-order integer reduction.

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

constexpr int kAppendThreads = 256;
constexpr int kCommitThreads = 1024;

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const uint4* __restrict__ k_rows, const uint4* __restrict__ v_rows, uint4* __restrict__ kp,
    uint4* __restrict__ vp, const int* __restrict__ bt, int max_pages, const int* __restrict__ pos,
    int n, int Hkv, int chunks_per_row, long long total) {
  const long long t = (long long)blockIdx.x * kAppendThreads + threadIdx.x;
  if (t >= total) return;
  const int c = (int)(t % chunks_per_row);
  const long long row = t / chunks_per_row;  // ((b * n + r) * Hkv + h)
  const int h = (int)(row % Hkv);
  const long long br = row / Hkv;
  const int r = (int)(br % n), b = (int)(br / n);
  const int p = pos[b] + r;
  if (p < 0 || p >= max_pages * kPage) return;  // outside the sequence's block table
  const int page = bt[(size_t)b * max_pages + p / kPage];
  const size_t dst = (((size_t)page * Hkv + h) * kPage + (p % kPage)) * chunks_per_row + c;
  kp[dst] = k_rows[t];
  vp[dst] = v_rows[t];
}

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(
    const int* __restrict__ n_out, const int* __restrict__ tokens, int B, int k, int* __restrict__ ctx_len,
    int* __restrict__ pending, int* __restrict__ cur_len, int* __restrict__ seq_len,
    long long* __restrict__ verified) {
  __shared__ long long part[kCommitThreads / kWave];
  const int tid = threadIdx.x;
  long long sum = 0;
  for (int b = tid; b < B; b += kCommitThreads) {
    const int n = n_out[b];
    if (n < 1 || n > k + 1) continue;  // not a round's output: the sequence is left as it is
    const int L1 = ctx_len[b] + n;
    ctx_len[b] = L1;
    if (pending != nullptr) pending[b] = tokens[(size_t)b * (k + 1) + n - 1];
    if (cur_len != nullptr)
      for (int j = 1; j <= k; ++j) cur_len[(size_t)(j - 1) * B + b] = L1 + j;
    if (seq_len != nullptr) seq_len[b] = L1 + k + 1;
    sum += n;
  }
  if (verified == nullptr) return;
  for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if ((tid & (kWave - 1)) == 0) part[tid / kWave] = sum;
  __syncthreads();
  if (tid == 0) {
    long long total = 0;
    for (int w = 0; w < kCommitThreads / kWave; ++w) total += part[w];
    verified[0] += total;
  }
}

hipError_t launch_kv_append(const void* k_rows, const void* v_rows, void* k_pages, void* v_pages,
                            const int* bt, int max_pages, const int* pos, int B, int n, int Hkv,
                            int row_bytes, hipStream_t stream) {
  const int chunks = row_bytes / 16;
  const long long total = (long long)B * n * Hkv * chunks;
  const long long blocks = (total + kAppendThreads - 1) / kAppendThreads;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream,
                     (const uint4*)k_rows, (const uint4*)v_rows, (uint4*)k_pages, (uint4*)v_pages, bt,
                     max_pages, pos, n, Hkv, chunks, total);
  return hipGetLastError();
}

hipError_t launch_commit(const int* n_out, const int* tokens, int B, int k, int* ctx_len, int* pending,
                         int* cur_len, int* seq_len, long long* verified, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(kCommitThreads), 0, stream, n_out, tokens, B, k, ctx_len,
                     pending, cur_len, seq_len, verified);
  return hipGetLastError();
}

}  // namespace s3r
