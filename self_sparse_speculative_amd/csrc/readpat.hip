// Measurement kernels: the HBM read patterns of the verification and of a
// draft step, with none of their arithmetic. They read exactly the bytes the
// two MFMA kernels read (every K and V row of the cache in 32-position
// subtiles of two pages; the kept rows of one draft step), in the same launch
// shape (workgroups of 256 threads, the verification's splits of at most 4096
// positions on the XCD-grouped 1-D grid, the draft's splits of at most 2048
// positions), with the same per-instruction layout and cache hints
// (nontemporal loads for the verification's V rows and for every row of a
// draft step, ordinary whole-line loads for the verification's K pages), and
// fold the loaded words into one 32-bit checksum per
// workgroup so that no load is dropped. Their time is the read ceiling the
// attention kernels are measured against; nothing in the method uses them.

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

constexpr int kRpThreads = 256;
constexpr int kRpWaves = kRpThreads / kWave;
constexpr int kRpSub = 32;

__device__ __forceinline__ uint32_t fold4(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Verification pattern: K and V of every position [0, seq_len[b]) of each
// (sequence, KV head), 16 B per lane per load in the verification's own
// per-instruction layout, waves on alternate subtiles.
__global__ __launch_bounds__(kRpThreads, 2) void read_verify_pattern_kernel(
    const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp, const int* __restrict__ bt, int max_pages,
    int npairs, int Hkv, const int* __restrict__ seq_len, int chunk, int nsplit, uint32_t* __restrict__ sink) {
  constexpr int D = 128;
  __shared__ int pages_sh[kVerChunkMfma / kPage];
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int pair = (local / nsplit) * 8 + xcd, split = local % nsplit;
  if (pair >= npairs) return;
  const int b = pair / Hkv, kv = pair % Hkv;
  const int S = seq_len[b];
  const int ch = ceil_div(ceil_div(S, ceil_div(S, chunk)), kRpSub) * kRpSub;
  const int c0 = split * ch;
  if (c0 >= S) return;
  const int c1 = min(S, c0 + ch);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int npg = ceil_div(c1 - c0, kPage);
  const int* bt_row = bt + (size_t)b * max_pages;
  for (int t = tid; t < npg; t += kRpThreads) pages_sh[t] = bt_row[(c0 >> 4) + t];
  __syncthreads();
  uint32_t acc = 0;
  const int nsub = ceil_div(c1 - c0, kRpSub);
  for (int st = wave; st < nsub; st += kRpWaves) {
    const int page_a = pages_sh[2 * st];
    const int page_b = (c0 + st * kRpSub + 16 < S) ? pages_sh[2 * st + 1] : page_a;
    uint4 w[16];
    // K as the verification loads it: each page's 4 KB block, 1 KB
    // contiguous per wave instruction, ordinary loads
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const bf16_t* kb = kp + ((size_t)(pt ? page_b : page_a) * Hkv + kv) * kPage * D + lane * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[pt * 4 + i] = *reinterpret_cast<const uint4*>(kb + i * 512);
    }
    // V as the verification loads it for its transpose: lane task (4 positions
    // a, 16 B chunk c), 8 rows x 128 B per instruction, nontemporal loads
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int task = lane + 64 * tt;
      const int a = task & 7, c = task >> 3;
      const int page = a < 4 ? page_a : page_b;
      const bf16_t* vb = vp + (((size_t)page * Hkv + kv) * kPage + (a & 3) * 4) * D + c * 8;
#pragma unroll
      for (int v = 0; v < 4; ++v) w[8 + tt * 4 + v] = load_nt16_u4(vb + v * D);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= fold4(w[i]);
  }
  // one word per workgroup: the xor over its lanes
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, kWave);
  __shared__ uint32_t red[kRpWaves];
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Draft pattern: the K and V rows of the kept positions idx[b][kv][0, n_sel)
// and of [sel_len, cur_len), 16 lanes per 256 B row.
__global__ __launch_bounds__(kRpThreads, 2) void read_draft_pattern_kernel(
    const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp, const int* __restrict__ bt, int max_pages,
    int Hkv, const int* __restrict__ idx, int nsel_cap, const int* __restrict__ n_sel,
    const int* __restrict__ sel_len, const int* __restrict__ cur_len, int chunk, uint32_t* __restrict__ sink) {
  constexpr int D = 128;
  __shared__ int rows[kDecChunkMfma];
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = n_sel[b], L = sel_len[b], cur = cur_len[b];
  const int total = ns + (cur - L);
  const int p0 = split * chunk;
  uint32_t acc = 0;
  if (p0 < total) {
    const int p1 = min(total, p0 + chunk);
    const int* idx_row = idx + ((size_t)b * Hkv + kv) * nsel_cap;
    const int* bt_row = bt + (size_t)b * max_pages;
    for (int j = p0 + tid; j < p1; j += kRpThreads) {
      const int pos = j < ns ? idx_row[j] : L + (j - ns);
      rows[j - p0] = (bt_row[pos >> 4] * Hkv + kv) * kPage + (pos & 15);
    }
    __syncthreads();
    const int n16 = lane & 15, g4 = lane >> 4;
    // a wave takes 4 rows per step (16 lanes per row, 16 B per lane)
    for (int j = wave * 4 + g4; j < p1 - p0; j += kRpWaves * 4) {
      const size_t row = (size_t)rows[j] * D + n16 * 8;
      acc ^= fold4(load_nt16_u4(kp + row)) ^ fold4(load_nt16_u4(vp + row));
    }
  }
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, kWave);
  __shared__ uint32_t red[kRpWaves];
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) sink[((size_t)b * gridDim.y + kv) * gridDim.x + split] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

size_t read_verify_pattern_words(int B, int Hkv, int max_seq_len) {
  return (size_t)ceil_div(B * Hkv, 8) * 8 * ceil_div(max_seq_len, kVerChunkMfma);
}

size_t read_draft_pattern_words(int B, int Hkv, int max_attend) {
  const int nsplit = ceil_div(max_attend, kDecChunkMfma);
  return (size_t)B * Hkv * nsplit;
}

hipError_t launch_read_verify_pattern(const void* kp, const void* vp, const int* bt, int max_pages, int Hkv,
                                      const int* seq_len, int B, int max_seq_len, uint32_t* sink,
                                      hipStream_t stream) {
  const int nsplit = ceil_div(max_seq_len, kVerChunkMfma);
  const int npairs = B * Hkv;
  const int nblocks = ceil_div(npairs, 8) * 8 * nsplit;
  hipLaunchKernelGGL(read_verify_pattern_kernel, dim3(nblocks), dim3(kRpThreads), 0, stream, (const bf16_t*)kp,
                     (const bf16_t*)vp, bt, max_pages, npairs, Hkv, seq_len, kVerChunkMfma, nsplit, sink);
  return hipGetLastError();
}

hipError_t launch_read_draft_pattern(const void* kp, const void* vp, const int* bt, int max_pages, int Hkv,
                                     const int* idx, int nsel_cap, const int* n_sel, const int* sel_len,
                                     const int* cur_len, int B, int max_attend, uint32_t* sink,
                                     hipStream_t stream) {
  // the draft kernel's equal splits of at most kDecChunkMfma positions
  const int nsplit = ceil_div(max_attend, kDecChunkMfma);
  const int chunk = ceil_div(ceil_div(max_attend, nsplit), 32) * 32;
  hipLaunchKernelGGL(read_draft_pattern_kernel, dim3(nsplit, Hkv, B), dim3(kRpThreads), 0, stream,
                     (const bf16_t*)kp, (const bf16_t*)vp, bt, max_pages, Hkv, idx, nsel_cap, n_sel, sel_len,
                     cur_len, chunk, sink);
  return hipGetLastError();
}

}  // namespace s3r
