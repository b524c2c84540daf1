// s3r_select kernel: newest window plus the top-scoring older positions per
// (sequence, KV head), in ascending position order.
//
// [explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
// mean?", mechanism paragraph: the sparse drafter reads the newest positions
// plus the top-scoring ones from the verifier's last attention pass.
//
// One workgroup per (KV head, sequence). The candidate scores are mapped to
// order-preserving 32-bit keys (-0.0 folded onto +0.0) and held in LDS; a
// 4-pass 8-bit radix select (wave-aggregated histogram atomics) finds the
// threshold key T and how many keys equal to T are needed; an ordered pass
// with wave ballots over per-wave segments then writes every key above T plus
// the lowest-position keys equal to T, in position order.
// Everything is integer work on the keys, so the result is exact.

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Add 1 to hist[digit] for every lane with `take`, aggregating lanes that share
// a digit: a few rounds serve the most common digits with one atomic each (the
// leading float bits of scores are highly repetitive), then the remaining
// lanes add individually.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool take, uint32_t digit, int lane) {
  uint64_t pending = __ballot(take);
#pragma unroll 1
  for (int round = 0; round < 4 && pending != 0ull; ++round) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const uint32_t d = __shfl(digit, leader, kWave);
    const uint64_t same = __ballot(take && digit == d) & pending;
    if (lane == leader) atomicAdd(&hist[d], (uint32_t)__popcll(same));
    pending &= ~same;
  }
  if ((pending >> lane) & 1ull) atomicAdd(&hist[digit], 1u);
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, int stride, const int* __restrict__ ctx_len, int Hkv,
    int s_num, int s_den, int window, int* __restrict__ idx, int nsel_cap, int* __restrict__ n_sel,
    int lds_keys) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ int wave_cnt[2][kSelWaves];
  __shared__ uint32_t bc_digit;
  __shared__ int bc_remaining, bc_count;

  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int L = ctx_len[b];
  const int newest = min(window, L);
  const long long frac = ((long long)s_num * L + s_den - 1) / s_den;
  const int n = (int)min((long long)L, max((long long)newest, frac));
  if (kv == 0 && tid == 0) n_sel[b] = n;
  const int ncand = L - newest, ntop = n - newest;
  int* out = idx + ((long long)b * Hkv + kv) * nsel_cap;
  for (int t = tid; t < newest; t += kSelThreads) out[ntop + t] = ncand + t;
  if (ntop <= 0) return;
  if (ntop >= ncand) {
    for (int t = tid; t < ncand; t += kSelThreads) out[t] = t;
    return;
  }
  const float* row = scores + ((long long)b * Hkv + kv) * stride;
  const bool in_lds = ncand <= lds_keys;
  if (in_lds) {
    // 8 loads in flight per thread
    constexpr int U = 8;
    for (int j0 = tid; j0 < ncand; j0 += U * kSelThreads) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kSelThreads;
        v[u] = j < ncand ? row[j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kSelThreads;
        if (j < ncand) keys[j] = score_key(v[u]);
      }
    }
  }
  __syncthreads();

  // Radix select of the ntop-th largest key, 8 bits at a time from the top.
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = ntop;  // rank of the wanted key among keys matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int t = tid; t < 256; t += kSelThreads) hist[t] = 0u;
    __syncthreads();
    for (int base = wave * kWave; base < ncand; base += kSelThreads) {
      const int j = base + lane;
      const bool valid = j < ncand;
      const uint32_t kk = valid ? (in_lds ? keys[j] : score_key(row[j])) : 0u;
      hist_add(hist, valid && (kk & pmask) == prefix, (kk >> shift) & 255u, lane);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l (top digits first)
      uint32_t c[4];
      uint32_t own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * lane - e];
        own += c[e];
      }
      uint32_t incl = own;  // inclusive prefix over lanes (counts of higher digits)
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
      }
      const uint32_t excl = incl - own;
      if (excl < (uint32_t)remaining && (uint32_t)remaining <= incl) {
        uint32_t cum = excl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (cum + c[e] >= (uint32_t)remaining) {
            bc_digit = 255u - 4u * lane - e;
            bc_remaining = remaining - (int)cum;
            bc_count = (int)c[e];
            break;
          }
          cum += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= bc_digit << shift;
    pmask |= 255u << shift;
    remaining = bc_remaining;
    const bool whole_bucket = bc_count == remaining;
    __syncthreads();
    if (whole_bucket) break;  // every key of the bucket is kept: lower digits decide nothing
  }
  // Keys are compared on the resolved prefix bits: above the prefix is kept,
  // equal to it is kept in position order while fewer than need_eq precede.
  const uint32_t T = prefix;
  const int need_eq = remaining;

  // Ordered compaction. Each wave owns one contiguous segment of positions:
  // pass A counts keys above T and equal to T per segment, one barrier
  // publishes the counts, pass B writes the kept positions in order.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int seg = ceil_div(ceil_div(ncand, kSelWaves), kWave) * kWave;
  const int s0 = wave * seg, s1 = min(ncand, s0 + seg);
  int cgt = 0, ceq = 0;
  for (int base = s0; base < s1; base += kWave) {
    const int j = base + lane;
    const bool valid = j < s1;
    const uint32_t kk = valid ? (in_lds ? keys[j] : score_key(row[j])) : 0u;
    cgt += __popcll(__ballot(valid && (kk & pmask) > T));
    ceq += __popcll(__ballot(valid && (kk & pmask) == T));
  }
  if (lane == 0) {
    wave_cnt[0][wave] = cgt;
    wave_cnt[1][wave] = ceq;
  }
  __syncthreads();
  int eq_run = 0, sel_run = 0;
  for (int w = 0; w < wave; ++w) {
    const int e = wave_cnt[1][w];
    const int taken = max(0, min(e, need_eq - eq_run));
    sel_run += wave_cnt[0][w] + taken;
    eq_run += e;
  }
  for (int base = s0; base < s1; base += kWave) {
    const int j = base + lane;
    const bool valid = j < s1;
    const uint32_t kk = valid ? (in_lds ? keys[j] : score_key(row[j])) : 0u;
    const bool eq = valid && (kk & pmask) == T;
    const uint64_t beq = __ballot(eq);
    const bool sel = (valid && (kk & pmask) > T) || (eq && eq_run + __popcll(beq & lt_mask) < need_eq);
    const uint64_t bsel = __ballot(sel);
    const int pos = sel_run + __popcll(bsel & lt_mask);
    if (sel && pos < ntop) out[pos] = j;
    eq_run += __popcll(beq);
    sel_run += __popcll(bsel);
  }
}

int select_lds_keys(int max_ncand) { return max_ncand < kSelLdsKeysMax ? max_ncand : kSelLdsKeysMax; }

hipError_t launch_select(const float* scores, int stride, const int* ctx_len, int B, int Hkv,
                         int max_ctx_len, int s_num, int s_den, int window, int* idx, int nsel_cap,
                         int* n_sel, hipStream_t stream) {
  const int lds_keys = select_lds_keys(max_ctx_len);
  const size_t lds = (size_t)lds_keys * sizeof(uint32_t);
  hipError_t e = hipFuncSetAttribute((const void*)select_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     kSelLdsKeysMax * (int)sizeof(uint32_t));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(Hkv, B), dim3(kSelThreads), lds, stream, scores, stride,
                     ctx_len, Hkv, s_num, s_den, window, idx, nsel_cap, n_sel, lds_keys);
  return hipGetLastError();
}

}  // namespace s3r
