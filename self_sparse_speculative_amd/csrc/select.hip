// s3r_select kernel: newest window plus the top-scoring older positions per
// (sequence, KV head), in ascending position order.
//
// [explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
// mean?", mechanism paragraph: the draft reads the most recent positions and
// those that the previous verification pass weighted most.
//
// One workgroup (512 threads) per (KV head, sequence). Scores are mapped to
// order-preserving 32-bit keys (-0.0 folded onto +0.0). A 12-bit histogram
// (wave-aggregated LDS atomics) finds the bucket that holds the threshold
// rank; the keys of that bucket are compacted into LDS and an exact radix
// select on their low 20 bits yields the threshold key T and how many keys
// equal to T are kept; an ordered pass with wave ballots then writes every key
// above T plus the lowest-position keys equal to T, in position order. The row
// is re-read from global memory (L2 / Infinity Cache) for each pass, which
// keeps the LDS footprint small. Long rows first try the sampled-threshold
// path below (one pass over the row, the rest in LDS). Everything is integer
// work on the keys, so the result is exact.

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

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
    const int leader = __ffsll((unsigned long long)pending) - 1;  // wave-uniform
    const uint32_t d = __builtin_amdgcn_readlane(digit, leader);
    const uint64_t same = __ballot(take && digit == d) & pending;
    if (lane == leader) atomicAdd(&hist[d], (uint32_t)__popcll(same));
    pending &= ~same;
  }
  if ((pending >> lane) & 1ull) atomicAdd(&hist[digit], 1u);
}

// ---------------------------------------------------------------------------
// Streaming selector (default). The candidate keys are read from global memory
// (the row stays in L2 / Infinity Cache between passes) so the workgroup needs
// little LDS and several workgroups share a CU:
//   A. 12-bit histogram of the keys (sign, exponent, 3 mantissa bits);
//   B. the bucket holding the threshold rank is compacted into an LDS list
//      (key, position) when it has at most kFsCap keys, and an exact radix
//      select over the remaining 20 bits runs on the list; a larger bucket
//      (e.g. many equal scores) continues with radix passes over the row;
//   C. the ordered output pass of the LDS kernel, on masked keys.
constexpr int kFsThreads = 512;
constexpr int kFsWaves = kFsThreads / kWave;
constexpr int kFsBins = 4096;
constexpr int kFsCap = 2048;

// Find the bucket holding the key of rank `rank` (1-based, counted from the
// largest key). hist has nbins counts in key order. Every thread returns the
// bucket, the rank inside it and the bucket's count.
__device__ __forceinline__ void find_rank_bucket(const uint32_t* hist, int nbins, int rank, int* wsum,
                                                 int* out3) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int per = (nbins + kFsThreads - 1) / kFsThreads;
  int own = 0;
  for (int e = 0; e < per; ++e) {
    const int i = tid * per + e;  // i-th bucket from the top
    if (i < nbins) own += (int)hist[nbins - 1 - i];
  }
  int incl = own;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int excl = before + incl - own;
  if (excl < rank && rank <= excl + own) {
    int cum = excl;
    for (int e = 0; e < per; ++e) {
      const int i = tid * per + e;
      const int c = (int)hist[nbins - 1 - i];
      if (cum + c >= rank) {
        out3[0] = nbins - 1 - i;
        out3[1] = rank - cum;
        out3[2] = c;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Sampled-threshold path for long rows (one full pass over the row instead of
// four). A sample of the keys (runs of 16 consecutive positions spread evenly
// over the row) gives a key t0 (19-bit resolution: an 11-bit and an 8-bit
// histogram of the sample) at sample rank r + 5 sqrt(r) + 12, r being the wanted count's
// share of the sample: about five standard deviations of the sample rank
// above it, so that rows falling back stay rare (a single row that falls back
// sets the launch's critical path).
// One ordered pass collects every key >= t0 with its position into LDS
// (position order). If the list holds at least the wanted count and fits,
// an exact radix select on the list gives the threshold key T and how many
// keys equal to T are kept, and an ordered scan of the list writes the
// result; otherwise the row takes the streaming path. Both paths give the
// same kept set: the rule is exact either way.
// The list capacity is a launch argument: the host sizes it (and the dynamic
// LDS) for the largest row's expected list, so large budgets keep the path.
// Positions are 16-bit offsets, so rows of more than 65536 candidates take the
// streaming path.
constexpr int kSpMinRow = 2048;   // shorter rows take the streaming path directly
constexpr int kSpMaxRow = 65536;  // longer rows do too (16-bit list positions)
constexpr int kSpSample = 2560;   // most sample keys
constexpr int kSpRun = 16;        // consecutive positions per sample run
constexpr int kSpBins = 2048;     // 11-bit digits
constexpr int kSpCapMin = 2560;   // list capacity bounds (entries of 6 B)
constexpr int kSpCapMax = 8192;
#ifndef S3R_SELECT_SEG
#define S3R_SELECT_SEG 4
#endif
constexpr int kSpSeg = S3R_SELECT_SEG;  // consecutive keys per thread per step of the collecting pass
#ifndef S3R_SELECT_PREFETCH
#define S3R_SELECT_PREFETCH 1
#endif
constexpr bool kSpPrefetch = S3R_SELECT_PREFETCH != 0;  // next step's keys loaded during this step's scan

// Sample rank of t0 for `ntop` wanted keys out of `ncand`, sampling `ns` keys.
__host__ __device__ __forceinline__ int sampled_want(int ntop, int ncand, int ns) {
  const float r = (float)ntop * (float)ns / (float)ncand;
  return (int)ceilf(r + 5.0f * sqrtf(r)) + 12;
}

__host__ __device__ __forceinline__ int sampled_count(int ncand) {
  return min(ncand / 128, kSpSample / kSpRun) * kSpRun;
}

// Dynamic LDS of select_stream_kernel for list capacity `cap`: the streaming
// path's 12-bit histogram and bucket list, or the sampled path's 11-bit
// histogram, list keys and 16-bit list positions.
static inline size_t select_lds_bytes(int cap) {
  return sizeof(uint32_t) * (size_t)max(kFsBins + kFsCap, kSpBins + cap + cap / 2);
}

// List capacity for rows of up to ncand_max candidates keeping up to
// ntop_max: the expected list of the largest row plus four standard
// deviations (the sample rank of t0 is about binomial), within the bounds.
static inline int sampled_list_cap(int ncand_max, int ntop_max) {
  if (ncand_max < kSpMinRow || ntop_max < 1) return kSpCapMin;
  const int ns = sampled_count(ncand_max);
  const double want = sampled_want(ntop_max, ncand_max, ns);
  const double per = (double)ncand_max / ns;
  const double list = (want + 4.0 * sqrt(want)) * per + 64.0;
  const int cap = ((int)list + 63) / 64 * 64;
  return min(kSpCapMax, max(kSpCapMin, cap));
}

// Exclusive prefix of v over the workgroup, in thread order; *total is the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int u = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += u;
  }
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kFsWaves; ++w) {
    const int x = wsum[w];
    before += w < wave ? x : 0;
    all += x;
  }
  *total = all;
  return before + incl - v;
}

__device__ bool sampled_select(const float* __restrict__ row, int ncand, int ntop, int* __restrict__ out,
                               uint32_t* hist, uint32_t* lkey, uint16_t* lpos, int cap, int* wsum, int* res) {
  const int tid = threadIdx.x;
  // 1. the sample: nrun runs of 16 keys, run i starting at i * stride
  const int ns = sampled_count(ncand);
  const int stride = ncand / (ns / kSpRun);
  const int want = sampled_want(ntop, ncand, ns);
  // uniform decisions, taken before any LDS is touched
  if (want >= ns) return false;
  if ((long long)want * ncand > (long long)cap * ns) return false;  // the expected list does not fit
  constexpr int kSpPerThread = kSpSample / kFsThreads;  // sample keys per thread (all loads issued first)
  uint32_t skey[kSpPerThread];
#pragma unroll
  for (int q = 0; q < kSpPerThread; ++q) {
    const int i = tid + q * kFsThreads;
    skey[q] = i < ns ? score_key(row[(i / kSpRun) * stride + (i % kSpRun)]) : 0u;
  }
  // t0: the 19-bit prefix of the sample key of rank `want` (an 11-bit, then an
  // 8-bit histogram of the sample)
  for (int t = tid; t < kSpBins; t += kFsThreads) hist[t] = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSpPerThread; ++q)
    if (tid + q * kFsThreads < ns) atomicAdd(&hist[skey[q] >> 21], 1u);
  __syncthreads();
  find_rank_bucket(hist, kSpBins, want, wsum, res);
  const uint32_t tb = (uint32_t)res[0];
  const int rin = res[1];
  for (int t = tid; t < 256; t += kFsThreads) hist[t] = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSpPerThread; ++q)
    if (tid + q * kFsThreads < ns && (skey[q] >> 21) == tb) atomicAdd(&hist[(skey[q] >> 13) & 0xffu], 1u);
  __syncthreads();
  find_rank_bucket(hist, 256, rin, wsum, res);
  const uint32_t t0 = (tb << 21) | ((uint32_t)res[0] << 13);
  // 2. ordered collection of the keys >= t0: each thread takes kSpSeg
  // consecutive positions per step, so thread order is position order
  int total = 0;
  // the next step's scores are loaded before this step's scan (kSpPrefetch),
  // so each step's loads are in flight during the previous step's scan
  float nxt[kSpSeg];
  auto load_step = [&](int base) {
    const int j0 = base + kSpSeg * tid;
#pragma unroll
    for (int v = 0; v < kSpSeg; ++v) nxt[v] = j0 + v < ncand ? row[j0 + v] : 0.f;
  };
  if (kSpPrefetch) load_step(0);
  for (int base = 0; base < ncand; base += kSpSeg * kFsThreads) {
    const int j0 = base + kSpSeg * tid;
    uint32_t kk[kSpSeg];
    if (kSpPrefetch) {
#pragma unroll
      for (int v = 0; v < kSpSeg; ++v) kk[v] = j0 + v < ncand ? score_key(nxt[v]) : 0u;
      if (base + kSpSeg * kFsThreads < ncand) load_step(base + kSpSeg * kFsThreads);
    } else {
#pragma unroll
      for (int v = 0; v < kSpSeg; ++v) kk[v] = j0 + v < ncand ? score_key(row[j0 + v]) : 0u;
    }
    int c = 0;
#pragma unroll
    for (int v = 0; v < kSpSeg; ++v) c += (j0 + v < ncand && kk[v] >= t0) ? 1 : 0;
    int chunk_total;
    int off = total + block_excl_scan(c, wsum, &chunk_total);
#pragma unroll
    for (int v = 0; v < kSpSeg; ++v) {
      if (j0 + v < ncand && kk[v] >= t0) {
        if (off < cap) {
          lkey[off] = kk[v];
          lpos[off] = (uint16_t)(j0 + v);
        }
        ++off;
      }
    }
    total += chunk_total;
    if (total > cap) break;  // uniform: every thread holds the same total
  }
  __syncthreads();
  if (total > cap || total < ntop) return false;
  // 3. exact rank select on the list: T and how many keys equal to T are kept
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = ntop;
  const int shifts[3] = {21, 10, 0};
  const uint32_t widths[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  for (int ps = 0; ps < 3; ++ps) {
    const int sh = shifts[ps];
    const int nb = (int)widths[ps] + 1;
    for (int t = tid; t < nb; t += kFsThreads) hist[t] = 0u;
    __syncthreads();
    for (int i = tid; i < total; i += kFsThreads) {
      const uint32_t key = lkey[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & widths[ps]], 1u);
    }
    __syncthreads();
    find_rank_bucket(hist, nb, remaining, wsum, res);
    prefix |= (uint32_t)res[0] << sh;
    pmask |= widths[ps] << sh;
    remaining = res[1];
    if (res[2] == remaining) break;  // the whole bucket is kept
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;
  // 4. ordered output: the list is in position order; each thread takes a run of entries
  const int per = ceil_div(total, kFsThreads);
  const int e0 = min(total, tid * per), e1 = min(total, e0 + per);
  int ceq = 0;
  for (int i = e0; i < e1; ++i) ceq += (lkey[i] & pmask) == T ? 1 : 0;
  int dummy;
  int eq_before = block_excl_scan(ceq, wsum, &dummy);
  int csel = 0;
  for (int i = e0; i < e1; ++i) {
    const uint32_t km = lkey[i] & pmask;
    if (km > T) {
      ++csel;
    } else if (km == T) {
      csel += eq_before < need_eq ? 1 : 0;
      ++eq_before;
    }
  }
  int nsel_all;
  int pos = block_excl_scan(csel, wsum, &nsel_all);
  eq_before -= ceq;  // back to this thread's first equal key
  for (int i = e0; i < e1; ++i) {
    const uint32_t km = lkey[i] & pmask;
    bool sel = km > T;
    if (km == T) {
      sel = eq_before < need_eq;
      ++eq_before;
    }
    if (sel && pos < ntop) out[pos++] = (int)lpos[i];
  }
  return true;
}

// top_count (nullable): keep exactly min(L, top_count[b]) of the L candidates
// and no window (the page variant passes its candidate pages this way).
__global__ __launch_bounds__(kFsThreads) void select_stream_kernel(
    const float* __restrict__ scores, int stride, const int* __restrict__ ctx_len, int Hkv,
    int s_num, int s_den, int window, int* __restrict__ idx, int nsel_cap, int* __restrict__ n_sel,
    const int* __restrict__ top_count, int sp_cap, int* __restrict__ order) {
  // select_lds_bytes(sp_cap) of dynamic LDS: the streaming path's histogram
  // and bucket list, or the sampled path's histogram and candidate list
  extern __shared__ uint32_t lds[];
  uint32_t* hist = lds;
  uint32_t* lkey = lds + kFsBins;
  __shared__ int wsum[kFsWaves];
  __shared__ int wave_cnt[2][kFsWaves];
  __shared__ int res[3];
  __shared__ int list_n;

  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int L = ctx_len[b];
  int newest, n;
  if (top_count != nullptr) {
    newest = 0;
    n = min(L, max(0, top_count[b]));
  } else {
    newest = min(window, L);
    const long long frac = ((long long)s_num * L + s_den - 1) / s_den;
    n = (int)min((long long)L, max((long long)newest, frac));
  }
  if (kv == 0 && tid == 0) n_sel[b] = n;
  if (order != nullptr && kv == 0) {
    // the draft steps' dispatch order: rank of this sequence among all by
    // descending length, ties by index (a stable sort)
    const int B = gridDim.y;
    int c = 0;
    for (int j = tid; j < B; j += kFsThreads) {
      const int lj = ctx_len[j];
      c += (lj > L || (lj == L && j < b)) ? 1 : 0;
    }
    int rank;
    block_excl_scan(c, wsum, &rank);
    if (tid == 0) order[rank] = b;
  }
  const int ncand = L - newest, ntop = n - newest;
  int* out = idx + ((long long)b * Hkv + kv) * nsel_cap;
  for (int t = tid; t < newest; t += kFsThreads) out[ntop + t] = ncand + t;
  if (ntop <= 0) return;
  if (ntop >= ncand) {
    for (int t = tid; t < ncand; t += kFsThreads) out[t] = t;
    return;
  }
  const float* row = scores + ((long long)b * Hkv + kv) * stride;
  if (kSelSampled && ncand >= kSpMinRow && ncand <= kSpMaxRow &&
      sampled_select(row, ncand, ntop, out, lds, lds + kSpBins, reinterpret_cast<uint16_t*>(lds + kSpBins + sp_cap),
                     sp_cap, wsum, res))
    return;

  // A. histogram of the top 12 bits
  for (int t = tid; t < kFsBins; t += kFsThreads) hist[t] = 0u;
  if (tid == 0) list_n = 0;
  __syncthreads();
  for (int base = wave * kWave * 4; base < ncand; base += kFsThreads * 4) {
    uint32_t kk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = base + u * kWave + lane;
      kk[u] = j < ncand ? score_key(row[j]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) hist_add(hist, base + u * kWave + lane < ncand, kk[u] >> 20, lane);
  }
  __syncthreads();
  find_rank_bucket(hist, kFsBins, ntop, wsum, res);
  uint32_t prefix = (uint32_t)res[0] << 20, pmask = 0xfff00000u;
  int remaining = res[1];
  const int bucket_n = res[2];

  if (bucket_n != remaining) {
    if (bucket_n <= kFsCap) {
      // B. compact the threshold bucket, then radix-select its low 20 bits in LDS
      for (int base = wave * kWave * 4; base < ncand; base += kFsThreads * 4) {
        uint32_t kv4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = base + u * kWave + lane;
          kv4[u] = j < ncand ? score_key(row[j]) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = base + u * kWave + lane;
          const bool in = j < ncand && (kv4[u] & pmask) == prefix;
          const uint64_t m = __ballot(in);
          int off = 0;
          if (lane == 0 && m) off = atomicAdd(&list_n, __popcll(m));
          off = __builtin_amdgcn_readfirstlane(off);
          if (in) lkey[off + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (kWave - lane))))] = kv4[u];
        }
      }
      __syncthreads();
      const int cnt = list_n;
      const int shifts[2] = {8, 0};
      const uint32_t widths[2] = {0xfffu, 0xffu};
      for (int ps = 0; ps < 2; ++ps) {
        const int sh = shifts[ps];
        const int nb = (int)widths[ps] + 1;
        for (int t = tid; t < nb; t += kFsThreads) hist[t] = 0u;
        __syncthreads();
        for (int i = tid; i < cnt; i += kFsThreads) {
          const uint32_t kk = lkey[i];
          if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> sh) & widths[ps]], 1u);
        }
        __syncthreads();
        find_rank_bucket(hist, nb, remaining, wsum, res);
        prefix |= (uint32_t)res[0] << sh;
        pmask |= widths[ps] << sh;
        remaining = res[1];
        if (res[2] == remaining) break;  // the whole bucket is kept
      }
    } else {
      // Large tie-heavy bucket: radix passes over the row for the low 20 bits.
      const int shifts[3] = {12, 4, 0};
      const uint32_t widths[3] = {0xffu, 0xffu, 0xfu};
      for (int ps = 0; ps < 3; ++ps) {
        const int sh = shifts[ps];
        const int nb = (int)widths[ps] + 1;
        for (int t = tid; t < nb; t += kFsThreads) hist[t] = 0u;
        __syncthreads();
        for (int base = wave * kWave * 4; base < ncand; base += kFsThreads * 4) {
          uint32_t kv4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = base + u * kWave + lane;
            kv4[u] = j < ncand ? score_key(row[j]) : 0u;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = base + u * kWave + lane;
            hist_add(hist, j < ncand && (kv4[u] & pmask) == prefix, (kv4[u] >> sh) & widths[ps], lane);
          }
        }
        __syncthreads();
        find_rank_bucket(hist, nb, remaining, wsum, res);
        prefix |= (uint32_t)res[0] << sh;
        pmask |= widths[ps] << sh;
        remaining = res[1];
        if (res[2] == remaining) break;
      }
    }
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;

  // C. ordered output on masked keys, one contiguous segment per wave
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int seg = ceil_div(ceil_div(ncand, kFsWaves), kWave) * kWave;
  const int s0 = wave * seg, s1 = min(ncand, s0 + seg);
  int cgt = 0, ceq = 0;
  for (int base = s0; base < s1; base += 4 * kWave) {
    uint32_t kv4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = base + u * kWave + lane;
      kv4[u] = j < s1 ? (score_key(row[j]) & pmask) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = base + u * kWave + lane < s1;
      cgt += __popcll(__ballot(valid && kv4[u] > T));
      ceq += __popcll(__ballot(valid && kv4[u] == T));
    }
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
  for (int base = s0; base < s1; base += 4 * kWave) {
    uint32_t kv4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = base + u * kWave + lane;
      kv4[u] = j < s1 ? (score_key(row[j]) & pmask) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = base + u * kWave + lane;
      const bool valid = j < s1;
      const bool eq = valid && kv4[u] == T;
      const uint64_t beq = __ballot(eq);
      const bool sel = (valid && kv4[u] > T) || (eq && eq_run + (int)__popcll(beq & lt_mask) < need_eq);
      const uint64_t bsel = __ballot(sel);
      const int pos = sel_run + __popcll(bsel & lt_mask);
      if (sel && pos < ntop) out[pos] = j;
      eq_run += __popcll(beq);
      sel_run += __popcll(bsel);
    }
  }
}

hipError_t launch_select(const float* scores, int stride, const int* ctx_len, int B, int Hkv,
                         int max_ctx_len, int s_num, int s_den, int window, int* idx, int nsel_cap,
                         int* n_sel, int* order, hipStream_t stream) {
  const int w = min(window, max_ctx_len);
  const long long frac = ((long long)s_num * max_ctx_len + s_den - 1) / s_den;
  const int n_max = (int)min((long long)max_ctx_len, max((long long)w, frac));
  const int cap = sampled_list_cap(max_ctx_len - w, n_max - w);
  hipLaunchKernelGGL(select_stream_kernel, dim3(Hkv, B), dim3(kFsThreads), select_lds_bytes(cap), stream, scores,
                     stride, ctx_len, Hkv, s_num, s_den, window, idx, nsel_cap, n_sel, (const int*)nullptr, cap,
                     order);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection variants. [explainer], mechanism paragraph: the kept set is
// described as whole pages, recent ones and those the verification favoured.
//   all heads: one kept set per sequence from the float32 sum of its KV heads'
//              scores (heads in ascending order), copied to every KV head;
//   pages:     the newest min(window, L) positions are kept as whole pages
//              from page f = floor((L - min(window, L)) / 16) on (wc = L - 16 f
//              positions); of the f full older pages, the
//              min(f, ceil(max(0, n - wc) / 16)) with the largest float32 sum of
//              their 16 scores (slot order) are kept, ties to the lower page,
//              n = the position budget. Every KV head keeps wc + 16 x that many.
// group_keys_kernel forms the summed keys (one thread per position or page,
// additions in the stated order) and each sequence's plan; the streaming
// selector picks on the keys; expand_kernel writes the kept positions.

struct PagePlan {
  int f, wc, ntop;
};

__device__ __forceinline__ PagePlan page_plan(int L, int s_num, int s_den, int window) {
  const int w = min(window, L);
  PagePlan pp;
  pp.f = (L - w) / kPage;
  pp.wc = L - pp.f * kPage;
  const long long frac = ((long long)s_num * L + s_den - 1) / s_den;
  const int n = (int)min((long long)L, max((long long)w, frac));
  pp.ntop = min(pp.f, ceil_div(max(0, n - pp.wc), kPage));
  return pp;
}

// Lanes per unit: the page sums over all heads use 16 lanes per page (one per
// position: coalesced reads of every head, then the page sum in slot order
// through shuffles); one head's page sums use one lane per page (16 reads).
template <bool PAGES, bool ALL>
constexpr int group_lanes() { return PAGES && ALL ? kPage : 1; }

template <bool PAGES, bool ALL>
__global__ __launch_bounds__(256) void group_keys_kernel(
    const float* __restrict__ scores, int stride, const int* __restrict__ ctx_len, int Hkv, int s_num,
    int s_den, int window, float* __restrict__ keys, int kstride, int* __restrict__ units,
    int* __restrict__ top, int* __restrict__ wcount) {
  constexpr int LPU = group_lanes<PAGES, ALL>();
  const int b = blockIdx.y, g = blockIdx.z;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int L = ctx_len[b];
  const PagePlan pp = page_plan(L, s_num, s_den, window);
  const int nunits = PAGES ? pp.f : L;
  if (t == 0 && g == 0) {
    units[b] = nunits;
    top[b] = pp.ntop;
    wcount[b] = pp.wc;
  }
  const int u = t / LPU;
  if (u >= nunits) return;  // a unit's lanes leave together
  const float* row = scores + (size_t)b * Hkv * stride;
  auto pos_key = [&](int j) {
    if (!ALL) return row[(size_t)g * stride + j];
    float a = 0.f;
    for (int h = 0; h < Hkv; ++h) a += row[(size_t)h * stride + j];
    return a;
  };
  float v;
  if (!PAGES) {
    v = pos_key(u);
  } else if (LPU == 1) {
    v = 0.f;
#pragma unroll
    for (int s = 0; s < kPage; ++s) v += pos_key(u * kPage + s);
  } else {
    // candidate pages are full: position t < 16 f
    const float x = pos_key(t);
    v = __shfl(x, 0, kPage);
#pragma unroll
    for (int s = 1; s < kPage; ++s) v += __shfl(x, s, kPage);
    if ((t & (kPage - 1)) != 0) return;
  }
  keys[((size_t)b * gridDim.z + g) * kstride + u] = v;
}

// Keys of the candidate pages from scores given per page (the page-score form
// of the verification): one lane per page; the sum over the KV heads in
// ascending order for one set per sequence. Also each sequence's plan.
template <bool ALL>
__global__ __launch_bounds__(256) void page_keys_kernel(
    const float* __restrict__ page_scores, int stride, const int* __restrict__ ctx_len, int Hkv, int s_num,
    int s_den, int window, float* __restrict__ keys, int kstride, int* __restrict__ units,
    int* __restrict__ top, int* __restrict__ wcount) {
  const int b = blockIdx.y, g = blockIdx.z;
  const int u = blockIdx.x * 256 + threadIdx.x;
  const PagePlan pp = page_plan(ctx_len[b], s_num, s_den, window);
  if (u == 0 && g == 0) {
    units[b] = pp.f;
    top[b] = pp.ntop;
    wcount[b] = pp.wc;
  }
  if (u >= pp.f) return;
  const float* row = page_scores + (size_t)b * Hkv * stride;
  float v;
  if (ALL) {
    v = 0.f;
    for (int h = 0; h < Hkv; ++h) v += row[(size_t)h * stride + u];
  } else {
    v = row[(size_t)g * stride + u];
  }
  keys[((size_t)b * gridDim.z + g) * kstride + u] = v;
}

// Also, when order is given, the draft steps' dispatch order (longest context
// first, ties by index; as s3r_length_order): the KV-head-0 workgroup of
// sequence b writes order[rank of b] = b, so no kernel of its own runs for it.
template <bool PAGES>
__global__ __launch_bounds__(256) void expand_kernel(
    const int* __restrict__ sel_u, int cap_u, int G, const int* __restrict__ n_u, const int* __restrict__ units,
    const int* __restrict__ wcount, int Hkv, int* __restrict__ idx, int nsel_cap, int* __restrict__ n_sel,
    const int* __restrict__ ctx_len, int* __restrict__ order) {
  const int h = blockIdx.x, b = blockIdx.y;
  if (order != nullptr && h == 0) {
    __shared__ int wrank[256 / kWave];
    const int B = gridDim.y, L = ctx_len[b];
    int c = 0;
    for (int j = threadIdx.x; j < B; j += 256) {
      const int lj = ctx_len[j];
      c += (lj > L || (lj == L && j < b)) ? 1 : 0;
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) c += __shfl_xor(c, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) wrank[threadIdx.x / kWave] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
      int rank = 0;
      for (int w = 0; w < 256 / kWave; ++w) rank += wrank[w];
      order[rank] = b;
    }
  }
  const int g = G == 1 ? 0 : h;
  const int* src = sel_u + ((size_t)b * G + g) * cap_u;
  const int nt = n_u[b];
  const int total = PAGES ? nt * kPage + wcount[b] : nt;
  const int wstart = PAGES ? units[b] * kPage : 0;
  int* out = idx + ((size_t)b * Hkv + h) * nsel_cap;
  for (int i = threadIdx.x; i < total; i += 256) {
    int v;
    if (!PAGES) v = src[i];
    else v = i < nt * kPage ? src[i / kPage] * kPage + (i % kPage) : wstart + (i - nt * kPage);
    out[i] = v;
  }
  if (h == 0 && threadIdx.x == 0) n_sel[b] = total;
}

GroupedSelectPlan grouped_select_plan(int B, int Hkv, int max_ctx_len, int s_num, int s_den, int window,
                                      int unit, int all_heads) {
  GroupedSelectPlan p;
  p.G = all_heads ? 1 : Hkv;
  const long long w = min(window, max_ctx_len);
  const long long frac = ((long long)s_num * max_ctx_len + s_den - 1) / s_den;
  const int n_max = (int)min((long long)max_ctx_len, max(w, frac));
  p.kstride = unit == 1 ? max_ctx_len : max(1, max_ctx_len / kPage);
  p.cap_u = unit == 1 ? max(1, n_max) : max(1, ceil_div(n_max, kPage) + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.off_keys = take((size_t)B * p.G * p.kstride * sizeof(float));
  p.off_units = take((size_t)B * sizeof(int));
  p.off_top = take((size_t)B * sizeof(int));
  p.off_wc = take((size_t)B * sizeof(int));
  p.off_sel = take((size_t)B * p.G * p.cap_u * sizeof(int));
  p.off_nsel = take((size_t)B * sizeof(int));
  p.bytes = off;
  return p;
}

int grouped_select_capacity(int max_ctx_len, int s_num, int s_den, int window, int unit) {
  const long long w = min(window, max_ctx_len);
  const long long frac = ((long long)s_num * max_ctx_len + s_den - 1) / s_den;
  const long long n_max = min((long long)max_ctx_len, max(w, frac));
  if (unit == 1) return (int)n_max;
  // at most window + 15 positions of window pages, and whole older pages
  // rounding the rest of the budget up by at most 15 positions
  return (int)min((long long)max_ctx_len, max(w + kPage - 1, n_max) + kPage - 1);
}

hipError_t launch_select_pages(const float* page_scores, int stride, const int* ctx_len, int B, int Hkv,
                               int max_ctx_len, int s_num, int s_den, int window, int all_heads, int* idx,
                               int nsel_cap, int* n_sel, int* order, void* ws, hipStream_t stream) {
  const GroupedSelectPlan p = grouped_select_plan(B, Hkv, max_ctx_len, s_num, s_den, window, kPage, all_heads);
  char* w = static_cast<char*>(ws);
  float* keys = reinterpret_cast<float*>(w + p.off_keys);
  int* units = reinterpret_cast<int*>(w + p.off_units);
  int* top = reinterpret_cast<int*>(w + p.off_top);
  int* wc = reinterpret_cast<int*>(w + p.off_wc);
  int* sel = reinterpret_cast<int*>(w + p.off_sel);
  int* nsel_u = reinterpret_cast<int*>(w + p.off_nsel);
  const dim3 kgrid(ceil_div(p.kstride, 256), B, p.G);
  if (all_heads)
    hipLaunchKernelGGL(page_keys_kernel<true>, kgrid, dim3(256), 0, stream, page_scores, stride, ctx_len, Hkv,
                       s_num, s_den, window, keys, p.kstride, units, top, wc);
  else
    hipLaunchKernelGGL(page_keys_kernel<false>, kgrid, dim3(256), 0, stream, page_scores, stride, ctx_len, Hkv,
                       s_num, s_den, window, keys, p.kstride, units, top, wc);
  const int cap = sampled_list_cap(p.kstride, p.cap_u);
  hipLaunchKernelGGL(select_stream_kernel, dim3(p.G, B), dim3(kFsThreads), select_lds_bytes(cap), stream, keys,
                     p.kstride, units, p.G, s_num, s_den, 0, sel, p.cap_u, nsel_u, (const int*)top, cap,
                     (int*)nullptr);
  hipLaunchKernelGGL(expand_kernel<true>, dim3(Hkv, B), dim3(256), 0, stream, sel, p.cap_u, p.G, nsel_u, units, wc,
                     Hkv, idx, nsel_cap, n_sel, ctx_len, order);
  return hipGetLastError();
}

hipError_t launch_select_grouped(const float* scores, int stride, const int* ctx_len, int B, int Hkv,
                                 int max_ctx_len, int s_num, int s_den, int window, int unit, int all_heads,
                                 int* idx, int nsel_cap, int* n_sel, int* order, void* ws, hipStream_t stream) {
  const GroupedSelectPlan p = grouped_select_plan(B, Hkv, max_ctx_len, s_num, s_den, window, unit, all_heads);
  char* w = static_cast<char*>(ws);
  float* keys = reinterpret_cast<float*>(w + p.off_keys);
  int* units = reinterpret_cast<int*>(w + p.off_units);
  int* top = reinterpret_cast<int*>(w + p.off_top);
  int* wc = reinterpret_cast<int*>(w + p.off_wc);
  int* sel = reinterpret_cast<int*>(w + p.off_sel);
  int* nsel_u = reinterpret_cast<int*>(w + p.off_nsel);
  const int lanes = (unit == 16 && all_heads) ? kPage : 1;
  const dim3 kgrid(ceil_div(p.kstride * lanes, 256), B, p.G);
  if (unit == 1) {
    hipLaunchKernelGGL((group_keys_kernel<false, true>), kgrid, dim3(256), 0, stream, scores, stride, ctx_len, Hkv,
                       s_num, s_den, window, keys, p.kstride, units, top, wc);
    const int w = min(window, max_ctx_len);
    const int cap = sampled_list_cap(max_ctx_len - w, p.cap_u - w);
    hipLaunchKernelGGL(select_stream_kernel, dim3(1, B), dim3(kFsThreads), select_lds_bytes(cap), stream, keys,
                       p.kstride, ctx_len, 1, s_num, s_den, window, sel, p.cap_u, nsel_u, (const int*)nullptr, cap,
                       (int*)nullptr);
    hipLaunchKernelGGL(expand_kernel<false>, dim3(Hkv, B), dim3(256), 0, stream, sel, p.cap_u, 1, nsel_u, units,
                       wc, Hkv, idx, nsel_cap, n_sel, ctx_len, order);
  } else {
    if (all_heads)
      hipLaunchKernelGGL((group_keys_kernel<true, true>), kgrid, dim3(256), 0, stream, scores, stride, ctx_len,
                         Hkv, s_num, s_den, window, keys, p.kstride, units, top, wc);
    else
      hipLaunchKernelGGL((group_keys_kernel<true, false>), kgrid, dim3(256), 0, stream, scores, stride, ctx_len,
                         Hkv, s_num, s_den, window, keys, p.kstride, units, top, wc);
    const int cap = sampled_list_cap(p.kstride, p.cap_u);
    hipLaunchKernelGGL(select_stream_kernel, dim3(p.G, B), dim3(kFsThreads), select_lds_bytes(cap), stream, keys,
                       p.kstride, units, p.G, s_num, s_den, 0, sel, p.cap_u, nsel_u, (const int*)top, cap,
                       (int*)nullptr);
    hipLaunchKernelGGL(expand_kernel<true>, dim3(Hkv, B), dim3(256), 0, stream, sel, p.cap_u, p.G, nsel_u, units,
                       wc, Hkv, idx, nsel_cap, n_sel, ctx_len, order);
  }
  return hipGetLastError();
}

}  // namespace s3r
