// s3r_spec_sample kernels: exact speculative sampling from caller uniforms.
//
// [explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
// mean?", Jargon "Exact speculative sampling" and the draft/verify
// illustration: accepted drafts are kept, the first mismatch is replaced by a
// corrected token, the rest is discarded. [news] "Long-context RL training
// stops waiting on autoregressive rollouts...", Interpretation: accept
// candidates or draw from the residual distribution. [listing] "S^3R: Fast
// and Faithful RL Rollouts via Self-Sparse Speculative Decoding", Table 7
// caption: a fully accepted round yields k + 1 tokens.
//
// The step reads 2k + 1 logit rows per sequence (vocabulary-sized), so it is
// an HBM stream. All probabilities are formed in float64 from the float32
// logits, because the inverse-CDF draw compares a cumulative sum over the
// whole vocabulary with u * Z and adjacent boundaries are only ~Z/V apart.
//   1. row_stats_kernel  (2k+1 rows x B): max, first argmax and the float64
//      normaliser sum exp((z - max) / T), one pass with per-thread online
//      rescaling, fixed-order tree merge;
//   2. decide_kernel     (B): the k ratio tests on k lanes, a ballot for the
//      first reject, token counts; greedy (T = 0) finishes here;
//   3. chunk_sum_kernel  (chunks x B): float64 sums of the draw weights
//      (residual max(0, p - q) or p) per vocabulary chunk, plus sums of p for
//      the all-zero-residual fallback;
//   4. final_draw_kernel (B): locate u * Z among the chunk sums (a wave scan,
//      one lane per chunk), then inside that chunk each thread weighs 16
//      consecutive tokens, a block scan gives its starting cumulative weight,
//      and the first token whose cumulative weight exceeds u * Z is taken.

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

constexpr int kSmpThreads = 256;
constexpr int kSmpWaves = kSmpThreads / kWave;

struct SampleWs {
  float* smax;    // [B][2k+1]
  double* ssum;   // [B][2k+1]
  int* sarg;      // [B][2k+1]
  int* desc;      // [B]: -1 done, else istar | (resid << 8)
  double* csum;   // [B][kSmpChunks][2]
};

static size_t align256s(size_t x) { return (x + 255) & ~(size_t)255; }

// Float64 exponential, table-driven (Tang, "Table-driven implementation of the
// exponential function in IEEE floating-point arithmetic", ACM TOMS 1989):
// x = (256 m + j) ln2/256 + r with |r| <= ln2/512, exp(x) = 2^m 2^(j/256) (1 + p(r)),
// p the degree-3 Taylor polynomial of expm1 (truncation r^4/24 < 1.5e-13
// relative). The 256 table entries 2^(j/256) are computed once per workgroup
// with the library exp2. Relative error under 1.5e-13 for the arguments used
// here (x <= 0), well inside the 1e-12 by which the sampling decisions must
// stay clear of a flip.
constexpr int kExpTab = 256;
struct Exp64Table {
  double t[kExpTab];
};

__device__ __forceinline__ void exp64_init(Exp64Table& tab) {
  for (int j = threadIdx.x; j < kExpTab; j += blockDim.x) tab.t[j] = exp2((double)j / kExpTab);
  __syncthreads();
}

__device__ __forceinline__ double exp64(double x, const Exp64Table& tab) {
  x = fmax(x, -1000.0);
  // m = round(x 256 / ln2): adding 1.5 * 2^52 leaves the integer in the low
  // word of the sum (round to nearest even), and subtracting it again gives m
  constexpr double kShift = 6755399441055744.0;
  const double t = fma(x, kExpTab / 0.6931471805599453, kShift);
  const int ki = __double2loint(t);
  const double kf = t - kShift;
  const double r = fma(-kf, 0.6931471805599453 / kExpTab, x);
  double p = fma(r, 1.0 / 6.0, 0.5);
  p = fma(r, p, 1.0);
  p = p * r;
  const double s = tab.t[ki & (kExpTab - 1)];
  return ldexp(fma(s, p, s), ki >> 8);
}

static SampleWs sample_ws(void* ws, int B, int k, size_t* bytes_out) {
  const size_t nr = (size_t)B * (2 * k + 1);
  size_t off = 0;
  SampleWs w;
  char* base = (char*)ws;
  w.smax = (float*)(base + off);
  off = align256s(off + nr * sizeof(float));
  w.ssum = (double*)(base + off);
  off = align256s(off + nr * sizeof(double));
  w.sarg = (int*)(base + off);
  off = align256s(off + nr * sizeof(int));
  w.desc = (int*)(base + off);
  off = align256s(off + (size_t)B * sizeof(int));
  w.csum = (double*)(base + off);
  off = align256s(off + (size_t)B * kSmpChunks * 2 * sizeof(double));
  if (bytes_out) *bytes_out = off;
  return w;
}

size_t sample_workspace_bytes(int B, int k, int V) {
  (void)V;
  size_t bytes = 0;
  sample_ws(nullptr, B, k, &bytes);
  return bytes;
}

__device__ __forceinline__ const float* logit_row(const float* zt, const float* zd, int b, int r, int k, int V) {
  return r <= k ? zt + ((size_t)b * (k + 1) + r) * V : zd + ((size_t)b * k + (r - k - 1)) * V;
}

// (max, sum, argmax) triple; sum is relative to max.
struct Stat {
  float m;
  double s;
  int i;
};

__device__ __forceinline__ Stat stat_merge(Stat a, Stat b, double invT, bool greedy, const Exp64Table& tab) {
  Stat r;
  r.m = fmaxf(a.m, b.m);
  r.i = a.m > b.m ? a.i : (b.m > a.m ? b.i : min(a.i, b.i));
  if (greedy) {
    r.s = 0.0;
  } else {
    const double sa = a.m == kNegInf ? 0.0 : a.s * exp64(((double)a.m - (double)r.m) * invT, tab);
    const double sb = b.m == kNegInf ? 0.0 : b.s * exp64(((double)b.m - (double)r.m) * invT, tab);
    r.s = sa + sb;
  }
  return r;
}

// Online update with one element, branch-free: if z raises the maximum the
// running sum is rescaled by exp((m - z) / T) and z contributes 1, otherwise z
// contributes exp((z - m) / T); both use exp(-|z - m| / T).
__device__ __forceinline__ void stat_add(Stat& st, float z, int y, double invT, bool greedy,
                                         const Exp64Table& tab) {
  const bool up = z > st.m;
  if (!greedy) {
    const double e = exp64(-fabs((double)z - (double)st.m) * invT, tab);  // m = -inf -> 0
    st.s = up ? fma(st.s, e, 1.0) : st.s + e;
  }
  st.i = up ? y : st.i;
  st.m = up ? z : st.m;
}

// UNIT: temperature 1, where the exponent's factor 1 / T is 1 and its
// multiply is dropped (the same values: the product is exact).
template <bool GREEDY, bool UNIT>
__global__ __launch_bounds__(kSmpThreads) void row_stats_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, int k, int V, double invT,
    float* __restrict__ smax, double* __restrict__ ssum, int* __restrict__ sarg) {
  __shared__ float sh_m[kSmpThreads];
  __shared__ double sh_s[kSmpThreads];
  __shared__ int sh_i[kSmpThreads];
  __shared__ Exp64Table tab;
  exp64_init(tab);
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* z = logit_row(zt, zd, b, r, k, V);
  Stat st = {kNegInf, 0.0, 0x7fffffff};
  constexpr bool gr = GREEDY;
  auto sc = [&](double x) { return UNIT ? x : x * invT; };
  if ((V & 3) == 0) {
    const float4* z4 = reinterpret_cast<const float4*>(z);
    const int n4 = V >> 2;
    constexpr int U = 8;  // float4 loads in flight per thread
    for (int t0 = tid; t0 < n4; t0 += U * kSmpThreads) {
      float4 vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kSmpThreads;
        if (t < n4) {
          const u32x4_t w = load_nt16(z4 + t);
          vv[u] = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
        } else {
          vv[u] = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kSmpThreads;
        const float4 v = vv[u];
        if (t >= n4) continue;
        if (gr) {
          stat_add(st, v.x, 4 * t, invT, gr, tab);
          stat_add(st, v.y, 4 * t + 1, invT, gr, tab);
          stat_add(st, v.z, 4 * t + 2, invT, gr, tab);
          stat_add(st, v.w, 4 * t + 3, invT, gr, tab);
          continue;
        }
        // raise the running maximum once per group of 4, then 4 plain terms
        const float gm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        if (__any(gm > st.m)) {
          const bool up = gm > st.m;
          const int gi = v.x == gm ? 0 : (v.y == gm ? 1 : (v.z == gm ? 2 : 3));
          const double a = st.m == kNegInf ? 0.0 : exp64(sc(((double)st.m - (double)gm)), tab);
          st.s = up ? st.s * a : st.s;
          st.i = up ? 4 * t + gi : st.i;
          st.m = up ? gm : st.m;
        }
        const double m = (double)st.m;
        st.s += exp64(sc((double)v.x - m), tab) + exp64(sc((double)v.y - m), tab) +
                exp64(sc((double)v.z - m), tab) + exp64(sc((double)v.w - m), tab);
      }
    }
  } else {
    for (int y = tid; y < V; y += kSmpThreads) stat_add(st, z[y], y, invT, gr, tab);
  }
  sh_m[tid] = st.m;
  sh_s[tid] = st.s;
  sh_i[tid] = st.i;
  __syncthreads();
  for (int half = kSmpThreads / 2; half > 0; half >>= 1) {
    if (tid < half) {
      Stat a = {sh_m[tid], sh_s[tid], sh_i[tid]};
      Stat c = {sh_m[tid + half], sh_s[tid + half], sh_i[tid + half]};
      Stat m = stat_merge(a, c, invT, gr, tab);
      sh_m[tid] = m.m;
      sh_s[tid] = m.s;
      sh_i[tid] = m.i;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const size_t o = (size_t)b * (2 * k + 1) + r;
    smax[o] = sh_m[0];
    ssum[o] = sh_s[0];
    sarg[o] = sh_i[0];
  }
}

// Probability of logit z in a row with maximum m and normaliser s, given as
// inv_s = 1 / s (one division per row instead of one per token).
template <bool UNIT = false>
__device__ __forceinline__ double prob(float z, float m, double inv_s, double invT, const Exp64Table& tab) {
  const double x = (double)z - (double)m;
  return exp64(UNIT ? x : x * invT, tab) * inv_s;
}

__global__ __launch_bounds__(kWave) void decide_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, const int* __restrict__ dtok,
    const float* __restrict__ u, int k, int V, double invT, int greedy,
    const float* __restrict__ smax, const double* __restrict__ ssum, const int* __restrict__ sarg,
    int* __restrict__ tokens, int* __restrict__ n_out, int8_t* __restrict__ accepted,
    int* __restrict__ desc) {
  __shared__ Exp64Table tab;
  exp64_init(tab);
  const int b = blockIdx.x, lane = threadIdx.x;
  const size_t so = (size_t)b * (2 * k + 1);
  // Lane i < k runs the ratio test of draft i; the first rejection ends the
  // round, so tests past it are computed but never used (their results are
  // the same as if the tests ran one after another and stopped there).
  int x = 0;
  bool acc = true;
  if (lane < k) {
    x = dtok[(size_t)b * k + lane];
    if (greedy) {
      acc = x == sarg[so + lane];
    } else if ((unsigned)x < (unsigned)V) {
      const double p = prob(zt[((size_t)b * (k + 1) + lane) * V + x], smax[so + lane], 1.0 / ssum[so + lane], invT, tab);
      const double qq = prob(zd[((size_t)b * k + lane) * V + x], smax[so + k + 1 + lane], 1.0 / ssum[so + k + 1 + lane],
                             invT, tab);
      acc = (p >= qq) || ((double)u[(size_t)b * (k + 1) + lane] * qq < p);
    } else {
      acc = false;  // a token outside the vocabulary is never accepted
    }
  }
  const uint64_t rej = __ballot(lane < k && !acc);
  const int istar = rej ? __ffsll((unsigned long long)rej) - 1 : k;
  if (lane < k) {
    if (accepted) accepted[(size_t)b * k + lane] = lane < istar ? 1 : (lane == istar ? 0 : -1);
    if (lane < istar) tokens[(size_t)b * (k + 1) + lane] = x;
  }
  for (int j = istar + 1 + lane; j <= k; j += kWave) tokens[(size_t)b * (k + 1) + j] = -1;
  if (lane == 0) {
    n_out[b] = istar + 1;
    if (greedy) {
      tokens[(size_t)b * (k + 1) + istar] = sarg[so + istar];
      desc[b] = -1;
    } else {
      desc[b] = istar | ((istar < k ? 1 : 0) << 8);
    }
  }
}

template <bool UNIT>
__global__ __launch_bounds__(kSmpThreads) void chunk_sum_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, int k, int V, double invT,
    const float* __restrict__ smax, const double* __restrict__ ssum, const int* __restrict__ desc,
    double* __restrict__ csum) {
  __shared__ double sh[2][kSmpThreads];
  __shared__ Exp64Table tab;
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int dsc = desc[b];
  if (dsc < 0) return;
  exp64_init(tab);
  const int istar = dsc & 0xff;
  const bool resid = (dsc >> 8) != 0;
  const int csz = ceil_div(V, kSmpChunks);
  const int y0 = c * csz, y1 = min(V, y0 + csz);
  const size_t so = (size_t)b * (2 * k + 1);
  const float* zr = zt + ((size_t)b * (k + 1) + istar) * V;
  const float* dr = resid ? zd + ((size_t)b * k + istar) * V : nullptr;
  const float mt = smax[so + istar];
  const double st = ssum[so + istar];
  const float md = resid ? smax[so + k + 1 + istar] : 0.f;
  const double sd = resid ? ssum[so + k + 1 + istar] : 1.0;
  double aw = 0.0, ap = 0.0;
  // Loads in flight per thread: a whole chunk of the vocabulary in one step
  // for V up to 64 x 256 x U, issued before the row statistics are waited on,
  // so a workgroup pays two memory round trips (descriptor, then statistics
  // and logits together).
  constexpr int U = 10;
  float zt_v[U], zd_v[U];
  auto load_step = [&](int y0u) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int y = y0u + u * kSmpThreads;
      zt_v[u] = y < y1 ? zr[y] : 0.f;
      zd_v[u] = (resid && y < y1) ? dr[y] : 0.f;
    }
  };
  load_step(y0 + tid);
  const double inv_st = 1.0 / st, inv_sd = resid ? 1.0 / sd : 1.0;
  for (int y0u = y0 + tid; y0u < y1; y0u += U * kSmpThreads) {
    if (y0u != y0 + tid) load_step(y0u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (y0u + u * kSmpThreads >= y1) continue;
      const double p = prob<UNIT>(zt_v[u], mt, inv_st, invT, tab);
      double w = p;
      if (resid) w = fmax(0.0, p - prob<UNIT>(zd_v[u], md, inv_sd, invT, tab));
      aw += w;
      ap += p;
    }
  }
  sh[0][tid] = aw;
  sh[1][tid] = ap;
  __syncthreads();
  for (int half = kSmpThreads / 2; half > 0; half >>= 1) {
    if (tid < half) {
      sh[0][tid] += sh[0][tid + half];
      sh[1][tid] += sh[1][tid + half];
    }
    __syncthreads();
  }
  if (tid == 0) {
    csum[((size_t)b * kSmpChunks + c) * 2] = sh[0][0];
    csum[((size_t)b * kSmpChunks + c) * 2 + 1] = sh[1][0];
  }
}

__global__ __launch_bounds__(kSmpThreads) void final_draw_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, const float* __restrict__ u, int k,
    int V, double invT, const float* __restrict__ smax, const double* __restrict__ ssum,
    const int* __restrict__ desc, const double* __restrict__ csum, int* __restrict__ tokens) {
  __shared__ int sh_chunk, sh_usep, sh_found, sh_lastpos;
  __shared__ double sh_carry, sh_t;
  __shared__ double wtot[kSmpWaves];
  __shared__ int wfound[kSmpWaves], wlast[kSmpWaves];
  __shared__ Exp64Table tab;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dsc = desc[b];
  if (dsc < 0) return;
  exp64_init(tab);
  const int istar = dsc & 0xff;
  const bool resid0 = (dsc >> 8) != 0;
  const double* cs = csum + (size_t)b * kSmpChunks * 2;
  static_assert(kSmpChunks == kWave, "one lane per vocabulary chunk");
  if (wave == 0) {
    // lane c holds chunk c: inclusive scans of the chunk sums give Z and the
    // chunk in which u * Z falls
    double cw = cs[2 * lane], cp = cs[2 * lane + 1];
    double iw = cw, ip = cp;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const double vw = __shfl_up(iw, off, kWave), vp = __shfl_up(ip, off, kWave);
      if (lane >= off) {
        iw += vw;
        ip += vp;
      }
    }
    double Z = __shfl(iw, kWave - 1, kWave);
    int usep = 0;
    if (!(Z > 0.0)) {  // all-zero residual: draw from p
      usep = 1;
      Z = __shfl(ip, kWave - 1, kWave);
      iw = ip;
      cw = cp;
    }
    const double t = (double)u[(size_t)b * (k + 1) + k] * Z;
    const uint64_t over = __ballot(iw > t);
    const uint64_t pos = __ballot(cw > 0.0);
    int chunk;
    double carry;
    if (over) {
      chunk = __ffsll((unsigned long long)over) - 1;
      carry = __shfl(iw - cw, chunk, kWave);
    } else {  // rounding left no crossing: last chunk with weight, which never crosses
      chunk = pos ? 63 - __clzll(pos) : 0;
      carry = -__builtin_huge_val();
    }
    if (lane == 0) {
      sh_chunk = chunk;
      sh_usep = usep;
      sh_carry = carry;
      sh_t = t;
      sh_found = -1;
      sh_lastpos = -1;
    }
  }
  __syncthreads();
  const int chunk = sh_chunk;
  const bool resid = resid0 && !sh_usep;
  const double t = sh_t;
  const int csz = ceil_div(V, kSmpChunks);
  const int y0 = chunk * csz, y1 = min(V, y0 + csz);
  const size_t so = (size_t)b * (2 * k + 1);
  const float* zr = zt + ((size_t)b * (k + 1) + istar) * V;
  const float* dr = resid ? zd + ((size_t)b * k + istar) * V : nullptr;
  const float mt = smax[so + istar];
  const double inv_st = 1.0 / ssum[so + istar];
  const float md = resid ? smax[so + k + 1 + istar] : 0.f;
  const double inv_sd = resid ? 1.0 / ssum[so + k + 1 + istar] : 1.0;
  // Segments of kSmpThreads x kDrawPer positions; thread tid takes kDrawPer
  // consecutive ones, so the weights are formed in parallel, one block scan of
  // the per-thread sums gives each thread its starting cumulative weight, and
  // the thread scans its own positions in token order.
  constexpr int kDrawPer = 16;
  for (int seg = y0; seg < y1; seg += kSmpThreads * kDrawPer) {
    const int a0 = seg + tid * kDrawPer;
    double w[kDrawPer];
    double tsum = 0.0;
    int tlast = -1;
#pragma unroll
    for (int e = 0; e < kDrawPer; ++e) {
      const int y = a0 + e;
      double we = 0.0;
      if (y < y1) {
        we = prob(zr[y], mt, inv_st, invT, tab);
        if (resid) we = fmax(0.0, we - prob(dr[y], md, inv_sd, invT, tab));
      }
      w[e] = we;
      tsum += we;
      tlast = we > 0.0 ? y : tlast;
    }
    // exclusive scan of the thread sums: inside the wave, then across waves
    double incl = tsum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const double v = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += v;
    }
    if (lane == kWave - 1) wtot[wave] = incl;
    int wl = tlast;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) wl = max(wl, __shfl_xor(wl, off, kWave));
    if (lane == 0) wlast[wave] = wl;
    __syncthreads();
    double cum = sh_carry + incl - tsum;
    for (int ww = 0; ww < wave; ++ww) cum += wtot[ww];
    int hit = -1;
#pragma unroll
    for (int e = 0; e < kDrawPer; ++e) {
      cum += w[e];
      if (hit < 0 && a0 + e < y1 && cum > t) hit = a0 + e;
    }
    int wf = hit < 0 ? 0x7fffffff : hit;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) wf = min(wf, __shfl_xor(wf, off, kWave));
    if (lane == 0) wfound[wave] = wf == 0x7fffffff ? -1 : wf;
    __syncthreads();
    if (tid == 0) {
      for (int ww = 0; ww < kSmpWaves; ++ww) {
        if (wlast[ww] >= 0) sh_lastpos = wlast[ww];
        if (sh_found < 0 && wfound[ww] >= 0) sh_found = wfound[ww];
      }
      double tot = 0.0;
      for (int ww = 0; ww < kSmpWaves; ++ww) tot += wtot[ww];
      sh_carry += tot;
    }
    __syncthreads();
    if (sh_found >= 0) break;
  }
  if (tid == 0) tokens[(size_t)b * (k + 1) + istar] = sh_found >= 0 ? sh_found : sh_lastpos;
}

hipError_t launch_spec_sample(const float* zt, const float* zd, const int* dtok, const float* u,
                              int B, int k, int V, float temperature, int* tokens, int* n_out,
                              int8_t* accepted, void* ws, hipStream_t stream) {
  SampleWs w = sample_ws(ws, B, k, nullptr);
  const int greedy = temperature == 0.f;
  const double invT = greedy ? 0.0 : 1.0 / (double)temperature;
  const bool unit = temperature == 1.f;
  if (greedy)
    hipLaunchKernelGGL((row_stats_kernel<true, false>), dim3(2 * k + 1, B), dim3(kSmpThreads), 0, stream, zt,
                       zd, k, V, invT, w.smax, w.ssum, w.sarg);
  else if (unit)
    hipLaunchKernelGGL((row_stats_kernel<false, true>), dim3(2 * k + 1, B), dim3(kSmpThreads), 0, stream, zt,
                       zd, k, V, invT, w.smax, w.ssum, w.sarg);
  else
    hipLaunchKernelGGL((row_stats_kernel<false, false>), dim3(2 * k + 1, B), dim3(kSmpThreads), 0, stream, zt,
                       zd, k, V, invT, w.smax, w.ssum, w.sarg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decide_kernel, dim3(B), dim3(kWave), 0, stream, zt, zd, dtok, u, k, V, invT,
                     greedy, w.smax, w.ssum, w.sarg, tokens, n_out, accepted, w.desc);
  e = hipGetLastError();
  if (e != hipSuccess || greedy) return e;
  if (unit)
    hipLaunchKernelGGL(chunk_sum_kernel<true>, dim3(kSmpChunks, B), dim3(kSmpThreads), 0, stream, zt, zd, k,
                       V, invT, w.smax, w.ssum, w.desc, w.csum);
  else
    hipLaunchKernelGGL(chunk_sum_kernel<false>, dim3(kSmpChunks, B), dim3(kSmpThreads), 0, stream, zt, zd, k,
                       V, invT, w.smax, w.ssum, w.desc, w.csum);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(final_draw_kernel, dim3(B), dim3(kSmpThreads), 0, stream, zt, zd, u, k, V, invT,
                     w.smax, w.ssum, w.desc, w.csum, tokens);
  return hipGetLastError();
}

}  // namespace s3r

namespace s3r {

// Scratch of the no-allocation entry point: the workspace of the kernels above
// in the library's own device memory, a fixed array that every GPU the library
// runs on holds until the process ends. In host code `scratch` is a host-side
// stand-in, not a device address: its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address reaches the kernels. Calls on one GPU share the array.
static __device__ __align__(256) char scratch[kSampleScratchBytes];

constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kScratchDevices] = {};

hipError_t sample_scratch(hipStream_t stream, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace s3r
