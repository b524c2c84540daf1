// s3r_sparse_decode_attn kernels: one sparse draft step.
//
// [news] "Long-context RL training stops waiting on autoregressive rollouts...",
// Interpretation: drafting uses the policy's own weights over a small set of
// selected historical KV entries. [explainer] "S3R - Self-sparse speculative
// rollouts for RL - What does it mean?", mechanism paragraph: k fast draft
// steps read only the selected positions.
//
// The step is a gather: every attended position costs one K row and one V row
// (2 * head_dim * element bytes) and the work per byte is G multiply-adds per
// element, so it is bound by HBM gather bandwidth, not by arithmetic. Grid
// (split, KV head, sequence); a split is a chunk of the attended list
// (selected positions first, then this round's positions). An optional order
// maps the grid's sequence index to a sequence: workgroups of similar length
// dispatched together (longest first) finish a batch of mixed lengths sooner.
//
// bf16, head_dim 128: sparse_decode_mfma_kernel (below), splits of at most
// 2048 positions made equal; a lone split writes the output itself.
//
// Other dtypes / head_dim 64 (sparse_decode_kernel), splits of 256:
//   * 16 lanes share one position row (each lane loads head_dim/16 contiguous
//     elements, 16 B for bf16 x 128), so one wave gathers 4 rows per load and
//     one workgroup (4 waves) keeps 16 position streams in flight;
//   * the G query heads of the KV head are served by the same gathered rows;
//   * the 16-lane dot products are reduced with DPP (quad_perm, row_ror), the
//     softmax is online per position stream in base 2, and the streams are
//     merged with shuffles and LDS at the end of the split;
//   * a second small kernel merges the splits (log-sum-exp weights) in split
//     order, so results are deterministic.

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

constexpr int kDecThreads = 256;
constexpr int kDecStreams = kDecThreads / 16;  // position streams per workgroup
constexpr int kDecUnroll = 8;                  // positions per stream per step

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes; every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  return v;
}

template <typename T, int EPL>
struct RowLoad;

template <>
struct RowLoad<bf16_t, 8> {  // 16 B
  uint4 raw;
  __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void to_f32(float* f) const {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16lo(w[i]);
      f[2 * i + 1] = bf16hi(w[i]);
    }
  }
};

template <>
struct RowLoad<bf16_t, 4> {  // 8 B
  uint2 raw;
  __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = bf16lo(raw.x);
    f[1] = bf16hi(raw.x);
    f[2] = bf16lo(raw.y);
    f[3] = bf16hi(raw.y);
  }
};

template <>
struct RowLoad<float, 4> {  // 16 B
  float4 raw;
  __device__ __forceinline__ void load(const float* p) { raw = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = raw.x;
    f[1] = raw.y;
    f[2] = raw.z;
    f[3] = raw.w;
  }
};

template <>
struct RowLoad<float, 8> {  // 32 B
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

template <typename T>
__device__ __forceinline__ float elem_f32(const T* p, int i);
template <>
__device__ __forceinline__ float elem_f32<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float elem_f32<bf16_t>(const bf16_t* p, int i) { return bf16_to_f32(p[i]); }

// Partial record per (sequence, query head, split): [m, l, acc[D]] with
// m the running maximum in base 2 and acc the unnormalised output.
template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void sparse_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ kp, const T* __restrict__ vp,
    const int* __restrict__ bt, int max_pages, int Hkv, const int* __restrict__ idx, int nsel_cap,
    const int* __restrict__ n_sel, const int* __restrict__ sel_len, const int* __restrict__ cur_len,
    const int* __restrict__ order, float scale_log2, int chunk, int nsplit, float* __restrict__ part) {
  constexpr int EPL = D / 16;
  __shared__ float red[kDecThreads / kWave][G][D + 2];
  __shared__ int rows[kDecChunk];  // cache row (page, KV head, slot) of each attended position

  const int split = blockIdx.x, kv = blockIdx.y;
  const int b = order != nullptr ? order[blockIdx.z] : (int)blockIdx.z;
  if ((unsigned)b >= gridDim.z) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15;
  const int stream = wave * 4 + (lane >> 4);
  const int ns = n_sel[b], L = sel_len[b], cur = cur_len[b];
  const int total = ns + (cur - L);
  const int p0 = split * chunk;
  if (p0 >= total) return;
  const int p1 = min(total, p0 + chunk);
  const int Hq = Hkv * G;

  float qv[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const T* qp = q + ((size_t)b * Hq + kv * G + g) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[g][e] = elem_f32<T>(qp, e) * scale_log2;
  }
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const int* idx_row = idx + ((size_t)b * Hkv + kv) * nsel_cap;
  const int* bt_row = bt + (size_t)b * max_pages;
  // Resolve the split's positions to cache rows once: position -> page -> row.
  for (int j = p0 + tid; j < p1; j += kDecThreads) {
    const int pos = j < ns ? idx_row[j] : L + (j - ns);
    rows[j - p0] = (bt_row[pos >> 4] * Hkv + kv) * kPage + (pos & 15);
  }
  __syncthreads();

  for (int j0 = p0 + stream; j0 < p1; j0 += kDecStreams * kDecUnroll) {
    bool ok[kDecUnroll];
    RowLoad<T, EPL> kr[kDecUnroll], vr[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * kDecStreams;
      ok[u] = j < p1;
      const size_t off = (size_t)rows[(ok[u] ? j : j0) - p0] * D + sub * EPL;
      kr[u].load(kp + off);
      vr[u].load(vp + off);
    }
    // Branch-free update (a position past the split end gets logit -inf), so
    // every load above stays in flight together.
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float kf[EPL], vf[EPL];
      kr[u].to_f32(kf);
      vr[u].to_f32(vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qv[g][e], kf[e], s);
        s = ok[u] ? row16_sum(s) : kNegInf;
        const float mn = fmaxf(m[g], s);
        const float base = mn == kNegInf ? 0.f : mn;
        const float a = exp2f_fast(m[g] - base);  // m = -inf -> 0
        const float p = exp2f_fast(s - base);     // s = -inf -> 0
        l[g] = l[g] * a + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e] * a);
        m[g] = mn;
      }
    }
  }

  // Merge the 4 position streams of each wave (lanes 16 and 32 apart).
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const float mo = __shfl_xor(m[g], mask, kWave);
      const float lo = __shfl_xor(l[g], mask, kWave);
      const float mn = fmaxf(m[g], mo);
      const float base = mn == kNegInf ? 0.f : mn;
      const float a = exp2f_fast(m[g] - base), c = exp2f_fast(mo - base);
      l[g] = l[g] * a + lo * c;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[g][e], mask, kWave);
        acc[g][e] = acc[g][e] * a + ao * c;
      }
      m[g] = mn;
    }
  }
  // Merge the waves through LDS.
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (sub == 0) {
        red[wave][g][D] = m[g];
        red[wave][g][D + 1] = l[g];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][g][sub * EPL + e] = acc[g][e];
    }
  }
  __syncthreads();
  for (int t = tid; t < G * D; t += kDecThreads) {
    const int g = t / D, d = t % D;
    float M = kNegInf;
    for (int w = 0; w < kDecThreads / kWave; ++w) M = fmaxf(M, red[w][g][D]);
    const float base = M == kNegInf ? 0.f : M;
    float Ls = 0.f, A = 0.f;
    for (int w = 0; w < kDecThreads / kWave; ++w) {
      const float c = exp2f_fast(red[w][g][D] - base);
      Ls += red[w][g][D + 1] * c;
      A += red[w][g][d] * c;
    }
    float* rec = part + (((size_t)b * Hq + kv * G + g) * nsplit + split) * (D + 2);
    rec[2 + d] = A;
    if (d == 0) {
      rec[0] = M;
      rec[1] = Ls;
    }
  }
}

// bf16, head_dim 128: the same step on MFMA. Per 32-position subtile a wave
// gathers the K rows straight into A fragments of 16x16x32 bf16 MFMA tiles
// (S^T = K Q^T, the G query heads of the KV head are the N side), keeps the
// online softmax per head in the lanes that own the head, transposes the
// gathered V rows through LDS and accumulates O^T += V^T P^T on MFMA. The
// vector ALU only does the softmax, so the kernel stays a pure gather.
typedef __bf16 dbf16x8_t __attribute__((ext_vector_type(8)));
typedef float df32x4_t __attribute__((ext_vector_type(4)));
constexpr int kDsub = 32;       // positions per subtile
constexpr int kDvtStride = 40;  // LDS row stride (uint16) of a transposed V subtile

__device__ __forceinline__ uint32_t dperm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ uint32_t du4_word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int NW>
__global__ __launch_bounds__(NW * kWave, 2) void sparse_decode_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp,
    const int* __restrict__ bt, int max_pages, int Hkv, int G, const int* __restrict__ idx,
    int nsel_cap, const int* __restrict__ n_sel, const int* __restrict__ sel_len,
    const int* __restrict__ cur_len, const int* __restrict__ order, float scale_log2, int chunk, int nsplit,
    float* __restrict__ part, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int D = 128;
  constexpr int kWaves = NW;
  constexpr int kThreads = NW * kWave;
  __shared__ __attribute__((aligned(16))) uint16_t vt[kWaves][D * kDvtStride];
  __shared__ float ml_sh[kWaves][2][16];
  __shared__ int rows[kDecChunkMfma];

  // Workgroups take the sequences in `order` (when given: longest first keeps
  // workgroups of similar length together).
  const int split = blockIdx.x, kv = blockIdx.y;
  const int z = (int)blockIdx.z;
  const int b = order != nullptr ? order[z] : z;
  if ((unsigned)b >= gridDim.z) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int ns = n_sel[b], L = sel_len[b], cur = cur_len[b];
  const int total = ns + (cur - L);
  const int p0 = split * chunk;
  const int Hq = Hkv * G;
  if (p0 >= total) {
    if (nsplit == 1) {  // nothing attended: zero output, lse = -inf
      for (int t = tid; t < G * D; t += kThreads) {
        out[((size_t)b * Hq + kv * G + t / D) * D + t % D] = 0.f;
        if (lse != nullptr && t % D == 0) lse[(size_t)b * Hq + kv * G + t / D] = kNegInf;
      }
    }
    return;
  }
  const int p1 = min(total, p0 + chunk);

  // Q fragments first: their loads overlap the position resolution below.
  dbf16x8_t qf[4];
  {
    const int r = n16;
    if (r < G) {
      const bf16_t* qp = q + ((size_t)b * Hq + kv * G + r) * D + g4 * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qf[kk] = *reinterpret_cast<const dbf16x8_t*>(qp + kk * 32);
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qf[kk] = dbf16x8_t{};
    }
  }
  // Resolve the split's positions to cache rows (page, KV head, slot) once:
  // every position load of the thread is issued, then every block-table load,
  // so the two dependent round trips are paid once, not once per position.
  const int* idx_row = idx + ((size_t)b * Hkv + kv) * nsel_cap;
  const int* bt_row = bt + (size_t)b * max_pages;
  constexpr int kRes = kDecChunkMfma / kThreads;
  int rpos[kRes], rpg[kRes];
#pragma unroll
  for (int u = 0; u < kRes; ++u) {
    const int j = p0 + tid + u * kThreads;
    rpos[u] = j < p1 ? (j < ns ? idx_row[j] : L + (j - ns)) : 0;
  }
#pragma unroll
  for (int u = 0; u < kRes; ++u) {
    const int j = p0 + tid + u * kThreads;
    rpg[u] = j < p1 ? bt_row[rpos[u] >> 4] : 0;
  }
#pragma unroll
  for (int u = 0; u < kRes; ++u) {
    const int j = p0 + tid + u * kThreads;
    if (j < p1) rows[j - p0] = (rpg[u] * Hkv + kv) * kPage + (rpos[u] & 15);
  }
  __syncthreads();
  const int cnt = p1 - p0;
  float m_run = kNegInf, l_run = 0.f;
  df32x4_t oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = df32x4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* my_vt = vt[wave];
  const int nsub = ceil_div(cnt, kDsub);

  for (int st = wave; st < nsub; st += kWaves) {
    const int j0 = st * kDsub;  // subtile start within the split
    // the gathered K and V rows are read once: nontemporal loads
    dbf16x8_t kf[2][4];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int jj = j0 + pt * 16 + n16;
      const size_t row = (size_t)rows[jj < cnt ? jj : j0];
      const bf16_t* kb = kp + row * D + g4 * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kf[pt][kk] = __builtin_bit_cast(dbf16x8_t, load_nt16(kb + kk * 32));
    }
    uint4 vraw[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int task = lane + 64 * tt;
      const int a = task & 7, c = task >> 3;
      // positions 4a..4a+3 of the subtile (first page half: a < 4)
      const int pbase = (a < 4 ? 0 : 16) + (a & 3) * 4;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int jj = j0 + pbase + v;
        const size_t row = (size_t)rows[jj < cnt ? jj : j0];
        vraw[tt][v] = load_nt16_u4(vp + row * D + c * 8);
      }
    }
    df32x4_t s[2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      df32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[pt][kk], qf[kk], acc, 0, 0, 0);
      s[pt] = acc;
    }
    float mx = kNegInf;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int jj = j0 + pt * 16 + 4 * g4 + v;
        const float x = jj < cnt ? s[pt][v] * scale_log2 : kNegInf;
        s[pt][v] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mn = fmaxf(m_run, mx);
    const float base = mn == kNegInf ? 0.f : mn;
    const float alpha = exp2f_fast(m_run - base);
    float pv[2][4];
    float psum = 0.f;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pv[pt][v] = exp2f_fast(s[pt][v] - base);
        psum += pv[pt][v];
      }
    }
    l_run = l_run * alpha + psum;
    m_run = mn;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    u32x4_t pw = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                  pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
    const dbf16x8_t pf = __builtin_bit_cast(dbf16x8_t, pw);
    wave_lds_sync();  // the previous subtile's reads of the buffer precede these writes
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int task = lane + 64 * tt;
      const int a = task & 7, c = task >> 3;
      const int slot = (a & 3) * 8 + (a >> 2) * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int wi = e >> 1;
        const uint32_t lo = dperm(du4_word(vraw[tt][1], wi), du4_word(vraw[tt][0], wi), sel);
        const uint32_t hi = dperm(du4_word(vraw[tt][3], wi), du4_word(vraw[tt][2], wi), sel);
        *reinterpret_cast<uint2*>(my_vt + (c * 8 + e) * kDvtStride + slot) = make_uint2(lo, hi);
      }
    }
    wave_lds_sync();  // each lane reads rows written by other lanes
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const dbf16x8_t vfrag = *reinterpret_cast<const dbf16x8_t*>(my_vt + (dt * 16 + n16) * kDvtStride + g4 * 8);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag, pf, oacc[dt], 0, 0, 0);
    }
  }

  // Merge the waves. Row (head) n16; l is a per-lane partial.
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  __syncthreads();
  if (g4 == 0) {
    ml_sh[wave][0][n16] = m_run;
    ml_sh[wave][1][n16] = l_run;
  }
  __syncthreads();
  float* obuf = reinterpret_cast<float*>(&vt[0][0]);  // 16 x D floats
  float M = kNegInf;
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml_sh[w][0][n16]);
  const float baseM = M == kNegInf ? 0.f : M;
  const float fac = exp2f_fast(m_run - baseM);
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int o = n16 * D + dt * 16 + g4 * 4 + v;
          const float val = oacc[dt][v] * fac;
          obuf[o] = (w == 0) ? val : obuf[o] + val;
        }
      }
    }
    __syncthreads();
  }
  if (nsplit == 1) {
    // The only split: normalise here (same arithmetic as the split merge with
    // one split, whose weight is exp2(0) = 1).
    for (int t = tid; t < G * D; t += kThreads) {
      const int g = t / D, d = t % D;
      float Mg = kNegInf;
      for (int w = 0; w < kWaves; ++w) Mg = fmaxf(Mg, ml_sh[w][0][g]);
      const float bg = Mg == kNegInf ? 0.f : Mg;
      float Ls = 0.f;
      for (int w = 0; w < kWaves; ++w) Ls += ml_sh[w][1][g] * exp2f_fast(ml_sh[w][0][g] - bg);
      const size_t h = (size_t)b * Hq + kv * G + g;
      out[h * D + d] = Ls > 0.f ? obuf[g * D + d] / Ls : 0.f;
      if (lse != nullptr && d == 0) lse[h] = Ls > 0.f ? (bg + __log2f(Ls)) * kLn2 : kNegInf;
    }
    return;
  }
  for (int t = tid; t < G * D; t += kThreads) {
    const int g = t / D, d = t % D;
    float* rec = part + (((size_t)b * Hq + kv * G + g) * nsplit + split) * (D + 2);
    rec[2 + d] = obuf[g * D + d];
    if (d == 0) {
      float Mg = kNegInf;
      for (int w = 0; w < kWaves; ++w) Mg = fmaxf(Mg, ml_sh[w][0][g]);
      const float bg = Mg == kNegInf ? 0.f : Mg;
      float Ls = 0.f;
      for (int w = 0; w < kWaves; ++w) Ls += ml_sh[w][1][g] * exp2f_fast(ml_sh[w][0][g] - bg);
      rec[0] = bg;
      rec[1] = Ls;
    }
  }
}

// Merge the splits of one (sequence, query head) in split order.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    const float* __restrict__ part, const int* __restrict__ n_sel, const int* __restrict__ sel_len,
    const int* __restrict__ cur_len, int Hq, int chunk, int nsplit, float* __restrict__ out,
    float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int total = n_sel[b] + (cur_len[b] - sel_len[b]);
  const int used = total > 0 ? min(nsplit, ceil_div(total, chunk)) : 0;
  const float* rec = part + ((size_t)b * Hq + h) * nsplit * (D + 2);
  float M = kNegInf;
  for (int c = 0; c < used; ++c) M = fmaxf(M, rec[c * (D + 2)]);
  const float base = M == kNegInf ? 0.f : M;
  float Ls = 0.f, A = 0.f;
  for (int c = 0; c < used; ++c) {
    const float w = exp2f_fast(rec[c * (D + 2)] - base);
    Ls += rec[c * (D + 2) + 1] * w;
    A += rec[c * (D + 2) + 2 + d] * w;
  }
  out[((size_t)b * Hq + h) * D + d] = Ls > 0.f ? A / Ls : 0.f;
  if (lse != nullptr && d == 0) lse[(size_t)b * Hq + h] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : kNegInf;
}

static int decode_chunk(int dtype, int D) { return (dtype == 1 && D == 128) ? kDecChunkMfma : kDecChunk; }

int decode_nsplit(int dtype, int D, int max_attend) {
  return ceil_div(max_attend < 1 ? 1 : max_attend, decode_chunk(dtype, D));
}

// Sized for the smaller (vector-path) chunk, so one size serves every path.
size_t decode_workspace_bytes(int B, int Hq, int D, int max_attend) {
  return (size_t)B * Hq * decode_nsplit(0, D, max_attend) * (D + 2) * sizeof(float);
}

template <typename T, int D, int G>
static hipError_t launch_decode_t(const void* q, const void* kp, const void* vp, const int* bt,
                                  int max_pages, int Hkv, const int* idx, int nsel_cap,
                                  const int* n_sel, const int* sel_len, const int* cur_len,
                                  const int* order, int B, float scale_log2, int nsplit, float* part,
                                  float* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL((sparse_decode_kernel<T, D, G>), dim3(nsplit, Hkv, B), dim3(kDecThreads), 0,
                     stream, (const T*)q, (const T*)kp, (const T*)vp, bt, max_pages, Hkv, idx,
                     nsel_cap, n_sel, sel_len, cur_len, order, scale_log2, kDecChunk, nsplit, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(Hkv * G, B), dim3(D), 0, stream, part, n_sel,
                     sel_len, cur_len, Hkv * G, kDecChunk, nsplit, out, lse);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(int G, const void* q, const void* kp, const void* vp,
                                  const int* bt, int max_pages, int Hkv, const int* idx,
                                  int nsel_cap, const int* n_sel, const int* sel_len,
                                  const int* cur_len, const int* order, int B, float scale_log2,
                                  int nsplit, float* part, float* out, float* lse, hipStream_t stream) {
#define S3R_DEC_CASE(GG)                                                                       \
  case GG:                                                                                     \
    return launch_decode_t<T, D, GG>(q, kp, vp, bt, max_pages, Hkv, idx, nsel_cap, n_sel,      \
                                     sel_len, cur_len, order, B, scale_log2, nsplit, part, out, \
                                     lse, stream);
  switch (G) {
    S3R_DEC_CASE(1)
    S3R_DEC_CASE(2)
    S3R_DEC_CASE(4)
    S3R_DEC_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef S3R_DEC_CASE
}

bool decode_supported(int dtype, int D, int G) {
  if (dtype == 1 && D == 128) return G >= 1 && G <= 16;
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

hipError_t launch_sparse_decode(int dtype, int D, int G, const void* q, const void* kp,
                                const void* vp, const int* bt, int max_pages, int Hkv,
                                const int* idx, int nsel_cap, const int* n_sel, const int* sel_len,
                                const int* cur_len, const int* order, int B, float scale, int max_attend,
                                float* out, float* lse, void* ws, hipStream_t stream) {
  const int nsplit = decode_nsplit(dtype, D, max_attend);
  const float sl2 = scale * kLog2e;
  float* part = (float*)ws;
  if (dtype == 1 && D == 128) {
    // At most kDecChunkMfma positions per split, spread evenly over the splits
    // the host bound needs (a multiple of the subtile): 4922 positions become
    // 3 x 1664 rather than 2048 + 2048 + 826.
    const int att = max_attend < 1 ? 1 : max_attend;
    const int ns = ceil_div(att, kDecChunkMfma);
    const int chunk = kDecBalance ? ceil_div(ceil_div(att, ns), kDsub) * kDsub : kDecChunkMfma;
    hipLaunchKernelGGL(sparse_decode_mfma_kernel<kDecMfmaWaves>, dim3(ns, Hkv, B), dim3(kDecMfmaWaves * kWave), 0,
                       stream,
                       (const bf16_t*)q, (const bf16_t*)kp, (const bf16_t*)vp, bt, max_pages, Hkv, G, idx,
                       nsel_cap, n_sel, sel_len, cur_len, order, sl2, chunk, ns, part, out, lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;  // one split writes the output itself
    hipLaunchKernelGGL((decode_combine_kernel<128>), dim3(Hkv * G, B), dim3(128), 0, stream, part, n_sel,
                       sel_len, cur_len, Hkv * G, chunk, ns, out, lse);
    return hipGetLastError();
  }
  if (dtype == 1) {
    if (D == 128)
      return launch_decode_d<bf16_t, 128>(G, q, kp, vp, bt, max_pages, Hkv, idx, nsel_cap, n_sel,
                                          sel_len, cur_len, order, B, sl2, nsplit, part, out, lse, stream);
    return launch_decode_d<bf16_t, 64>(G, q, kp, vp, bt, max_pages, Hkv, idx, nsel_cap, n_sel,
                                       sel_len, cur_len, order, B, sl2, nsplit, part, out, lse, stream);
  }
  if (D == 128)
    return launch_decode_d<float, 128>(G, q, kp, vp, bt, max_pages, Hkv, idx, nsel_cap, n_sel,
                                       sel_len, cur_len, order, B, sl2, nsplit, part, out, lse, stream);
  return launch_decode_d<float, 64>(G, q, kp, vp, bt, max_pages, Hkv, idx, nsel_cap, n_sel,
                                    sel_len, cur_len, order, B, sl2, nsplit, part, out, lse, stream);
}

}  // namespace s3r
