// s3r_verify_attn kernels: dense block verification plus next-round scores.
//
// [news] "Long-context RL training stops waiting on autoregressive rollouts...",
// Interpretation: verification recomputes the proposed block against the
// complete historical KV cache. [listing] "S^3R: Fast and Faithful RL Rollouts
// via Self-Sparse Speculative Decoding", Table 7: verification (T_V) is one
// eager pass over the whole cache. [explainer] "S3R - Self-sparse speculative
// rollouts for RL - What does it mean?", mechanism paragraph: the selector's
// scores come from the verifier's last attention pass.
//
// Work split: one workgroup per (split, KV head, sequence); a split is a fixed
// chunk of the context (at most 4096 positions on the MFMA path, sized evenly). The (k+1) * G query
// rows of one KV head share every K/V byte read, so each chunk is streamed
// once for all rows.
//
// bf16, head_dim 128 (verify_mfma_kernel): the rows are the N side of
// 16x16x32 bf16 MFMA tiles; a 1-D grid puts consecutive splits of one
// (sequence, KV head) pair on one XCD. Per 32-position subtile a wave
//   - loads K straight from the page into A fragments (16 B per lane) and
//     computes S^T = K Q^T (positions x rows) with Q^T resident in registers
//     (read from LDS for three row tiles, see kVerQLds);
//   - keeps the online-softmax state per row in the lanes that hold that row
//     (lane % 16), so row rescales are lane-local;
//   - writes the probabilities (relative to the running row maximum, fp16)
//     and that maximum as score partials;
//   - transposes its V subtile through LDS (ds_write_b64 of 4 positions,
//     ds_read_b128 of 8 slots) and accumulates O^T += V^T P^T on MFMA, with P
//     already in B-fragment layout (the position order inside the contraction
//     is permuted consistently for P and V).
// The four waves of a workgroup take alternate subtiles and merge their
// states through LDS at the end of the split.
//
// Other dtypes / head_dim 64 (verify_generic_kernel): a plain per-row kernel
// that re-reads the (cache-resident) chunk for each row; correctness path.
//
// verify_finalize_kernel merges the splits per row (log-sum-exp weights, split
// order) and turns the score partials into normalised probabilities summed
// over the rows; its output-row blocks and score blocks can run as one launch
// or, for s3r_verify_attn_deferred + s3r_verify_scores, as two. Splits meet
// at a kernel boundary: merging inside the main kernel (by the last split to
// arrive, or by splits that exchange row statistics and keep their
// probabilities on chip) measured slower on this part.

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kVerThreads = 256;
constexpr int kVerWaves = kVerThreads / kWave;
constexpr int kSub = 32;         // positions per subtile (two pages)
constexpr int kVtStride = 40;    // LDS row stride (uint16) of a transposed V subtile: 32 slots + pad

// Floats per tile in the row-maxima record. Rounded up to whole 128 B lines
// when that adds at most 12 floats, so no two tiles share a line and every
// line is written whole: lines written in parts by different waves cost
// more, but so do the padding bytes (measured at the 24K workload: R = 20
// and 28 faster padded, R = 12, 14 and 36 faster packed).
__host__ __device__ __forceinline__ int max_stride(int R) {
  const int padded = (R + 31) & ~31;
  return padded - R <= 12 ? padded : R;
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t u4_word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int NT, bool QL>
__global__ __launch_bounds__(kVerThreads, (NT <= 2 || QL) ? 2 : 1) void verify_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp,
    const int* __restrict__ bt, int max_pages, int npairs, int Hkv, int G,
    const int* __restrict__ seq_len, int k, float scale_log2, int chunk, int nsplit, int ntile_cap,
    int with_scores, float* __restrict__ part_o, float* __restrict__ part_ml,
    _Float16* __restrict__ sc_val, float* __restrict__ sc_max) {
  constexpr int D = 128;
  constexpr int RP = 16 * NT;
  __shared__ __attribute__((aligned(16))) uint16_t vt[kVerWaves][D * kVtStride];
  __shared__ float ml_sh[kVerWaves][2][RP];
  __shared__ int pages_sh[kVerChunkMfma / kPage];
  // QL: Q rows as B fragments, slot (nt, kk, lane) = row nt*16 + lane%16,
  // elements kk*32 + 8*(lane/16) .. +8 (zero rows past R)
  __shared__ uint4 q_sh[QL ? NT * 4 * 64 : 1];

  // Workgroups are dispatched round-robin over the XCDs; consecutive splits of
  // one (sequence, KV head) pair go to the same XCD. Draft step j of a round
  // visits the sequences backwards when j is odd, so after k draft steps the
  // last sequence was read last when k is even: the pairs are then taken from
  // the last, and the first workgroups may find their pages in the Infinity
  // Cache.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int pair0 = (local / nsplit) * 8 + xcd, split = local % nsplit;
  if (pair0 >= npairs) return;
  const int pair = (kVerFollowDraft && !(k & 1)) ? npairs - 1 - pair0 : pair0;
  const int b = pair / Hkv, kv = pair % Hkv;
  const int S = seq_len[b];
  // `chunk` is the most positions a split holds; each sequence spreads its
  // ceil(S / chunk) splits evenly (a multiple of the subtile)
  const int ch = kVerBalance ? ceil_div(ceil_div(S, ceil_div(S, chunk)), kSub) * kSub : chunk;
  const int c0 = split * ch;
  if (c0 >= S) return;
  const int c1 = min(S, c0 + ch);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int Hq = Hkv * G;
  const int R = (k + 1) * G;
  const int P0 = S - (k + 1);
  const size_t bkv = (size_t)pair;

  bf16x8_t qf[QL ? 1 : NT][4];
  int row_last[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n16;
    row_last[nt] = r < R ? P0 + r / G : -1;
    if constexpr (!QL) {
      if (r < R) {
        const int i = r / G, h = kv * G + r % G;
        const bf16_t* qp = q + (((size_t)b * (k + 1) + i) * Hq + h) * D + g4 * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[nt][kk] = *reinterpret_cast<const bf16x8_t*>(qp + kk * 32);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[nt][kk] = bf16x8_t{};
      }
    }
  }
  if constexpr (QL) {
    for (int t = tid; t < NT * 4 * 64; t += kVerThreads) {
      const int nt = t >> 8, kk = (t >> 6) & 3, l = t & 63;
      const int r = nt * 16 + (l & 15);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < R) {
        const int i = r / G, h = kv * G + r % G;
        v = *reinterpret_cast<const uint4*>(q + (((size_t)b * (k + 1) + i) * Hq + h) * D + kk * 32 + (l >> 4) * 8);
      }
      q_sh[t] = v;
    }
  }

  float m_run[NT], l_run[NT];
  f32x4_t oacc[NT][8];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[nt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // The chunk's physical pages, read once.
  const int* bt_row = bt + (size_t)b * max_pages;
  const int npg = ceil_div(c1 - c0, kPage);
  for (int t = tid; t < npg; t += kVerThreads) pages_sh[t] = bt_row[(c0 >> 4) + t];
  __syncthreads();
  uint16_t* my_vt = vt[wave];
  const int nsub = ceil_div(c1 - c0, kSub);

  struct Sub {
    bf16x8_t kf[2][4];  // K rows as A fragments: lane (n16 = position in the 16-row tile, g4 = k group)
    uint4 vraw[2][4];   // V rows for the LDS transpose: task = (4 positions a, 8-wide d chunk c)
  };
  auto load_sub = [&](int st, Sub& d) {
    const int pos0 = c0 + st * kSub;
    const int page_a = pages_sh[2 * st];
    const int page_b = (pos0 + 16 < S) ? pages_sh[2 * st + 1] : page_a;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const bf16_t* kb = kp + (((size_t)(pt ? page_b : page_a) * Hkv + kv) * kPage + n16) * D + g4 * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) d.kf[pt][kk] = *reinterpret_cast<const bf16x8_t*>(kb + kk * 32);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int task = lane + 64 * tt;
      const int a = task & 7, c = task >> 3;
      const int page = a < 4 ? page_a : page_b;
      const bf16_t* vb = vp + (((size_t)page * Hkv + kv) * kPage + (a & 3) * 4) * D + c * 8;
#pragma unroll
      for (int v = 0; v < 4; ++v) d.vraw[tt][v] = *reinterpret_cast<const uint4*>(vb + v * D);
    }
  };

  Sub cur;
  if (wave < nsub) load_sub(wave, cur);
  for (int st = wave; st < nsub; st += kVerWaves) {
    const int pos0 = c0 + st * kSub;
    const auto& kf = cur.kf;
    const auto& vraw = cur.vraw;

    // S^T = K Q^T: s[pt][nt][v] is position pos0 + pt*16 + 4*g4 + v, row nt*16 + n16
    f32x4_t s[2][NT];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf[pt][kk], QL ? __builtin_bit_cast(bf16x8_t, q_sh[(nt * 4 + kk) * 64 + lane]) : qf[QL ? 0 : nt][kk],
              acc, 0, 0, 0);
        s[pt][nt] = acc;
      }
    }

    const int tile = pos0 / kSub;
    bf16x8_t pf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = kNegInf;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = pos0 + pt * 16 + 4 * g4 + v;
          float x = s[pt][nt][v] * scale_log2;
          x = p > row_last[nt] ? kNegInf : x;
          s[pt][nt][v] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mn = fmaxf(m_run[nt], mx);
      const float base = mn == kNegInf ? 0.f : mn;
      const float alpha = exp2f_fast(m_run[nt] - base);
      float pv[2][4];
      float psum = 0.f;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[pt][v] = exp2f_fast(s[pt][nt][v] - base);
          psum += pv[pt][v];
        }
      }
      l_run[nt] = l_run[nt] * alpha + psum;
      m_run[nt] = mn;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[nt][dt] *= alpha;
      // B fragment of P^T: slots 0..3 -> first page, 4..7 -> second page
      uint32_t w0 = pack_bf16x2(pv[0][0], pv[0][1]);
      uint32_t w1 = pack_bf16x2(pv[0][2], pv[0][3]);
      uint32_t w2 = pack_bf16x2(pv[1][0], pv[1][1]);
      uint32_t w3 = pack_bf16x2(pv[1][2], pv[1][3]);
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      u32x4_t pw = {w0, w1, w2, w3};
      pf[nt] = __builtin_bit_cast(bf16x8_t, pw);

      const int r = nt * 16 + n16;
      if (with_scores && r < R) {
        _Float16* dst = sc_val + ((bkv * ntile_cap + tile) * R + r) * kSub;
        typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
        f16x4_t h0 = {(_Float16)pv[0][0], (_Float16)pv[0][1], (_Float16)pv[0][2], (_Float16)pv[0][3]};
        f16x4_t h1 = {(_Float16)pv[1][0], (_Float16)pv[1][1], (_Float16)pv[1][2], (_Float16)pv[1][3]};
        *reinterpret_cast<f16x4_t*>(dst + 4 * g4) = h0;
        *reinterpret_cast<f16x4_t*>(dst + 16 + 4 * g4) = h1;
        if (g4 == 0) sc_max[(bkv * ntile_cap + tile) * max_stride(R) + r] = base;
      }
    }

    // V^T into LDS: row d holds 32 slots; slot g*8 + pt*4 + v <- position pt*16 + 4g + v
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
        const uint32_t lo = perm_b32(u4_word(vraw[tt][1], wi), u4_word(vraw[tt][0], wi), sel);
        const uint32_t hi = perm_b32(u4_word(vraw[tt][3], wi), u4_word(vraw[tt][2], wi), sel);
        *reinterpret_cast<uint2*>(my_vt + (c * 8 + e) * kVtStride + slot) = make_uint2(lo, hi);
      }
    }
    wave_lds_sync();  // each lane reads rows written by other lanes
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8_t vfrag = *reinterpret_cast<const bf16x8_t*>(my_vt + (dt * 16 + n16) * kVtStride + g4 * 8);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        oacc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag, pf[nt], oacc[nt][dt], 0, 0, 0);
    }
    if (st + kVerWaves < nsub) load_sub(st + kVerWaves, cur);
  }

  // Merge the waves: rows are lane % 16 (+16 nt); l is a per-lane partial.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    l_run[nt] += __shfl_xor(l_run[nt], 16, kWave);
    l_run[nt] += __shfl_xor(l_run[nt], 32, kWave);
  }
  __syncthreads();
  if (g4 == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ml_sh[wave][0][nt * 16 + n16] = m_run[nt];
      ml_sh[wave][1][nt * 16 + n16] = l_run[nt];
    }
  }
  __syncthreads();
  float* obuf = reinterpret_cast<float*>(&vt[0][0]);  // RP x D floats (fits in the V buffers)
  float fac[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n16;
    float M = kNegInf;
    for (int w = 0; w < kVerWaves; ++w) M = fmaxf(M, ml_sh[w][0][r]);
    const float base = M == kNegInf ? 0.f : M;
    fac[nt] = exp2f_fast(m_run[nt] - base);
  }
  for (int w = 0; w < kVerWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int o = (nt * 16 + n16) * D + dt * 16 + g4 * 4 + v;
            const float val = oacc[nt][dt][v] * fac[nt];
            obuf[o] = (w == 0) ? val : obuf[o] + val;
          }
        }
      }
    }
    __syncthreads();
  }
  const size_t rec = (bkv * nsplit + split) * RP;
  float4* po = reinterpret_cast<float4*>(part_o + rec * D);
  const float4* ob4 = reinterpret_cast<const float4*>(obuf);
  for (int t = tid; t < RP * D / 4; t += kVerThreads) po[t] = ob4[t];
  if (tid < RP) {
    float M = kNegInf;
    for (int w = 0; w < kVerWaves; ++w) M = fmaxf(M, ml_sh[w][0][tid]);
    const float base = M == kNegInf ? 0.f : M;
    float Ls = 0.f;
    for (int w = 0; w < kVerWaves; ++w) Ls += ml_sh[w][1][tid] * exp2f_fast(ml_sh[w][0][tid] - base);
    part_ml[(rec + tid) * 2] = base;
    part_ml[(rec + tid) * 2 + 1] = Ls;
  }

}

// Generic path: one row at a time, two passes over the chunk (max, then
// weights), 16 lanes per position row.
template <typename T, int D>
__global__ __launch_bounds__(kVerThreads) void verify_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ kp, const T* __restrict__ vp,
    const int* __restrict__ bt, int max_pages, int Hkv, int G, const int* __restrict__ seq_len,
    int k, float scale_log2, int chunk, int nsplit, int ntile_cap, int RP, int with_scores,
    float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ sc_val,
    float* __restrict__ sc_max) {
  constexpr int EPL = D / 16;
  constexpr int kStreams = kVerThreads / 16;
  __shared__ float red[kVerWaves][D + 2];
  __shared__ float bc;

  const int split = blockIdx.x, pair = blockIdx.y;
  const int b = pair / Hkv, kv = pair % Hkv;
  const int S = seq_len[b];
  const int c0 = split * chunk;
  if (c0 >= S) return;
  const int c1 = min(S, c0 + chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, sub = lane & 15;
  const int stream = wave * 4 + (lane >> 4);
  const int Hq = Hkv * G, R = (k + 1) * G, P0 = S - (k + 1);
  const size_t bkv = (size_t)pair;
  const int* bt_row = bt + (size_t)b * max_pages;
  const size_t head_stride = (size_t)kPage * D;

  for (int r = 0; r < R; ++r) {
    const int i = r / G, h = kv * G + r % G;
    const int hi = min(c1, P0 + i + 1);
    float qv[EPL];
    const T* qp = q + (((size_t)b * (k + 1) + i) * Hq + h) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = (float)qp[e] * scale_log2;
    auto logit = [&](int j) {
      const size_t off = ((size_t)bt_row[j >> 4] * Hkv + kv) * head_stride + (size_t)(j & 15) * D + sub * EPL;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qv[e], (float)kp[off + e], s);
#pragma unroll
      for (int mask = 1; mask < 16; mask <<= 1) s += __shfl_xor(s, mask, kWave);
      return s;
    };
    float mx = kNegInf;
    for (int j = c0 + stream; j < hi; j += kStreams) mx = fmaxf(mx, logit(j));
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    if (lane == 0) red[wave][0] = mx;
    __syncthreads();
    if (tid == 0) {
      float M = kNegInf;
      for (int w = 0; w < kVerWaves; ++w) M = fmaxf(M, red[w][0]);
      bc = M;
    }
    __syncthreads();
    const float M = bc;
    const float base = M == kNegInf ? 0.f : M;
    float l = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int j = c0 + stream; j < c1; j += kStreams) {
      float p = 0.f;
      if (j < hi) {
        p = exp2f_fast(logit(j) - base);
        const size_t off = ((size_t)bt_row[j >> 4] * Hkv + kv) * head_stride + (size_t)(j & 15) * D + sub * EPL;
        l += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, (float)vp[off + e], acc[e]);
      }
      if (with_scores && sub == 0) sc_val[((bkv * ntile_cap + j / kSub) * R + r) * kSub + (j % kSub)] = p;
    }
    if (with_scores) {
      for (int t = c0 / kSub + tid; t < ceil_div(c1, kSub); t += kVerThreads)
        sc_max[(bkv * ntile_cap + t) * max_stride(R) + r] = base;
    }
    // reduce l and acc over the 16 streams
    __syncthreads();
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc[e] += __shfl_xor(acc[e], 16, kWave);
      acc[e] += __shfl_xor(acc[e], 32, kWave);
    }
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][sub * EPL + e] = acc[e];
      if (sub == 0) red[wave][D] = l;
    }
    __syncthreads();
    const size_t rec = (bkv * nsplit + split) * RP + r;
    for (int d = tid; d < D; d += kVerThreads) {
      float A = 0.f;
      for (int w = 0; w < kVerWaves; ++w) A += red[w][d];
      part_o[rec * D + d] = A;
    }
    if (tid == 0) {
      float Ls = 0.f;
      for (int w = 0; w < kVerWaves; ++w) Ls += red[w][D];
      part_ml[rec * 2] = base;
      part_ml[rec * 2 + 1] = Ls;
    }
    __syncthreads();
  }
}

// Merge the splits of each (sequence, KV head) pair and normalise the score
// partials. Blocks [0, nblk_o) each write 256 outputs of the merged rows;
// the remaining blocks each normalise kFinTiles tiles of score partials.
// Every block first merges the per-split (max, sum) of all rows, in split
// order, so every value is computed the same way by every block.
constexpr int kFinTiles = kVerThreads / (kSub / 4);  // score tiles per finalize block (4 positions per thread)

template <typename VT, int D>
__global__ __launch_bounds__(kVerThreads) void verify_finalize_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, const VT* __restrict__ sc_val,
    const float* __restrict__ sc_max, const int* __restrict__ seq_len, int k, int Hkv, int G, int chunk,
    int nsplit, int ntile_cap, int RP, int nblk_o, int x0, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ scores, int score_stride) {
  __shared__ float mrow[64], lrow[64], l2row[64];
  __shared__ float wt[kFinTiles][64];
  const int pair = blockIdx.y, tid = threadIdx.x;
  const int b = pair / Hkv, kv = pair % Hkv;
  const int S = seq_len[b];
  const int x = x0 + (int)blockIdx.x;
  const int tile_beg = (x - nblk_o) * kFinTiles;
  if (x >= nblk_o && tile_beg * kSub >= S) return;
  const int used = min(nsplit, ceil_div(S, chunk));
  const int R = (k + 1) * G, Hq = Hkv * G;
  const size_t bkv = (size_t)pair;
  // Row statistics: 4 lanes per row, each over every 4th split, then a fixed
  // butterfly over the 4 lanes (same order in every block).
  for (int r0 = 0; r0 < R; r0 += kVerThreads / 4) {
    const int r = r0 + tid / 4, c4 = tid & 3;
    float m = kNegInf, l = 0.f;
    if (r < R) {
      for (int c = c4; c < used; c += 4) m = fmaxf(m, part_ml[((bkv * nsplit + c) * RP + r) * 2]);
    }
    m = fmaxf(m, __shfl_xor(m, 1, kWave));
    m = fmaxf(m, __shfl_xor(m, 2, kWave));
    const float base = m == kNegInf ? 0.f : m;
    if (r < R) {
      for (int c = c4; c < used; c += 4) {
        const size_t rc = (bkv * nsplit + c) * RP + r;
        l += part_ml[rc * 2 + 1] * exp2f_fast(part_ml[rc * 2] - base);
      }
    }
    l += __shfl_xor(l, 1, kWave);
    l += __shfl_xor(l, 2, kWave);
    if (r < R && c4 == 0) {
      mrow[r] = base;
      lrow[r] = l;
      l2row[r] = base + __log2f(l);
    }
  }
  __syncthreads();
  if (x < nblk_o) {
    const int t = x * kVerThreads + tid;
    if (t < R * D) {
      const int r = t / D, d = t % D;
      float A = 0.f;
      for (int c = 0; c < used; ++c) {
        const size_t rc = (bkv * nsplit + c) * RP + r;
        A += part_o[rc * D + d] * exp2f_fast(part_ml[rc * 2] - mrow[r]);
      }
      const int i = r / G, h = kv * G + r % G;
      out[(((size_t)b * (k + 1) + i) * Hq + h) * D + d] = A / lrow[r];
      if (lse != nullptr && d == 0) lse[((size_t)b * (k + 1) + i) * Hq + h] = l2row[r] * kLn2;
    }
    return;
  }
  const int ntiles = ceil_div(S, kSub);
  const int tile_end = min(ntiles, tile_beg + kFinTiles);
  // weights of every (tile, row) of this block, then 4 positions per thread
  for (int e = tid; e < kFinTiles * R; e += kVerThreads) {
    const int et = e / R, r = e % R, tile = tile_beg + et;
    wt[et][r] = tile < tile_end ? exp2f_fast(sc_max[(bkv * ntile_cap + tile) * max_stride(R) + r] - l2row[r]) : 0.f;
  }
  __syncthreads();
  const int tl = tid / (kSub / 4), j4 = (tid % (kSub / 4)) * 4;
  const int tile = tile_beg + tl, pos = tile * kSub + j4;
  if (tile < tile_end && pos < S) {
    const VT* vals = sc_val + (bkv * ntile_cap + tile) * R * kSub + j4;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int r = 0; r < R; ++r) {
      const float w = wt[tl][r];
      const VT* v = vals + r * kSub;
      a0 = fmaf(w, (float)v[0], a0);
      a1 = fmaf(w, (float)v[1], a1);
      a2 = fmaf(w, (float)v[2], a2);
      a3 = fmaf(w, (float)v[3], a3);
    }
    float* dst = scores + bkv * score_stride + pos;
    dst[0] = a0;
    if (pos + 1 < S) dst[1] = a1;
    if (pos + 2 < S) dst[2] = a2;
    if (pos + 3 < S) dst[3] = a3;
  }
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

VerifyPlan verify_plan(int B, int k, int Hq, int Hkv, int D, int dtype, int max_seq_len) {
  VerifyPlan p;
  p.G = Hq / Hkv;
  p.R = (k + 1) * p.G;
  p.mfma = (dtype == 1 && D == 128);
  p.NT = ceil_div(p.R, 16);
  p.RP = 16 * p.NT;
  // MFMA path: at most kVerChunkMfma positions per split; the kernel spreads
  // each sequence's splits evenly (24583 positions: 7 x 3520 rather than
  // 6 x 4096 + 7). The split count of a sequence, ceil(S / chunk), is the
  // same either way.
  p.chunk = p.mfma ? kVerChunkMfma : kVerChunkGeneric;
  p.nsplit = ceil_div(max_seq_len, p.chunk);
  p.ntile_cap = ceil_div(max_seq_len, kSub);
  // Partial records per (sequence, KV head) pair.
  const size_t nbkv = (size_t)B * Hkv;
  size_t off = 0;
  p.off_part_o = off;
  off = align256(off + nbkv * p.nsplit * p.RP * D * sizeof(float));
  p.off_part_ml = off;
  off = align256(off + nbkv * p.nsplit * p.RP * 2 * sizeof(float));
  p.off_sc_max = off;
  off = align256(off + nbkv * p.ntile_cap * max_stride(p.R) * sizeof(float));
  p.off_sc_val = off;
  off = align256(off + nbkv * p.ntile_cap * p.R * kSub * (p.mfma ? sizeof(_Float16) : sizeof(float)));
  p.bytes = off;
  return p;
}

template <int NT>
static void launch_mfma(const VerifyPlan& p, const void* q, const void* kp, const void* vp,
                        const int* bt, int max_pages, int Hkv, const int* seq_len, int npairs, int k,
                        float sl2, int with_scores, char* ws, hipStream_t stream) {
  const int nblocks = ceil_div(npairs, 8) * 8 * p.nsplit;
  hipLaunchKernelGGL((verify_mfma_kernel<NT, kVerQLds && NT == 3>), dim3(nblocks), dim3(kVerThreads), 0, stream,
                     (const bf16_t*)q, (const bf16_t*)kp, (const bf16_t*)vp, bt, max_pages, npairs, Hkv,
                     p.G, seq_len, k, sl2, p.chunk, p.nsplit, p.ntile_cap, with_scores,
                     (float*)(ws + p.off_part_o), (float*)(ws + p.off_part_ml),
                     (_Float16*)(ws + p.off_sc_val), (float*)(ws + p.off_sc_max));
}

// Finalize blocks [x0, x0 + nx) of the (output rows | score tiles) range.
static hipError_t launch_finalize(const VerifyPlan& p, int D, const int* seq_len, int npairs, int k,
                                  int Hkv, int x0, int nx, float* out, float* lse, float* scores,
                                  int score_stride, const char* ws, hipStream_t stream) {
  if (nx <= 0) return hipSuccess;
  const int nblk_o = ceil_div(p.R * D, kVerThreads);
  const dim3 grid(nx, npairs);
#define S3R_FIN(VT, DD)                                                                              \
  hipLaunchKernelGGL((verify_finalize_kernel<VT, DD>), grid, dim3(kVerThreads), 0, stream,          \
                     (const float*)(ws + p.off_part_o), (const float*)(ws + p.off_part_ml),          \
                     (const VT*)(ws + p.off_sc_val), (const float*)(ws + p.off_sc_max), seq_len, k,  \
                     Hkv, p.G, p.chunk, p.nsplit, p.ntile_cap, p.RP, nblk_o, x0, out, lse, scores,   \
                     score_stride)
  if (p.mfma) {
    S3R_FIN(_Float16, 128);
  } else if (D == 128) {
    S3R_FIN(float, 128);
  } else {
    S3R_FIN(float, 64);
  }
#undef S3R_FIN
  return hipGetLastError();
}

hipError_t launch_verify(int dtype, int D, const void* q, const void* kp, const void* vp,
                         const int* bt, int max_pages, int Hkv, const int* seq_len, int B, int k,
                         int Hq, float scale, int max_seq_len, float* out, float* lse,
                         float* scores, int score_stride, bool defer_scores, void* ws_v,
                         hipStream_t stream) {
  const VerifyPlan p = verify_plan(B, k, Hq, Hkv, D, dtype, max_seq_len);
  char* ws = (char*)ws_v;
  const float sl2 = scale * kLog2e;
  const int with_scores = (scores != nullptr || defer_scores) ? 1 : 0;
  const int npairs = B * Hkv;
  if (p.mfma) {
#define S3R_MFMA(NTV) \
  launch_mfma<NTV>(p, q, kp, vp, bt, max_pages, Hkv, seq_len, npairs, k, sl2, with_scores, ws, stream)
    switch (p.NT) {
      case 1: S3R_MFMA(1); break;
      case 2: S3R_MFMA(2); break;
      case 3: S3R_MFMA(3); break;
      case 4: S3R_MFMA(4); break;
      default: return hipErrorInvalidValue;
    }
#undef S3R_MFMA
  } else {
#define S3R_GEN(TT, DD)                                                                               \
  hipLaunchKernelGGL((verify_generic_kernel<TT, DD>), dim3(p.nsplit, npairs), dim3(kVerThreads), 0,  \
                     stream, (const TT*)q, (const TT*)kp, (const TT*)vp, bt, max_pages, Hkv, p.G,    \
                     seq_len, k, sl2, p.chunk, p.nsplit, p.ntile_cap, p.RP, with_scores,              \
                     (float*)(ws + p.off_part_o), (float*)(ws + p.off_part_ml),                       \
                     (float*)(ws + p.off_sc_val), (float*)(ws + p.off_sc_max))
    if (dtype == 1) {
      if (D == 128) S3R_GEN(BF16Val, 128); else S3R_GEN(BF16Val, 64);
    } else {
      if (D == 128) S3R_GEN(float, 128); else S3R_GEN(float, 64);
    }
#undef S3R_GEN
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk_o = ceil_div(p.R * D, kVerThreads);
  const int nblk_s = (scores != nullptr && !defer_scores) ? ceil_div(p.ntile_cap, kFinTiles) : 0;
  return launch_finalize(p, D, seq_len, npairs, k, Hkv, 0, nblk_o + nblk_s, out, lse,
                         defer_scores ? nullptr : scores, score_stride, ws, stream);
}

hipError_t launch_verify_scores(int dtype, int D, const int* seq_len, int B, int k, int Hq, int Hkv,
                                int max_seq_len, float* scores, int score_stride, const void* ws,
                                hipStream_t stream) {
  const VerifyPlan p = verify_plan(B, k, Hq, Hkv, D, dtype, max_seq_len);
  const int nblk_o = ceil_div(p.R * D, kVerThreads);
  return launch_finalize(p, D, seq_len, B * Hkv, k, Hkv, nblk_o, ceil_div(p.ntile_cap, kFinTiles), nullptr,
                         nullptr, scores, score_stride, (const char*)ws, stream);
}

}  // namespace s3r
