// s3r_verify_attn kernels: dense block verification plus next-round scores.
//
// [news] "Long-context RL training stops waiting on autoregressive rollouts...",
// Interpretation: verification recomputes the proposed block against the
// complete historical KV cache. [listing] "S^3R: Fast and Faithful RL Rollouts
// via Self-Sparse Speculative Decoding", Table 7: verification (T_V) is one
// eager pass over the whole cache. [explainer] "S3R - Self-sparse speculative
// rollouts for RL - What does it mean?", mechanism paragraph: what the
// selector ranks is the attention the previous verification paid to each
// position.
//
// Work split: one workgroup per (split, KV head, sequence); a split is a fixed
// chunk of the context (at most 4096 positions on the MFMA path, sized evenly). The (k+1) * G query
// rows of one KV head share every K/V byte read, so each chunk is streamed
// once for all rows.
//
// bf16, head_dim 128 (verify_mfma_kernel): the rows are the N side of
// 16x16x32 bf16 MFMA tiles; a 1-D grid puts consecutive splits of one
// (sequence, KV head) pair on one XCD. Per 32-position subtile a wave
//   - loads each page's K block with whole lines per instruction (1 KB per
//     wave), reshapes it into A fragments through its LDS buffer, and
//     computes S^T = K Q^T (positions x rows) with Q^T resident in registers
//     (read from LDS for three row tiles, see kVerQLds);
//   - keeps the online-softmax state per row in the lanes that hold that row
//     (lane % 16), so row rescales are lane-local;
//   - writes the probabilities (relative to the running row maximum, as
//     12-bit codes of the bf16 values that also weight V) and that maximum
//     as score partials;
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

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kVerThreads = 256;
constexpr int kVerWaves = kVerThreads / kWave;
constexpr int kSub = 32;         // positions per subtile (two pages)
constexpr int kVtStride = 40;    // LDS row stride (uint16) of a transposed V subtile: 32 slots + pad
// The running reference maximum of a row is raised only when a logit exceeds
// it by more than this (log2 units): probabilities stay below 2^8.
constexpr float kLazyRescale = 8.f;

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

// Position score partials are 12-bit codes of the bf16 probabilities that
// weight V (so the scores carry the precision the output does): the bf16 bit
// pattern less kCodeBias, i.e. a 5-bit exponent spanning 2^-23 .. 2^9 over
// the 7 mantissa bits. The probabilities lie in [0, 2^kLazyRescale], so the
// codes stay below 4096; anything at or below 2^-23 becomes code 0, which
// stands for zero. A lane's eight probabilities of a subtile (four positions
// on each of its pages) pack into three words, code i at bits 12 i.
constexpr uint32_t kCodeBias = 0x3400u;  // bf16 pattern of 2^-23
constexpr int kCodeWords = kSub * 12 / 32;  // words per (subtile, row) record
// Records are grouped by 16 consecutive tiles: group, then row, then the 16
// tiles' records side by side, so a finalize wave (8 tiles of a group; lane =
// tile, lane group, page) reads each row's records of its tiles as one
// contiguous run.
constexpr int kCodeGroup = 16;
__host__ __device__ __forceinline__ size_t code_record(size_t bkv, int ngrp, int R, int tile, int r) {
  return ((bkv * ngrp + (tile >> 4)) * R + r) * (kCodeGroup * kCodeWords) + (tile & 15) * kCodeWords;
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t codes_of_pair(uint32_t w) {
  u16x2_t h = __builtin_bit_cast(u16x2_t, w);
  h = __builtin_elementwise_sub_sat(h, u16x2_t{(unsigned short)kCodeBias, (unsigned short)kCodeBias});
  h = __builtin_elementwise_min(h, u16x2_t{4095, 4095});
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void pack_codes(const bf16x8_t& p, uint32_t& w0, uint32_t& w1, uint32_t& w2) {
  const uint4 b = __builtin_bit_cast(uint4, p);
  const uint32_t d0 = codes_of_pair(b.x), d1 = codes_of_pair(b.y);  // (c1, c0), (c3, c2)
  const uint32_t d2 = codes_of_pair(b.z), d3 = codes_of_pair(b.w);  // (c5, c4), (c7, c6)
  w0 = (d0 & 0xfffu) | ((d0 >> 4) & 0xfff000u) | (d1 << 24);
  w1 = ((d1 >> 8) & 0xfu) | (d1 >> 12) | (d2 << 16 & 0xfff0000u) | (d2 >> 16 << 28);
  w2 = (d2 >> 20) | ((d3 & 0xfffu) << 8) | ((d3 >> 16) << 20);
}

// Decoding: the code shifted to bits 16..27 is a float of the probability
// times 2^-104 (exponent field 0x68 lower), so the finalize folds 2^104 into
// its row weight and needs a mask per code. Codes below 128 (probabilities
// under 2^-22 of the reference maximum) land in the denormal range and come
// out within 2^-22 of their value; code 0 is 0.
constexpr float kCodeScaleLog2 = 104.f;

// Page records are gathered in LDS (and written as bf16) for up to two row
// tiles; with three the LDS already holds the Q fragments, with four the
// buffer would take 64 KB, and they go out as floats as they are formed.
__host__ __device__ constexpr bool page_records_bf16(int NT) { return NT <= 2 && kVerPageBurst; }

// Score partials the split kernel writes (SM): none; per position (coded
// probabilities relative to the row's reference maximum, plus that maximum per
// tile); or per page (the page's probability mass in the row: bf16 relative
// to the split's row base, or its float log2 beyond two row tiles).
constexpr int kScoresNone = 0, kScoresPositions = 1, kScoresPages = 2;

template <int NT, bool QL, int SM>
__global__ __launch_bounds__(kVerThreads, (NT <= 2 || QL) ? 2 : 1) void verify_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp,
    const int* __restrict__ bt, int max_pages, int npairs, int Hkv, int G,
    const int* __restrict__ seq_len, int k, float scale_log2, int chunk, int nsplit, int ntile_cap,
    float* __restrict__ part_o, float* __restrict__ part_ml, void* __restrict__ sc_val,
    float* __restrict__ sc_max) {
  constexpr int D = 128;
  constexpr int RP = 16 * NT;
  __shared__ __attribute__((aligned(16))) uint16_t vt[kVerWaves][D * kVtStride];
  __shared__ float ml_sh[kVerWaves][2][RP];
  __shared__ int pages_sh[kVerChunkMfma / kPage];
  // QL: Q rows as B fragments, slot (nt, kk, lane) = row nt*16 + lane%16,
  // elements kk*32 + 8*(lane/16) .. +8 (zero rows past R)
  __shared__ uint4 q_sh[QL ? NT * 4 * 64 : 1];
  // Page scores with at most two row tiles: the split's page masses are
  // gathered here and written out at the end of the split, in one contiguous
  // burst and as bf16 relative to the split's row bases (scattered 256 B
  // writes during the stream cost far more).
  constexpr bool PB = SM == kScoresPages && page_records_bf16(NT);
  __shared__ __attribute__((aligned(16))) float pbuf[PB ? (kVerChunkMfma / kPage) * RP : 1];
  // Position scores: the partials of a group of kPosGroup consecutive
  // subtiles (probability codes and row maxima) are gathered here and written
  // out once the group is done, each row's records as one run. (Eight
  // subtiles with three row tiles, whose Q fragments also sit in LDS, so two
  // workgroups still fit a CU.)
  constexpr bool QB = SM == kScoresPositions && kVerPosBurst;
  constexpr int kPosGroup = NT <= 2 ? 16 : 8;
  __shared__ __attribute__((aligned(16))) uint32_t qbuf[QB ? RP * kPosGroup * kCodeWords : 1];  // [row][slot]
  __shared__ __attribute__((aligned(16))) float qmax[QB ? kPosGroup * RP : 1];

  // Workgroups are dispatched round-robin over the XCDs; consecutive splits of
  // one (sequence, KV head) pair go to the same XCD.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int pair0 = (local / nsplit) * 8 + xcd, split = local % nsplit;
  if (pair0 >= npairs) return;
  const int pair = pair0;
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
  const int ngrp = ceil_div(ntile_cap, kCodeGroup);

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
    bf16x8_t kf[2][4];  // K chunks as loaded: page pt, chunk 64 i + lane of its 4 KB block
    uint4 vraw[2][4];   // V rows for the LDS transpose: task = (4 positions a, 8-wide d chunk c)
  };
  auto sub_pages = [&](int st, int& page_a, int& page_b) {
    page_a = pages_sh[2 * st];
    page_b = (c0 + st * kSub + 16 < S) ? pages_sh[2 * st + 1] : page_a;
  };
  // K: each page's 4 KB block with 1 KB contiguous per wave instruction
  // (whole lines; ordinary loads), reshaped into the operand fragments through
  // LDS at the start of the subtile. V: nontemporal loads (8 rows x 128 B per
  // instruction, read once).
  auto load_k = [&](int st, Sub& d) {
    int page_a, page_b;
    sub_pages(st, page_a, page_b);
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const bf16_t* kb = kp + ((size_t)(pt ? page_b : page_a) * Hkv + kv) * kPage * D + lane * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) d.kf[pt][i] = *reinterpret_cast<const bf16x8_t*>(kb + i * 512);
    }
  };
  auto load_v = [&](int st, Sub& d) {
    int page_a, page_b;
    sub_pages(st, page_a, page_b);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int task = lane + 64 * tt;
      const int a = task & 7, c = task >> 3;
      const int page = a < 4 ? page_a : page_b;
      const bf16_t* vb = vp + (((size_t)page * Hkv + kv) * kPage + (a & 3) * 4) * D + c * 8;
#pragma unroll
      for (int v = 0; v < 4; ++v) d.vraw[tt][v] = load_nt16_u4(vb + v * D);
    }
  };

  Sub cur;
  if (wave < nsub) {
    load_k(wave, cur);
    load_v(wave, cur);
  }
  // One subtile. EDGE: some position of it lies past some row's last one (the
  // block's causal triangle, the end of the sequence), so the logits are
  // masked; every row sees all positions of the earlier subtiles. (Rows past R
  // then see logits 0 of their zero queries: they are never read.) The two
  // forms are separate code, so the common one carries no mask arithmetic.
  auto subtile = [&](int st, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int pos0 = c0 + st * kSub;
    const auto& vraw = cur.vraw;
    // K through the wave's LDS buffer: the chunks go in as loaded (row
    // 16 pt + 4 i + lane / 16, 16 B chunk lane % 16; rows padded to 272 B so
    // the fragment reads of 16 rows hit distinct banks), the A fragments come
    // out: lane (n16 = position in the 16-row tile, g4 = k group)
    constexpr int kKStride = D + 8;
    static_assert(2 * kPage * kKStride <= D * kVtStride, "K subtile exceeds the wave's LDS buffer");
    wave_lds_sync();  // the previous subtile's reads of the buffer precede these writes
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<bf16x8_t*>(my_vt + (pt * 16 + i * 4 + (lane >> 4)) * kKStride + (lane & 15) * 8) =
            cur.kf[pt][i];
    wave_lds_sync();  // each lane reads rows written by other lanes
    bf16x8_t kf[2][4];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kf[pt][kk] = *reinterpret_cast<const bf16x8_t*>(my_vt + (pt * 16 + n16) * kKStride + kk * 32 + g4 * 8);

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
    // The K fragments are consumed: the wave's next subtile's K loads go out
    // now, so they are in flight during the rest of this subtile. (The last
    // subtile of a wave reloads itself from the cache instead, so every path
    // through the loop issues the same loads and the wait at the top of the
    // next subtile covers only its K loads.)
    const int st_next = st + kVerWaves < nsub ? st + kVerWaves : st;
    if (kVerEarlyLoads) {
      load_k(st_next, cur);
      pin_issued_loads();
    }

    const int tile = pos0 / kSub;
    bf16x8_t pf[NT];
    float pmass[NT];  // page masses of this lane's rows (page scores)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = kNegInf;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x = s[pt][nt][v] * scale_log2;
          if constexpr (EDGE) x = pos0 + pt * 16 + 4 * g4 + v > row_last[nt] ? kNegInf : x;
          s[pt][nt][v] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      // The probabilities are relative to a reference maximum m_run that is
      // raised only when a row's logit exceeds it by more than kLazyRescale
      // (log2 units), so they stay below 2^kLazyRescale and the rescale of the
      // accumulators is skipped in nearly every subtile (a wave-uniform test).
      // Rows without a finite logit so far keep -inf (their sums are 0).
      if (__any(mx > m_run[nt] + kLazyRescale)) {
        const float mn = mx > m_run[nt] + kLazyRescale ? mx : m_run[nt];
        const float alpha = m_run[nt] == kNegInf ? 0.f : exp2f_fast(m_run[nt] - mn);
        l_run[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[nt][dt] *= alpha;
        m_run[nt] = mn;
      }
      const float base = m_run[nt] == kNegInf ? 0.f : m_run[nt];
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
      l_run[nt] += psum;
      // B fragment of P^T: slots 0..3 -> first page, 4..7 -> second page
      // (bf16, round to nearest even)
      pf[nt] = bf16x8_t{(__bf16)pv[0][0], (__bf16)pv[0][1], (__bf16)pv[0][2], (__bf16)pv[0][3],
                        (__bf16)pv[1][0], (__bf16)pv[1][1], (__bf16)pv[1][2], (__bf16)pv[1][3]};

      const int r = nt * 16 + n16;
      if constexpr (SM == kScoresPositions) {
        // record (tile, row): kCodeWords words, lane group g4 at word 3 g4
        if (r < R) {
          uint32_t w0, w1, w2;
          pack_codes(pf[nt], w0, w1, w2);
          uint32_t* dst = QB ? qbuf + (r * kPosGroup + st % kPosGroup) * kCodeWords + 3 * g4
                             : static_cast<uint32_t*>(sc_val) + code_record(bkv, ngrp, R, tile, r) + 3 * g4;
          dst[0] = w0;
          dst[1] = w1;
          dst[2] = w2;
          if (g4 == 0) {
            if constexpr (QB) qmax[(st % kPosGroup) * RP + r] = base;
            else sc_max[(bkv * ntile_cap + tile) * max_stride(R) + r] = base;
          }
        }
      } else if constexpr (SM == kScoresPages) {
        // Each of the subtile's two pages: the row's probability mass on it (the
        // four lane groups' sums in a fixed order), kept as base + log2(mass)
        // (-inf for none); lanes of group 0 keep page 2 tile, group 1 page
        // 2 tile + 1.
        float pa = (pv[0][0] + pv[0][1]) + (pv[0][2] + pv[0][3]);
        float pb = (pv[1][0] + pv[1][1]) + (pv[1][2] + pv[1][3]);
        pa += __shfl_xor(pa, 16, kWave);
        pb += __shfl_xor(pb, 16, kWave);
        pa += __shfl_xor(pa, 32, kWave);
        pb += __shfl_xor(pb, 32, kWave);
        pmass[nt] = base + __log2f(g4 == 0 ? pa : pb);
      }
    }
    if constexpr (SM == kScoresPages) {
      // One store per subtile: a page's record holds row nt * 16 + n at float
      // n * NT + nt, so each lane writes its NT rows as one vector and the two
      // pages' records (RP floats each, adjacent) are written as whole lines.
      const int page = 2 * tile + g4;
      if (PB && g4 < 2) {
        float* dst = pbuf + (2 * st + g4) * RP + n16 * NT;
        if constexpr (NT == 1) dst[0] = pmass[0];
        else *reinterpret_cast<float2*>(dst) = make_float2(pmass[0], pmass[NT - 1]);
      } else if (!PB && g4 < 2 && page * kPage < S) {
        float* dst = static_cast<float*>(sc_val) + (bkv * 2 * ntile_cap + page) * RP + n16 * NT;
        if constexpr (NT == 1) {
          dst[0] = pmass[0];
        } else if constexpr (NT == 2) {
          *reinterpret_cast<float2*>(dst) = make_float2(pmass[0], pmass[1]);
        } else if constexpr (NT == 3) {
          typedef float f32x3_t __attribute__((ext_vector_type(3)));
          *reinterpret_cast<f32x3_t*>(dst) = f32x3_t{pmass[0], pmass[1], pmass[2]};
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(pmass[0], pmass[1], pmass[2], pmass[3]);
        }
      }
    }

    // The sequence's last subtile: slots at and past S hold whatever the cache
    // pool holds there. Their probabilities are 0, but 0 * NaN or 0 * Inf is NaN
    // in the contraction below, so their V words are cleared. (Their K rows only
    // reach logits that the causal mask above replaces by -inf.)
    if (EDGE && pos0 + kSub > S) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int a = (lane + 64 * tt) & 7;
        const int first = pos0 + (a >> 2) * 16 + (a & 3) * 4;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (first + v >= S) cur.vraw[tt][v] = make_uint4(0u, 0u, 0u, 0u);
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
    // The V words are in LDS: the next subtile's V loads go out now.
    if (kVerEarlyLoads) {
      load_v(st_next, cur);
      pin_issued_loads();
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
    if (!kVerEarlyLoads && st + kVerWaves < nsub) {
      load_k(st + kVerWaves, cur);
      load_v(st + kVerWaves, cur);
    }
  };
  auto run_subtile = [&](int st) {
    if (!kVerSplitEdge || c0 + st * kSub + kSub - 1 > P0)
      subtile(st, std::true_type{});
    else
      subtile(st, std::false_type{});
  };
  if constexpr (QB) {
    // groups of kPosGroup subtiles; after each, the group's partials go out
    // (a row's records of consecutive tiles are contiguous within a group of
    // kCodeGroup tiles; the maxima records are max_stride(R) floats per tile)
    const int tile0 = c0 / kSub;
    const int ms = max_stride(R);
    for (int g0 = 0; g0 < nsub; g0 += kPosGroup) {
      const int gn = min(kPosGroup, nsub - g0);
      for (int st = g0 + wave; st < g0 + gn; st += kVerWaves) run_subtile(st);
      __syncthreads();
      // 16 B chunks of codes, row-major over (row, tile) so neighbouring
      // threads write neighbouring tiles of a row; nontemporal stores, since
      // the finalize reads them only after the rest of the split pass
      uint32_t* pd = static_cast<uint32_t*>(sc_val);
      constexpr int kChunks = kCodeWords / 4;
      for (int t = tid; t < R * gn * kChunks; t += kVerThreads) {
        const int part = t % kChunks, rt = t / kChunks, r = rt / gn, tl = rt % gn;
        store_nt16(pd + code_record(bkv, ngrp, R, tile0 + g0 + tl, r) + 4 * part,
                   *reinterpret_cast<const u32x4_t*>(qbuf + (r * kPosGroup + tl) * kCodeWords + 4 * part));
      }
      for (int t = tid; t < gn * R; t += kVerThreads) {
        const int tl = t / R, r = t % R;
        __builtin_nontemporal_store(qmax[tl * RP + r], sc_max + (bkv * ntile_cap + tile0 + g0 + tl) * ms + r);
      }
      __syncthreads();
    }
  } else {
    for (int st = wave; st < nsub; st += kVerWaves) run_subtile(st);
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
  if constexpr (PB) {
    // The split's page records, pages [c0 / 16, ceil(c1 / 16)), written as one
    // run once the split's row bases are known: per page RP bf16 slots in row
    // order, each the page's probability mass relative to the base the split's
    // (m, l) record carries (at most 2^12: 16 positions below 2^8 each), two
    // rows a word. A thread keeps one pair of rows (kVerThreads is a multiple
    // of RP / 2).
    const int cw = tid % (RP / 2);
    float bse[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 2 * cw + h;
      float M = kNegInf;
      for (int w = 0; w < kVerWaves; ++w) M = fmaxf(M, ml_sh[w][0][r]);
      bse[h] = M == kNegInf ? 0.f : M;
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(sc_val) + (bkv * 2 * ntile_cap + c0 / kPage) * RP);
    const int nw = ceil_div(c1 - c0, kPage) * RP / 2;
    for (int t = tid; t < nw; t += kVerThreads) {
      const int pl = t / (RP / 2);
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 2 * cw + h;
        v[h] = r < R ? exp2f_fast(pbuf[pl * RP + (r & 15) * NT + (r >> 4)] - bse[h]) : 0.f;
      }
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      dst[t] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)v[0], (__bf16)v[1]});
    }
  }
  // The waves' output accumulators are summed in LDS (the V buffers, free
  // now), rows padded to OS floats so that the 16 rows a wave writes at one
  // column fall in distinct banks. Up to two row tiles there is room for two
  // buffers: waves 0 and 1 write them, waves 2 and 3 add into them, and their
  // sum goes out ((w0 + w2) + (w1 + w3)); with more, one buffer and the waves
  // in turn. Only the R real rows are written to the split's record.
  constexpr int OS = D + 4;
  constexpr bool TWO = NT <= 2;
  static_assert((TWO ? 2 : 1) * RP * OS * sizeof(float) <= sizeof(vt), "merge buffers exceed the V buffers");
  float* obuf = reinterpret_cast<float*>(&vt[0][0]);
  float fac[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n16;
    float M = kNegInf;
    for (int w = 0; w < kVerWaves; ++w) M = fmaxf(M, ml_sh[w][0][r]);
    const float base = M == kNegInf ? 0.f : M;
    fac[nt] = exp2f_fast(m_run[nt] - base);
  }
  auto put = [&](float* buf, bool add) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        float4* dst = reinterpret_cast<float4*>(buf + (nt * 16 + n16) * OS + dt * 16 + g4 * 4);
        float4 val = make_float4(oacc[nt][dt][0] * fac[nt], oacc[nt][dt][1] * fac[nt], oacc[nt][dt][2] * fac[nt],
                                 oacc[nt][dt][3] * fac[nt]);
        if (add) {
          const float4 o = *dst;
          val = make_float4(o.x + val.x, o.y + val.y, o.z + val.z, o.w + val.w);
        }
        *dst = val;
      }
    }
  };
  const size_t rec = (bkv * nsplit + split) * RP;
  float4* po = reinterpret_cast<float4*>(part_o + rec * D);
  constexpr int C4 = D / 4;
  if constexpr (TWO) {
    if (wave < 2) put(obuf + wave * RP * OS, false);
    __syncthreads();
    if (wave >= 2) put(obuf + (wave - 2) * RP * OS, true);
    __syncthreads();
    for (int t = tid; t < R * C4; t += kVerThreads) {
      const float4 a = *reinterpret_cast<const float4*>(obuf + (t / C4) * OS + (t % C4) * 4);
      const float4 c = *reinterpret_cast<const float4*>(obuf + RP * OS + (t / C4) * OS + (t % C4) * 4);
      po[t] = make_float4(a.x + c.x, a.y + c.y, a.z + c.z, a.w + c.w);
    }
  } else {
    for (int w = 0; w < kVerWaves; ++w) {
      if (wave == w) put(obuf, w > 0);
      __syncthreads();
    }
    for (int t = tid; t < R * C4; t += kVerThreads)
      po[t] = *reinterpret_cast<const float4*>(obuf + (t / C4) * OS + (t % C4) * 4);
  }
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
// partials. Blocks [0, nblk_o) each write 256 (page form: 512) outputs of the merged rows;
// the remaining blocks each normalise kFinTiles tiles of position partials
// (4 positions per thread: float partials, or a lane group's codes on one
// page of a subtile) or, PAGES, kVerThreads pages of page masses, one page
// per thread.
// Every block first merges the per-split (max, sum) of all rows, in split
// order, so every value is computed the same way by every block.
constexpr int kFinTiles = kVerThreads / (kSub / 4);  // score tiles per finalize block (8 threads per tile)

template <typename VT, int D, bool PAGES>
__global__ __launch_bounds__(kVerThreads) void verify_finalize_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, const VT* __restrict__ sc_val,
    const float* __restrict__ sc_max, const int* __restrict__ seq_len, int k, int Hkv, int G, int chunk,
    int nsplit, int ntile_cap, int RP, int nblk_o, int x0, int balanced, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ scores, int score_stride) {
  constexpr bool CODES = std::is_same<VT, uint32_t>::value && !PAGES;
  __shared__ float mrow[64], lrow[64], l2row[64];
  __shared__ float wt[PAGES ? 1 : kFinTiles][65];  // padded: a wave's tiles read distinct banks
  __shared__ float wsp[PAGES ? 4 : 1][64];  // page records in bf16: weights of the block's splits
  const int pair = blockIdx.y, tid = threadIdx.x;
  const int b = pair / Hkv, kv = pair % Hkv;
  const int S = seq_len[b];
  const int x = x0 + (int)blockIdx.x;
  const int tile_beg = (x - nblk_o) * kFinTiles;
  const int page_beg = (x - nblk_o) * kVerThreads;
  if (x >= nblk_o && (PAGES ? page_beg * kPage : tile_beg * kSub) >= S) return;
  // the splits the split pass wrote: balanced splits (MFMA path) may leave the
  // last of ceil(S / chunk) empty once a sequence has hundreds of them
  const int used = balanced ? ceil_div(S, ceil_div(ceil_div(S, ceil_div(S, chunk)), kSub) * kSub)
                            : min(nsplit, ceil_div(S, chunk));
  const int R = (k + 1) * G, Hq = Hkv * G;
  const size_t bkv = (size_t)pair;
  // Position-form score blocks: the first tile maxima the block's weights need
  // do not depend on the row statistics, so they are loaded first and arrive
  // while the statistics are formed. (Loading the code words up front as well
  // costs more occupancy than the round trip it saves.)
  float pmv[4];
  if constexpr (CODES) {
    if (x >= nblk_o) {
      const int ms = max_stride(R), tend = min(ceil_div(S, kSub), tile_beg + kFinTiles);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + i * kVerThreads, et = e / R, r = e % R, tile = tile_beg + et;
        pmv[i] = (e < kFinTiles * R && tile < tend) ? sc_max[(bkv * ntile_cap + tile) * ms + r] : kNegInf;
      }
    }
  }
  // Row statistics: 4 lanes per row, each over every 4th split, then a fixed
  // butterfly over the 4 lanes (same order in every block). Up to 8 splits
  // each lane loads its (max, sum) pairs once.
  for (int r0 = 0; r0 < R; r0 += kVerThreads / 4) {
    const int r = r0 + tid / 4, c4 = tid & 3;
    float m = kNegInf, l = 0.f;
    if (used <= 8) {
      float2 ml0 = make_float2(kNegInf, 0.f), ml1 = make_float2(kNegInf, 0.f);
      if (r < R && c4 < used) ml0 = *reinterpret_cast<const float2*>(part_ml + ((bkv * nsplit + c4) * RP + r) * 2);
      if (r < R && c4 + 4 < used)
        ml1 = *reinterpret_cast<const float2*>(part_ml + ((bkv * nsplit + c4 + 4) * RP + r) * 2);
      m = fmaxf(ml0.x, ml1.x);
      m = fmaxf(m, __shfl_xor(m, 1, kWave));
      m = fmaxf(m, __shfl_xor(m, 2, kWave));
      const float base = m == kNegInf ? 0.f : m;
      if (r < R && c4 < used) l += ml0.y * exp2f_fast(ml0.x - base);
      if (r < R && c4 + 4 < used) l += ml1.y * exp2f_fast(ml1.x - base);
    } else {
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
    }
    const float base = m == kNegInf ? 0.f : m;
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
    // EPT neighbouring elements (r, d .. d + EPT - 1) per thread: two for the
    // page form, whose finalize is mostly this merge (one measured slower for
    // the position form, whose score blocks dominate)
    constexpr int EPT = PAGES ? 2 : 1;
    const int t = (x * kVerThreads + tid) * EPT;
    if (t < R * D) {
      const int r = t / D, d = t % D;
      float A[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) A[e] = 0.f;
      // splits in order, loads of 8 splits issued together
      for (int c0 = 0; c0 < used; c0 += 8) {
        float po[8][EPT], pm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const size_t rc = (bkv * nsplit + min(c0 + i, used - 1)) * RP + r;
#pragma unroll
          for (int e = 0; e < EPT; ++e) po[i][e] = part_o[rc * D + d + e];
          pm[i] = part_ml[rc * 2];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (c0 + i < used) {
            const float w = exp2f_fast(pm[i] - mrow[r]);
#pragma unroll
            for (int e = 0; e < EPT; ++e) A[e] += po[i][e] * w;
          }
        }
      }
      const int i = r / G, h = kv * G + r % G;
#pragma unroll
      for (int e = 0; e < EPT; ++e) out[(((size_t)b * (k + 1) + i) * Hq + h) * D + d + e] = A[e] / lrow[r];
      if (lse != nullptr && d == 0) lse[((size_t)b * (k + 1) + i) * Hq + h] = l2row[r] * kLn2;
    }
    return;
  }
  if constexpr (PAGES && std::is_same<VT, uint16_t>::value) {
    // bf16 page records (row order) relative to the base of the page's split:
    // page score = sum over the rows, in order, of the split's weight
    // exp2(base - log2 of the row's normaliser) times the record's mass. The
    // block's 256 pages span at most 3 splits (a sequence cut into several
    // splits has splits of at least 2048 positions); their weights go to LDS.
    const int ch = balanced ? ceil_div(ceil_div(S, ceil_div(S, chunk)), kSub) * kSub : chunk;
    const int npages = ceil_div(S, kPage);
    const int s_lo = page_beg * kPage / ch;
    const int s_hi = min(used - 1, (min(page_beg + kVerThreads, npages) - 1) * kPage / ch);
    for (int e = tid; e < 4 * R; e += kVerThreads) {
      const int i = e / R, r = e % R;
      wsp[i][r] = s_lo + i <= s_hi ? exp2f_fast(part_ml[((bkv * nsplit + s_lo + i) * RP + r) * 2] - l2row[r]) : 0.f;
    }
    __syncthreads();
    const int page = page_beg + tid;
    if (page < npages) {
      const int sp = page * kPage / ch, si = sp - s_lo;
      const uint4* m4 = reinterpret_cast<const uint4*>(sc_val + (bkv * 2 * ntile_cap + page) * RP);
      float acc = 0.f;
      for (int i0 = 0; i0 < RP; i0 += 16) {
        const uint4 ua = m4[i0 / 8], ub = m4[i0 / 8 + 1];
        const uint32_t u[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = i0 + j;
          if (r < R) {
            const float w = si < 4 ? wsp[si][r]
                                   : exp2f_fast(part_ml[((bkv * nsplit + sp) * RP + r) * 2] - l2row[r]);
            acc = fmaf(w, __uint_as_float((j & 1) ? (u[j >> 1] & 0xffff0000u) : (u[j >> 1] << 16)), acc);
          }
        }
      }
      scores[bkv * score_stride + page] = acc;
    }
    return;
  } else if constexpr (PAGES) {
    // page score = sum over the rows of exp2(mass - log2 of the row's normaliser)
    // record slot i holds row (i % NT) * 16 + i / NT (NT = RP / 16 row tiles);
    // the rows are summed in slot order
    const int NT = RP / 16;
    const int page = page_beg + tid;
    if (page * kPage < S) {
      // the record (RP floats, 16 B aligned) loaded whole, 16 floats at a time
      const float4* m4 = reinterpret_cast<const float4*>(sc_val + (bkv * 2 * ntile_cap + page) * RP);
      float acc = 0.f;
      for (int i0 = 0; i0 < RP; i0 += 16) {
        float m[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 v = m4[i0 / 4 + j];
          m[4 * j] = v.x;
          m[4 * j + 1] = v.y;
          m[4 * j + 2] = v.z;
          m[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int i = i0 + j, r = (i % NT) * 16 + i / NT;
          if (r < R) acc += exp2f_fast(m[j] - l2row[r]);
        }
      }
      scores[bkv * score_stride + page] = acc;
    }
    return;
  }
  const int ntiles = ceil_div(S, kSub);
  const int tile_end = min(ntiles, tile_beg + kFinTiles);
  // weights of every (tile, row) of this block, then 4 positions per thread
  // (the block's maxima records are one contiguous run: loads issued 4 at a time)
  const float sh = CODES ? kCodeScaleLog2 : 0.f;
  const int ms = max_stride(R);
  for (int e0 = tid; e0 < kFinTiles * R; e0 += 4 * kVerThreads) {
    float mv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + i * kVerThreads, et = e / R, r = e % R, tile = tile_beg + et;
      if (CODES && e0 == tid)
        mv[i] = pmv[i];  // loaded before the row statistics
      else
        mv[i] = (e < kFinTiles * R && tile < tile_end) ? sc_max[(bkv * ntile_cap + tile) * ms + r] : kNegInf;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + i * kVerThreads;
      if (e < kFinTiles * R) wt[e / R][e % R] = mv[i] == kNegInf ? 0.f : exp2f_fast(mv[i] - l2row[e % R] + sh);
    }
  }
  __syncthreads();
  if constexpr (CODES) {
    // wave = one group of kCodeGroup tiles, lane = (tile, lane group g4):
    // thread (tile, lane group g4, page h): positions 16 h + 4 g4 .. +3
    const int tl = tid >> 3, g4 = (tid >> 1) & 3, h = tid & 1;
    const int tile = tile_beg + tl, pos = tile * kSub + 16 * h + 4 * g4;
    if (tile < tile_end && pos < S) {
      const int ngrp = ceil_div(ntile_cap, kCodeGroup);
      const uint32_t* rec = sc_val + code_record(bkv, ngrp, R, tile, 0) + 3 * g4 + h;
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      constexpr int kRowBatch = 7;  // divides R at G = 2 and 4 with k = 6 (14, 28 rows)
      for (int r0 = 0; r0 < R; r0 += kRowBatch) {
        uint32_t wv[kRowBatch][2];
#pragma unroll
        for (int i = 0; i < kRowBatch; ++i) {
          const uint32_t* v = rec + (size_t)min(r0 + i, R - 1) * kCodeGroup * kCodeWords;
          wv[i][0] = v[0];
          wv[i][1] = v[1];
        }
#pragma unroll
        for (int i = 0; i < kRowBatch; ++i) {
          const float w = r0 + i < R ? wt[tl][r0 + i] : 0.f;
          const uint32_t x = wv[i][0], y = wv[i][1];
          constexpr uint32_t M = 0x0fff0000u;
          const uint32_t f0 = h ? x & M : (x << 16) & M;
          const uint32_t f1 = h ? __builtin_amdgcn_alignbit(y, x, 12) & M : (x << 4) & M;
          const uint32_t f2 = h ? (y << 8) & M : __builtin_amdgcn_alignbit(y, x, 8) & M;
          const uint32_t f3 = h ? (y >> 4) & M : (y << 12) & M;
          a[0] = fmaf(w, __uint_as_float(f0), a[0]);
          a[1] = fmaf(w, __uint_as_float(f1), a[1]);
          a[2] = fmaf(w, __uint_as_float(f2), a[2]);
          a[3] = fmaf(w, __uint_as_float(f3), a[3]);
        }
      }
      float* dst = scores + bkv * score_stride + pos;
      if (((reinterpret_cast<uintptr_t>(dst) & 15) == 0) && pos + 4 <= S) {
        *reinterpret_cast<float4*>(dst) = make_float4(a[0], a[1], a[2], a[3]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (pos + j < S) dst[j] = a[j];
      }
    }
  } else {
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
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Output-merge blocks of the finalize (two elements per thread in the page form).
static int fin_out_blocks(const VerifyPlan& p, int D) {
  return ceil_div(p.R * D, kVerThreads * ((p.mfma && p.pages) ? 2 : 1));
}

// Page scores of the generic path: the position scores (staged in the
// workspace, row stride `stride`) summed over each page in slot order.
__global__ __launch_bounds__(256) void page_sum_kernel(const float* __restrict__ pos_scores, int stride,
                                                       const int* __restrict__ seq_len, int Hkv,
                                                       float* __restrict__ page_scores, int page_stride) {
  const int pair = blockIdx.y;
  const int S = seq_len[pair / Hkv];
  const int page = blockIdx.x * 256 + threadIdx.x;
  if (page * kPage >= S) return;
  const float* row = pos_scores + (size_t)pair * stride;
  float acc = 0.f;
  for (int j = page * kPage; j < min(S, page * kPage + kPage); ++j) acc += row[j];
  page_scores[(size_t)pair * page_stride + page] = acc;
}

VerifyPlan verify_plan(int B, int k, int Hq, int Hkv, int D, int dtype, int max_seq_len, bool pages) {
  VerifyPlan p;
  p.G = Hq / Hkv;
  p.R = (k + 1) * p.G;
  p.mfma = (dtype == 1 && D == 128);
  p.pages = pages;
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
  p.off_tmp = 0;
  if (pages && p.mfma) {
    // one value per (page, row slot): 2 pages per subtile; bf16 masses when
    // the split kernel gathers them in LDS, float log2 masses otherwise
    p.off_sc_max = off;
    p.off_sc_val = off;
    off = align256(off + nbkv * 2 * p.ntile_cap * p.RP * (page_records_bf16(p.NT) ? sizeof(uint16_t) : sizeof(float)));
  } else {
    p.off_sc_max = off;
    off = align256(off + nbkv * p.ntile_cap * max_stride(p.R) * sizeof(float));
    p.off_sc_val = off;
    off = align256(off + (p.mfma ? nbkv * ceil_div(p.ntile_cap, kCodeGroup) * kCodeGroup * p.R * kCodeWords * sizeof(uint32_t)
                                 : nbkv * p.ntile_cap * p.R * kSub * sizeof(float)));
    if (pages) {  // generic path: position scores staged for the page sums
      p.off_tmp = off;
      off = align256(off + nbkv * (size_t)max_seq_len * sizeof(float));
    }
  }
  p.bytes = off;
  return p;
}

template <int NT, int SM>
static void launch_mfma_sm(const VerifyPlan& p, const void* q, const void* kp, const void* vp, const int* bt,
                           int max_pages, int Hkv, const int* seq_len, int npairs, int k, float sl2, char* ws,
                           hipStream_t stream) {
  const int nblocks = ceil_div(npairs, 8) * 8 * p.nsplit;
  hipLaunchKernelGGL((verify_mfma_kernel<NT, kVerQLds && NT == 3, SM>), dim3(nblocks), dim3(kVerThreads), 0,
                     stream, (const bf16_t*)q, (const bf16_t*)kp, (const bf16_t*)vp, bt, max_pages, npairs, Hkv,
                     p.G, seq_len, k, sl2, p.chunk, p.nsplit, p.ntile_cap, (float*)(ws + p.off_part_o),
                     (float*)(ws + p.off_part_ml), (void*)(ws + p.off_sc_val), (float*)(ws + p.off_sc_max));
}

template <int NT>
static void launch_mfma(const VerifyPlan& p, const void* q, const void* kp, const void* vp, const int* bt,
                        int max_pages, int Hkv, const int* seq_len, int npairs, int k, float sl2, int sm, char* ws,
                        hipStream_t stream) {
  if (sm == kScoresPositions)
    launch_mfma_sm<NT, kScoresPositions>(p, q, kp, vp, bt, max_pages, Hkv, seq_len, npairs, k, sl2, ws, stream);
  else if (sm == kScoresPages)
    launch_mfma_sm<NT, kScoresPages>(p, q, kp, vp, bt, max_pages, Hkv, seq_len, npairs, k, sl2, ws, stream);
  else
    launch_mfma_sm<NT, kScoresNone>(p, q, kp, vp, bt, max_pages, Hkv, seq_len, npairs, k, sl2, ws, stream);
}

// Finalize blocks [x0, x0 + nx) of the (output rows | score tiles or pages) range.
static hipError_t launch_finalize(const VerifyPlan& p, int D, const int* seq_len, int npairs, int k,
                                  int Hkv, int x0, int nx, float* out, float* lse, float* scores,
                                  int score_stride, const char* ws, hipStream_t stream) {
  if (nx <= 0) return hipSuccess;
  const int nblk_o = fin_out_blocks(p, D);
  const dim3 grid(nx, npairs);
#define S3R_FIN(VT, DD, PG)                                                                          \
  hipLaunchKernelGGL((verify_finalize_kernel<VT, DD, PG>), grid, dim3(kVerThreads), 0, stream,      \
                     (const float*)(ws + p.off_part_o), (const float*)(ws + p.off_part_ml),          \
                     (const VT*)(ws + p.off_sc_val), (const float*)(ws + p.off_sc_max), seq_len, k,  \
                     Hkv, p.G, p.chunk, p.nsplit, p.ntile_cap, p.RP, nblk_o, x0,                     \
                     (p.mfma && kVerBalance) ? 1 : 0, out, lse, scores, score_stride)
  if (p.mfma && p.pages && page_records_bf16(p.NT)) {
    S3R_FIN(uint16_t, 128, true);
  } else if (p.mfma && p.pages) {
    S3R_FIN(float, 128, true);
  } else if (p.mfma) {
    S3R_FIN(uint32_t, 128, false);
  } else if (D == 128) {
    S3R_FIN(float, 128, false);
  } else {
    S3R_FIN(float, 64, false);
  }
#undef S3R_FIN
  return hipGetLastError();
}

hipError_t launch_verify(int dtype, int D, const void* q, const void* kp, const void* vp,
                         const int* bt, int max_pages, int Hkv, const int* seq_len, int B, int k,
                         int Hq, float scale, int max_seq_len, float* out, float* lse,
                         float* scores, int score_stride, bool pages, bool defer_scores, void* ws_v,
                         hipStream_t stream) {
  const VerifyPlan p = verify_plan(B, k, Hq, Hkv, D, dtype, max_seq_len, pages);
  char* ws = (char*)ws_v;
  const float sl2 = scale * kLog2e;
  const int with_scores = (scores != nullptr || defer_scores) ? 1 : 0;
  const int npairs = B * Hkv;
  if (p.mfma) {
    const int sm = !with_scores ? kScoresNone : (pages ? kScoresPages : kScoresPositions);
#define S3R_MFMA(NTV) \
  launch_mfma<NTV>(p, q, kp, vp, bt, max_pages, Hkv, seq_len, npairs, k, sl2, sm, ws, stream)
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
  const int nblk_o = fin_out_blocks(p, D);
  const bool now = scores != nullptr && !defer_scores;
  if (pages && !p.mfma && now) {
    // generic path: position scores into the workspace, then their page sums
    float* pos = (float*)(ws + p.off_tmp);
    e = launch_finalize(p, D, seq_len, npairs, k, Hkv, 0, nblk_o + ceil_div(p.ntile_cap, kFinTiles), out, lse, pos,
                        max_seq_len, ws, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(page_sum_kernel, dim3(ceil_div(ceil_div(max_seq_len, kPage), 256), npairs), dim3(256), 0,
                       stream, pos, max_seq_len, seq_len, Hkv, scores, score_stride);
    return hipGetLastError();
  }
  const int nblk_s = !now ? 0 : (pages ? ceil_div(2 * p.ntile_cap, kVerThreads) : ceil_div(p.ntile_cap, kFinTiles));
  return launch_finalize(p, D, seq_len, npairs, k, Hkv, 0, nblk_o + nblk_s, out, lse, now ? scores : nullptr,
                         score_stride, ws, stream);
}

hipError_t launch_verify_scores(int dtype, int D, const int* seq_len, int B, int k, int Hq, int Hkv,
                                int max_seq_len, float* scores, int score_stride, const void* ws,
                                hipStream_t stream) {
  const VerifyPlan p = verify_plan(B, k, Hq, Hkv, D, dtype, max_seq_len, false);
  const int nblk_o = fin_out_blocks(p, D);
  return launch_finalize(p, D, seq_len, B * Hkv, k, Hkv, nblk_o, ceil_div(p.ntile_cap, kFinTiles), nullptr,
                         nullptr, scores, score_stride, (const char*)ws, stream);
}

}  // namespace s3r
