// Body of the bf16-KV decode workgroup (the kernel that runs it alone is in
// decode_bf16.hip, the windowed decode runs it for the window workgroups):
// work item `wid` = (split, sequence, KV head).
#pragma once
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace b16 {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWaves = 4;
constexpr int kStep = 2;   // pages per step (one 32-token PV product)

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_val(uint16_t b) { return u2f(static_cast<uint32_t>(b) << 16); }

// limb `lam` (0 = hi, 1 = mid, 2 = lo, 3 = none) of x as bf16 bits
__device__ __forceinline__ uint16_t bf16_limb(float x, int lam) {
  const uint16_t h = bf16_bits(x);
  const float r1 = x - bf16_val(h);
  const uint16_t m = bf16_bits(r1);
  const uint16_t l = bf16_bits(r1 - bf16_val(m));
  return lam == 0 ? h : lam == 1 ? m : lam == 2 ? l : static_cast<uint16_t>(0);
}

__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppRowHalfMirror>(x);
  return x + dpp_f<kDppRowMirror>(x);
}

template <int D>
__device__ __forceinline__ int pv_channel(int n, int tau) {
  if constexpr (D == 128) return 8 * n + tau;
  else return 8 * (n & 7) + 2 * tau + (n >> 3);
}

__device__ __forceinline__ v8bf as_bf(u32x4 w) { return __builtin_bit_cast(v8bf, w); }

template <int D, int NS>
struct SmemB {
  static constexpr int kGP = 4 * NS;
  union {
    float qs[kGP][D];
    struct {
      float acc[kWaves][kGP][D];
      float m[kWaves][kGP];
      float l[kWaves][kGP];
      float o[kGP][D];
    } merge;
  } u;
  uint16_t pl[kWaves][NS][4][4][kStep][16];   // [wave][set][limb][head][page][token]
};

// BAL: a balanced call (balanced_split_pages), built apart so that the
// planned calls carry none of its code
template <int D, int NS, bool QBF16, bool BAL>
__device__ __forceinline__ void decode_bf16_body(const DecodeArgs& a, uint32_t wid) {
  constexpr int kSlab = 4 * kPage * D;   // bytes
  constexpr int kNT = D / 16;
  constexpr int kNK = D / 32;            // QK MFMAs per page
  constexpr int kGP = 4 * NS;
  __shared__ SmemB<D, NS> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int g = lane >> 4, n = lane & 15, hs = n >> 2, lam = n & 3;
  // Work item (split s, sequence b, KV head), KV head fastest and split
  // slowest, last split first.  Each split is one contiguous run of
  // workgroups that the round-robin dispatch spreads over every XCD and CU
  // (with the split fastest, a period of 2, 4 or 8 left most CUs with the
  // empty splits of short sequences only), and the later splits, busy only
  // for the longest sequences, start first instead of last.
  const int kvh = static_cast<int>(wid % a.num_kv_heads);
  const int b = static_cast<int>((wid / a.num_kv_heads) % a.batch);
  // pages per split, and the split: last first, unless the device grew the
  // splits (then the later ones are empty, and first-split-first keeps them
  // from holding the machine before the work starts)
  const int sp = BAL ? balanced_split_pages(a.split_pages, a.seq_lens, a.batch, a.max_seq_len,
                                            a.num_kv_heads)
                     : a.split_pages;
  const int s = BAL && sp != a.split_pages
                    ? static_cast<int>(wid / a.num_kv_heads / a.batch)
                    : a.nsplit - 1 - static_cast<int>(wid / a.num_kv_heads / a.batch);
  const int G = a.num_q_heads / a.num_kv_heads;

  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  if (a.len_cap > 0 && len > a.len_cap) len = a.len_cap;   // window pass: the window's tokens
  const int npg = (len + kPage - 1) / kPage;
  const int p0 = s * sp;
  const int p1 = min(npg, p0 + sp);
  if (p0 >= p1) {
    if (a.nsplit == 1 && !a.force_partial) {
      for (int e = tid; e < G * D; e += 64 * kWaves)
        a.out[(static_cast<int64_t>(b) * a.num_q_heads + kvh * G + e / D) * D + e % D] = 0.0f;
    }
    return;
  }
  // a sequence whose pages all lie in one split is finished here (the split
  // merge skips its rows); windowed calls always store partials
  const bool direct = !a.force_partial && (a.nsplit == 1 || (npg - 1) / sp == 0);

  const int span = p1 - p0;
  const int per_wave = ((span + kWaves - 1) / kWaves + kStep - 1) / kStep * kStep;
  const int pw0 = p0 + wave * per_wave;
  const int pw1 = min(p1, pw0 + per_wave);
  const uint8_t* pool_h = a.pool + static_cast<int64_t>(kvh) * kSlab;
  const int64_t page_stride = static_cast<int64_t>(a.num_kv_heads) * kSlab;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  const int vn = n & (D / 8 - 1);
  const int k_off = (n * D + 8 * g) * 2;
  const int v_off = (kPage * D + (vn * (kPage / 4) + g) * 32) * 2;

  // The query is requested first; then the page ids (scalar loads, always
  // inside the row: pages at or past pw1 read a clamped entry and are
  // dropped) and the first step's pages, so that the query's wait leaves
  // the pages in flight while the query is staged into limbs.
  constexpr int kQPer = kGP * D / (64 * kWaves);   // query elements per thread
  uint16_t qraw[kQPer];
#pragma unroll
  for (int r = 0; r < kQPer; ++r) {
    const int e = tid + r * 64 * kWaves, j = e / D, c = e % D;
    qraw[r] = j < G ? a.q[(static_cast<int64_t>(b) * a.num_q_heads + kvh * G + j) * D + c] : 0;
  }
  using ConstI32 = const __attribute__((address_space(4))) int32_t;
  ConstI32* bt_s = (ConstI32*)bt;   // generic to constant address space
  auto ids = [&](int p, int32_t (&id)[kStep]) {
#pragma unroll
    for (int i = 0; i < kStep; ++i) id[i] = bt_s[min(p + i, pw1 - 1)];
  };
  u32x4 kx[kStep][kNK], vx[kStep][4];
  bool pv[kStep];
  bool all_ok = true;
  auto load_step = [&](int p, const int32_t (&id)[kStep]) {
    all_ok = true;
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      pv[i] = p + i < pw1 && id[i] >= 0 && id[i] < a.num_pages;
      all_ok = all_ok && pv[i];
      const uint8_t* sl = pool_h + static_cast<int64_t>(pv[i] ? id[i] : 0) * page_stride;
#pragma unroll
      for (int mu = 0; mu < kNK; ++mu) kx[i][mu] = *reinterpret_cast<const u32x4*>(sl + k_off + 64 * mu);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) vx[i][qq] = *reinterpret_cast<const u32x4*>(sl + v_off + 16 * qq);
    }
  };
  int32_t idc[kStep];
  if constexpr (NS <= 2) {   // (with four sets the step buffer held here would cost a wave per SIMD)
    ids(pw0, idc);
    load_step(pw0, idc);
    ids(pw0 + kStep, idc);
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int r = 0; r < kQPer; ++r) {
    const int e = tid + r * 64 * kWaves, j = e / D, c = e % D;
    const uint16_t u = qraw[r];
    sm.u.qs[j][c] = j < G ? (QBF16 ? u2f(static_cast<uint32_t>(u) << 16) : static_cast<float>(__builtin_bit_cast(_Float16, u))) : 0.0f;
  }
  for (int e = tid; e < kWaves * NS * 4 * 4 * kStep * 16; e += 64 * kWaves)
    (&sm.pl[0][0][0][0][0][0])[e] = 0;   // limb-3 rows stay zero
  __syncthreads();

  // A operand of QK: row (head hs, limb lam), channels 32mu + 8g .. +7
  u32x4 aq[NS][kNK];
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int mu = 0; mu < kNK; ++mu) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * mu + 8 * g + 2 * i;
        w[i] = static_cast<uint32_t>(bf16_limb(sm.u.qs[4 * st + hs][c], lam)) |
               (static_cast<uint32_t>(bf16_limb(sm.u.qs[4 * st + hs][c + 1], lam)) << 16);
      }
      aq[st][mu] = w;
    }

  float m_run[NS], l_run[NS], acc[NS][kNT];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    m_run[st] = kNegInf;
    l_run[st] = 0.0f;
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[st][t] = 0.0f;
  }
  const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int p = pw0; p < pw1; p += kStep) {
    if constexpr (NS > 2) {   // loads at the top of the step
      ids(p, idc);
      load_step(p, idc);
    }
    const bool tail = !all_ok || (p + kStep) * kPage > len;
    if (tail) {
      // zero the values of tokens past the end (or of unusable pages) so that
      // stale bits there never meet the zero weights as NaN or Inf
#pragma unroll
      for (int i = 0; i < kStep; ++i) {
        const int t0 = (p + i) * kPage + 4 * g;
        const uint32_t m01 = (pv[i] && t0 < len ? 0x0000FFFFu : 0u) | (pv[i] && t0 + 1 < len ? 0xFFFF0000u : 0u);
        const uint32_t m23 = (pv[i] && t0 + 2 < len ? 0x0000FFFFu : 0u) | (pv[i] && t0 + 3 < len ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          vx[i][qq][0] &= m01;
          vx[i][qq][1] &= m23;
          vx[i][qq][2] &= m01;
          vx[i][qq][3] &= m23;
        }
      }
    }

    float lg[NS][kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const bool ok = !tail || (pv[i] && (p + i) * kPage + n < len);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        v4f c = zero4;
#pragma unroll
        for (int mu = 0; mu < kNK; ++mu) c = mfma_bf16(as_bf(aq[st][mu]), as_bf(kx[i][mu]), c);
        lg[st][i] = ok ? ((c[0] + c[1]) + c[2]) * a.sm_log2 : kNegInf;
      }
    }

    float alpha[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float mc = lg[st][0];
#pragma unroll
      for (int i = 1; i < kStep; ++i) mc = fmaxf(mc, lg[st][i]);
      mc = row_max16_ordered(mc);
      const float mnew = fmaxf(m_run[st], mc);
      const float muse = mnew == kNegInf ? 0.0f : mnew;
      alpha[st] = fast_exp2(m_run[st] - muse);
      m_run[st] = mnew;
      float psum = 0.0f;
      uint16_t* pl = &sm.pl[wave][st][0][0][0][0];
#pragma unroll
      for (int i = 0; i < kStep; ++i) {
        const float pp = fast_exp2(lg[st][i] - muse);
        psum += pp;
        const uint16_t h = bf16_bits(pp);
        const float r1 = pp - bf16_val(h);
        const uint16_t m = bf16_bits(r1);
        const uint16_t lo = bf16_bits(r1 - bf16_val(m));
        pl[((0 * 4 + g) * kStep + i) * 16 + n] = h;
        pl[((1 * 4 + g) * kStep + i) * 16 + n] = m;
        pl[((2 * 4 + g) * kStep + i) * 16 + n] = lo;
      }
      l_run[st] = __builtin_fmaf(l_run[st], alpha[st], psum);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    u32x4 apv[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const uint16_t* pl = &sm.pl[wave][st][0][0][0][0];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(pl + ((lam * 4 + hs) * kStep + 0) * 16 + 4 * g);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(pl + ((lam * 4 + hs) * kStep + 1) * 16 + 4 * g);
      apv[st] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }

#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) {
      const int jj = (D == 128) ? tau : 2 * tau + (n >> 3);   // channel 8*vn + jj
      u32x4 bv;
#pragma unroll
      for (int i = 0; i < kStep; ++i) {
        const int w0 = 2 * jj;   // four tokens of one channel = words 2jj, 2jj+1
        bv[2 * i] = vx[i][w0 >> 2][w0 & 3];
        bv[2 * i + 1] = vx[i][(w0 + 1) >> 2][(w0 + 1) & 3];
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const v4f c = mfma_bf16(as_bf(apv[st]), as_bf(bv), zero4);
        acc[st][tau] = __builtin_fmaf(acc[st][tau], alpha[st], (c[0] + c[1]) + c[2]);
      }
    }
    if constexpr (NS <= 2) {   // the next step's loads, then the ids of the step after it
      if (p + kStep >= pw1) break;
      load_step(p + kStep, idc);
      ids(p + 2 * kStep, idc);
    }
  }

  __syncthreads();
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const float lt = row_sum16(l_run[st]);
    const int j = 4 * st + g;
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) sm.u.merge.acc[wave][j][pv_channel<D>(n, tau)] = acc[st][tau];
    if (n == 0) {
      sm.u.merge.m[wave][j] = m_run[st];
      sm.u.merge.l[wave][j] = lt;
    }
  }
  __syncthreads();
  const int64_t hq0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * G;
  for (int e = tid; e < G * D; e += 64 * kWaves) {
    const int j = e / D, c = e % D;
    float mstar = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm.u.merge.m[w][j]);
    const float muse = mstar == kNegInf ? 0.0f : mstar;
    float lsum = 0.0f, osum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm.u.merge.m[w][j] - muse);
      lsum = __builtin_fmaf(sm.u.merge.l[w][j], f, lsum);
      osum = __builtin_fmaf(sm.u.merge.acc[w][j][c], f, osum);
    }
    if (direct) {
      a.out[(hq0 + j) * D + c] = lsum > 0.0f ? osum / lsum : 0.0f;
    } else {
      const int64_t idx = (hq0 + j) * a.part_stride + a.part_slot0 + s;
      a.part_acc[idx * D + c] = osum;
      if (c == 0) {
        a.part_ml[idx * 2 + 0] = mstar;
        a.part_ml[idx * 2 + 1] = lsum;
      }
    }
  }
}

}  // namespace b16
}  // namespace kvq
