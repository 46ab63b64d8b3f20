// Read path: split-K paged decode attention over the INT4 cache with the
// dequantization folded into the products ("SAW-INT4", summary page: fused
// attention execution over paged quantized KV; "BitDecoding-FP4", Abstract:
// the query heads of a GQA group stacked into one matrix product per KV page;
// the factoring of the per-token scale out of the dot product follows the
// same idea as "InnerQ", Figure 1).
//
// One wave = one (sequence b, KV head, split s).  Per page (16 tokens) and
// per group of four query heads:
//   QK:  C[token][(head, limb)] = sum_c code[token][c] * qlimb[c]   (int8 MFMA)
//        The rotated query is held as a 23-bit fixed-point integer split into
//        three signed 8-bit limbs; the 4-bit codes are exact int8; products
//        and sums are exact in int32.  logit = sm * 2^(e-22) *
//        (k_scale * sum_c code*qfix + k_zero * sum_c qfix).
//   softmax: online, in base 2, per query head.
//   PV:  acc[(head, limb)][c] = sum_t wlimb[t] * code_v[t][c]       (int8 MFMA)
//        with w = p * v_scale as a 23-bit fixed-point integer relative to the
//        chunk's largest w (power-of-two scale), plus sum_t p * v_zero added
//        to every channel.
// Partials (m, l, unnormalised output) go to the workspace; the reduce kernel
// merges the splits and rotates the output back.
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// byte `lam` of the balanced base-256 split v = l0*2^16 + l1*2^8 + l2 with
// l1, l2 in [-128, 127] (|v| <= 2^22); lam = 3 gives 0.
__device__ __forceinline__ uint32_t limb_byte(int32_t v, int lam) {
  const int32_t y = v + 0x8080;
  const uint32_t b0 = static_cast<uint32_t>(y >> 16) & 0xFFu;
  const uint32_t b1 = ((static_cast<uint32_t>(y) >> 8) & 0xFFu) ^ 0x80u;
  const uint32_t b2 = (static_cast<uint32_t>(y) & 0xFFu) ^ 0x80u;
  return lam == 0 ? b0 : lam == 1 ? b1 : lam == 2 ? b2 : 0u;
}

// channel of k-slot (dword i, byte k) of the QK operand `op` for lane group g
template <int D>
__device__ __forceinline__ int qk_channel(int g, int op, int i, int k) {
  if constexpr (D == 128) return 32 * g + 8 * i + 2 * k + op;
  else return 16 * g + 8 * (i & 1) + 2 * k + (i >> 1);
}

// output channel of PV tile tau for lane column n
template <int D>
__device__ __forceinline__ int pv_channel(int n, int tau) {
  if constexpr (D == 128) return 8 * n + tau;
  else return 8 * (n & 7) + 2 * tau + (n >> 3);
}

template <int D, int NS, bool QBF16>
__global__ __launch_bounds__(64) void decode_int4_kernel(DecodeArgs a) {
  constexpr int kSlab = kPage * (D + 8);
  constexpr int kNT = D / 16;          // PV tiles = output channels per lane
  constexpr int kOps = D / 64;         // QK MFMAs per page and head group
  constexpr int kGP = 4 * NS;          // padded heads per KV head

  const int lane = threadIdx.x;
  const int g = lane >> 4, n = lane & 15, hs = n >> 2, lam = n & 3;
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.num_q_heads / a.num_kv_heads;

  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const int npg = (len + kPage - 1) / kPage;
  const int p0 = s * a.split_pages;
  const int p1 = min(npg, p0 + a.split_pages);
  if (p0 >= p1) return;

  __shared__ float qs[kGP][D];
  __shared__ int32_t qi[kGP][D];
  __shared__ float hA[kGP], hS[kGP];

  // ---- query: load, rotate (fp32 butterfly), fixed point, limbs ----------
  for (int e = lane; e < kGP * D; e += 64) {
    const int j = e / D, c = e % D;
    float v = 0.0f;
    if (j < G) {
      const uint16_t u = a.q[(static_cast<int64_t>(b) * a.num_q_heads + kvh * G + j) * D + c];
      v = QBF16 ? u2f(static_cast<uint32_t>(u) << 16) : static_cast<float>(__builtin_bit_cast(_Float16, u));
    }
    qs[j][c] = v;
  }
  __syncthreads();
  if (a.block > 0) {
    for (int hh = 1; hh < a.block; hh *= 2) {
      for (int pi = lane; pi < kGP * D / 2; pi += 64) {
        const int j = pi / (D / 2), q = pi % (D / 2);
        const int i = (q / hh) * (2 * hh) + (q % hh);
        const float u = qs[j][i], w = qs[j][i + hh];
        qs[j][i] = u + w;
        qs[j][i + hh] = u - w;
      }
      __syncthreads();
    }
    const float sb = block_norm(a.block);
    for (int e = lane; e < kGP * D; e += 64) qs[e / D][e % D] *= sb;
    __syncthreads();
  }
  for (int j0 = 0; j0 < kGP; j0 += 4) {
    const int j = j0 + g;
    float am = 0.0f;
    for (int c = n; c < D; c += 16) am = fmaxf(am, fabsf(qs[j][c]));
    for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
    int ex = 0;
    frexpf(am, &ex);                    // am < 2^ex
    const float sc = ldexpf(1.0f, 22 - ex);
    int32_t sum = 0;
    for (int c = n; c < D; c += 16) {
      const int32_t v = static_cast<int32_t>(rintf(qs[j][c] * sc));
      qi[j][c] = v;
      sum += v;
    }
    for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o);
    if (n == 0) {
      hA[j] = a.sm_log2 * ldexpf(1.0f, ex - 22);
      hS[j] = static_cast<float>(sum);
    }
  }
  __syncthreads();

  v4i bq[NS][kOps];
  float qA[NS], qS[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int j = 4 * st + hs;
    qA[st] = hA[j];
    qS[st] = hS[j];
#pragma unroll
    for (int op = 0; op < kOps; ++op) {
      v4i v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) w |= limb_byte(qi[j][qk_channel<D>(g, op, i, k)], lam) << (8 * k);
        v[i] = static_cast<int32_t>(w);
      }
      bq[st][op] = v;
    }
  }
  const float wlam = lam == 0 ? 65536.0f : lam == 1 ? 256.0f : lam == 2 ? 1.0f : 0.0f;

  // ---- stream the split's pages, four per step -----------------------------
  float m_run[NS], l_run[NS], z_run[NS], acc[NS][kNT];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    m_run[st] = kNegInf;
    l_run[st] = 0.0f;
    z_run[st] = 0.0f;
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[st][t] = 0.0f;
  }
  const uint8_t* pool_h = a.pool + static_cast<int64_t>(kvh) * kSlab;
  const int64_t page_stride = static_cast<int64_t>(a.num_kv_heads) * kSlab;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  const int vn = n & (D / 8 - 1);
  const v4i zero4 = {0, 0, 0, 0};

  for (int p = p0; p < p1; p += 4) {
    u32x4 kx[4], vx[4], km[4], vm[4];
    bool pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pg = p + i;
      const int pid = pg < p1 ? bt[pg] : -1;
      pv[i] = pid >= 0 && pid < a.num_pages;
      if (pv[i]) {
        const uint8_t* sl = pool_h + static_cast<int64_t>(pid) * page_stride;
        if constexpr (D == 128) {
          kx[i] = *reinterpret_cast<const u32x4*>(sl + n * (D / 2) + g * 16);
        } else {
          const u32x2 t2 = *reinterpret_cast<const u32x2*>(sl + n * (D / 2) + g * 8);
          kx[i] = u32x4{t2[0], t2[1], 0u, 0u};
        }
        vx[i] = *reinterpret_cast<const u32x4*>(sl + kPage * D / 2 + (vn * kPage + 4 * g) * 4);
        km[i] = *reinterpret_cast<const u32x4*>(sl + kPage * D + 16 * g);
        vm[i] = *reinterpret_cast<const u32x4*>(sl + kPage * D + 4 * kPage + 16 * g);
      } else {
        kx[i] = vx[i] = km[i] = vm[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    // QK and logits (base-2), rows = tokens 4g..4g+3 of each page
    float lg[NS][4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4i a0, a1;
      if constexpr (D == 128) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          a0[w] = static_cast<int32_t>(kx[i][w] & kLowNibbles);
          a1[w] = static_cast<int32_t>((kx[i][w] >> 4) & kLowNibbles);
        }
      } else {
        a0 = v4i{static_cast<int32_t>(kx[i][0] & kLowNibbles), static_cast<int32_t>(kx[i][1] & kLowNibbles),
                 static_cast<int32_t>((kx[i][0] >> 4) & kLowNibbles),
                 static_cast<int32_t>((kx[i][1] >> 4) & kLowNibbles)};
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        v4i c = mfma_i8(a0, bq[st][0], zero4);
        if constexpr (kOps == 2) c = mfma_i8(a1, bq[st][1], c);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float v = static_cast<float>(c[rr]) * wlam;
          v += dpp_f<kDppXor1>(v);
          v += dpp_f<kDppXor2>(v);
          const uint32_t mk = km[i][rr];
          const int tok = (p + i) * kPage + 4 * g + rr;
          const bool ok = pv[i] && tok < len;
          const float l2 = qA[st] * __builtin_fmaf(half_hi(mk), qS[st], half_lo(mk) * v);
          lg[st][i][rr] = ok ? l2 : kNegInf;
        }
      }
    }

    // online softmax and the PV operand (limb `lam` of p * v_scale)
    v4i apv[NS];
    float alpha_pv[NS], sw_pv[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float mc = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mc = fmaxf(mc, lg[st][i][rr]);
      mc = max_rows(mc);
      const float mnew = fmaxf(m_run[st], mc);
      const float muse = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = exp2f(m_run[st] - muse);
      m_run[st] = mnew;
      float psum = 0.0f, zsum = 0.0f, wmax = 0.0f;
      float w[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bool ok = lg[st][i][rr] != kNegInf;
          const float pp = exp2f(lg[st][i][rr] - muse);
          const uint32_t mv = vm[i][rr];
          psum += pp;
          zsum += ok ? pp * half_hi(mv) : 0.0f;
          w[i][rr] = ok ? pp * half_lo(mv) : 0.0f;
          wmax = fmaxf(wmax, w[i][rr]);
        }
      l_run[st] = l_run[st] * alpha + psum;
      z_run[st] = z_run[st] * alpha + zsum;
      wmax = max_rows(wmax);
      int ew = 0;
      frexpf(wmax, &ew);                 // wmax < 2^ew
      const float wsc = ldexpf(1.0f, 22 - ew);
      v4i av;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t dw = 0;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          dw |= limb_byte(static_cast<int32_t>(rintf(w[i][rr] * wsc)), lam) << (8 * rr);
        av[i] = static_cast<int32_t>(dw);
      }
      apv[st] = av;
      // PV-layout lane (g, n) holds head g of this set: take its scalars from
      // QK-layout lane 4g (row 0), which holds head g as well.
      alpha_pv[st] = lane_read(alpha, 4 * g);
      sw_pv[st] = lane_read(ldexpf(1.0f, ew - 22), 4 * g);
    }

    // V codes: 4x4 byte transposes give, per page, one word of four tokens'
    // codes for each channel pair; low / high nibbles are the two channels.
    uint32_t vt[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) transpose_bytes4(vx[i][0], vx[i][1], vx[i][2], vx[i][3], vt[i]);
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) {
      v4i bv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t y;
        if constexpr (D == 128) y = (tau & 1) ? (vt[i][tau >> 1] >> 4) : vt[i][tau >> 1];
        else y = vt[i][tau] >> (4 * (n >> 3));
        bv[i] = static_cast<int32_t>(y & kLowNibbles);
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const v4i c = mfma_i8(apv[st], bv, zero4);
        const float f = __builtin_fmaf(static_cast<float>(c[0]), 65536.0f,
                                       __builtin_fmaf(static_cast<float>(c[1]), 256.0f,
                                                      static_cast<float>(c[2])));
        acc[st][tau] = __builtin_fmaf(acc[st][tau], alpha_pv[st], f * sw_pv[st]);
      }
    }
  }

  // ---- partial results -------------------------------------------------------
  const int64_t hq0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * G;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const float lt = sum_rows(lam == 0 ? l_run[st] : 0.0f);
    const float zt = sum_rows(lam == 0 ? z_run[st] : 0.0f);
    const float z_pv = lane_read(zt, 4 * g);
    const int jp = 4 * st + g;           // PV-layout head
    if (jp < G) {
      const int64_t idx = (hq0 + jp) * a.nsplit + s;
      float* dst = a.part_acc + idx * D;
#pragma unroll
      for (int tau = 0; tau < kNT; ++tau) dst[pv_channel<D>(n, tau)] = acc[st][tau] + z_pv;
    }
    const int jq = 4 * st + hs;          // QK-layout head
    if (g == 0 && lam == 0 && jq < G) {
      const int64_t idx = (hq0 + jq) * a.nsplit + s;
      a.part_ml[idx * 2 + 0] = m_run[st];
      a.part_ml[idx * 2 + 1] = lt;
    }
  }
}

template <int D, int NS>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.nsplit, a.num_kv_heads, a.batch);
  if (a.in_bf16)
    decode_int4_kernel<D, NS, true><<<grid, 64, 0, s>>>(a);
  else
    decode_int4_kernel<D, NS, false><<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ns(const DecodeArgs& a, hipStream_t s) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g <= 4) return launch_d<D, 1>(a, s);
  if (g <= 8) return launch_d<D, 2>(a, s);
  return launch_d<D, 4>(a, s);
}

}  // namespace

hipError_t launch_decode_int4(const DecodeArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_ns<128>(a, s) : launch_ns<64>(a, s);
}

}  // namespace kvq
