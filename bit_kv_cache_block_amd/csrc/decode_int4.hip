// Read path: split-K paged decode attention over the INT4 cache with the
// dequantization folded into the products ("SAW-INT4", summary page: fused
// attention execution over paged quantized KV; "BitDecoding-FP4", Abstract:
// the query heads of a GQA group stacked into one matrix product per KV page;
// factoring the per-token scale out of the dot product follows the grouping
// idea of "InnerQ", Figure 1).
//
// A workgroup of four waves owns one (sequence b, KV head, split s) and each
// wave streams a quarter of its pages, four pages per step.  Per page and per
// group of four query heads:
//   QK:  C[(head, limb)][token] = sum_c qlimb[c] * code[token][c]   (int8 MFMA)
//        The rotated query is a 23-bit fixed-point integer split into three
//        signed 8-bit limbs (rows of the tile); codes are exact int8; products
//        and sums are exact in int32.  Each lane ends with the four limb rows
//        of one (head, token) and combines them in-lane:
//        logit = sm * 2^(e-22) * (k_scale * sum_c code*qfix + k_zero * sum_c qfix).
//   softmax: online, base 2; one row of 16 lanes = one head.
//   PV:  acc[(head, limb)][c] = sum_t wlimb[t] * code_v[t][c]        (int8 MFMA)
//        w = p * v_scale as a 23-bit fixed-point integer relative to the
//        step's largest w of the head (power-of-two scale), its limbs moved to
//        the operand layout through a 1 KiB LDS tile; sum_t p * v_zero is added
//        to every channel at the end.
// The four waves merge in LDS.  With one split the workgroup normalises,
// rotates back and writes the output; otherwise it writes a partial
// (max, sum, unnormalised output) for the reduce kernel.
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWaves = 4;
constexpr int kStep = 4;   // pages per step

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

// max / sum over the 16 lanes of a row, result in every lane of the row
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
  return fmaxf(x, dpp_f<kDppRowMirror>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppRowHalfMirror>(x);
  return x + dpp_f<kDppRowMirror>(x);
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

template <int D, int NS>
struct Smem {
  static constexpr int kGP = 4 * NS;
  union {
    struct {
      float qs[kGP][D];
      int32_t qi[kGP][D];
    } setup;
    struct {
      float acc[kWaves][kGP][D];
      float m[kWaves][kGP];
      float l[kWaves][kGP];
      float o[kGP][D];
    } merge;
  } u;
  float hA[kGP], hS[kGP];
  uint32_t wl[kWaves][NS][4][4][16];   // [wave][set][limb][head][token] = 4 pages' bytes
};

template <int D, int NS, bool QBF16>
__global__ __launch_bounds__(64 * kWaves) void decode_int4_kernel(DecodeArgs a) {
  constexpr int kSlab = kPage * (D + 8);
  constexpr int kNT = D / 16;          // PV tiles = output channels per lane
  constexpr int kOps = D / 64;         // QK MFMAs per page and head group
  constexpr int kGP = 4 * NS;          // padded heads per KV head
  __shared__ Smem<D, NS> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int g = lane >> 4, n = lane & 15, hs = n >> 2, lam = n & 3;
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.num_q_heads / a.num_kv_heads;

  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const int npg = (len + kPage - 1) / kPage;
  const int p0 = s * a.split_pages;
  const int p1 = min(npg, p0 + a.split_pages);
  if (p0 >= p1) {
    if (a.nsplit == 1) {   // empty sequence: zero output rows
      for (int e = tid; e < G * D; e += 64 * kWaves)
        a.out[(static_cast<int64_t>(b) * a.num_q_heads + kvh * G + e / D) * D + e % D] = 0.0f;
    }
    return;
  }

  // ---- query: load, rotate (fp32 butterfly), fixed point -------------------
  for (int e = tid; e < kGP * D; e += 64 * kWaves) {
    const int j = e / D, c = e % D;
    float v = 0.0f;
    if (j < G) {
      const uint16_t u = a.q[(static_cast<int64_t>(b) * a.num_q_heads + kvh * G + j) * D + c];
      v = QBF16 ? u2f(static_cast<uint32_t>(u) << 16) : static_cast<float>(__builtin_bit_cast(_Float16, u));
    }
    sm.u.setup.qs[j][c] = v;
  }
  for (int e = tid; e < kWaves * NS * 4 * 4 * 16; e += 64 * kWaves)
    (&sm.wl[0][0][0][0][0])[e] = 0u;   // the limb-3 rows stay zero
  __syncthreads();
  if (a.block > 0) {
    for (int hh = 1; hh < a.block; hh *= 2) {
      for (int pi = tid; pi < kGP * D / 2; pi += 64 * kWaves) {
        const int j = pi / (D / 2), q = pi % (D / 2);
        const int i = (q / hh) * (2 * hh) + (q % hh);
        const float u = sm.u.setup.qs[j][i], w = sm.u.setup.qs[j][i + hh];
        sm.u.setup.qs[j][i] = u + w;
        sm.u.setup.qs[j][i + hh] = u - w;
      }
      __syncthreads();
    }
    const float sb = block_norm(a.block);
    for (int e = tid; e < kGP * D; e += 64 * kWaves) sm.u.setup.qs[e / D][e % D] *= sb;
    __syncthreads();
  }
  for (int j = wave; j < kGP; j += kWaves) {   // one wave per head
    float am = 0.0f;
    for (int c = lane; c < D; c += 64) am = fmaxf(am, fabsf(sm.u.setup.qs[j][c]));
    for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
    int ex = 0;
    frexpf(am, &ex);                    // am < 2^ex
    ex = ex < -100 ? -100 : ex;         // keeps 2^(22-ex) finite; smaller q is ~0
    const float sc = ldexpf(1.0f, 22 - ex);
    int32_t sum = 0;
    for (int c = lane; c < D; c += 64) {
      const int32_t v = static_cast<int32_t>(rintf(sm.u.setup.qs[j][c] * sc));
      sm.u.setup.qi[j][c] = v;
      sum += v;
    }
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) {
      sm.hA[j] = a.sm_log2 * ldexpf(1.0f, ex - 22);
      sm.hS[j] = static_cast<float>(sum);
    }
  }
  __syncthreads();

  // A operand of QK: row (head hs, limb lam), k-slots of lane group g
  v4i aq[NS][kOps];
  float qA[NS], qS[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    qA[st] = sm.hA[4 * st + g];          // C-layout head of this lane: row group g
    qS[st] = sm.hS[4 * st + g];
#pragma unroll
    for (int op = 0; op < kOps; ++op) {
      v4i v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w |= limb_byte(sm.u.setup.qi[4 * st + hs][qk_channel<D>(g, op, i, k)], lam) << (8 * k);
        v[i] = static_cast<int32_t>(w);
      }
      aq[st][op] = v;
    }
  }

  // ---- this wave's share of the split's pages --------------------------------
  const int span = p1 - p0;
  const int per_wave = ((span + kWaves - 1) / kWaves + kStep - 1) / kStep * kStep;
  const int pw0 = p0 + wave * per_wave;
  const int pw1 = min(p1, pw0 + per_wave);

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
  const int wl_row = ((0 * 4 + lam) * 4 + hs) * 16 + 4 * g;   // reader offset (set 0) in dwords

  const int k_off = (D == 128) ? n * (D / 2) + g * 16 : n * (D / 2) + g * 8;
  const int v_off = kPage * D / 2 + (vn * kPage + 4 * g) * 4;
  const int km_off = kPage * D + 4 * n;
  for (int p = pw0; p < pw1; p += kStep) {
    // page ids are wave-uniform; an id outside the pool reads page 0 and is
    // masked out of the softmax (the masked path also zeroes its weights)
    int pid[kStep];
    bool pv[kStep];
    bool all_ok = true;
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const int pg = p + i;
      const int id = pg < pw1 ? bt[pg] : -1;
      pv[i] = id >= 0 && id < a.num_pages;
      pid[i] = pv[i] ? id : 0;
      all_ok = all_ok && pv[i];
    }
    const bool tail = !all_ok || (p + kStep) * kPage > len;
    u32x4 kx[kStep], vx[kStep];
    uint32_t km[kStep], vm[kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const uint8_t* sl = pool_h + static_cast<int64_t>(pid[i]) * page_stride;
      if constexpr (D == 128) {
        kx[i] = *reinterpret_cast<const u32x4*>(sl + k_off);
      } else {
        const u32x2 t2 = *reinterpret_cast<const u32x2*>(sl + k_off);
        kx[i] = u32x4{t2[0], t2[1], 0u, 0u};
      }
      vx[i] = *reinterpret_cast<const u32x4*>(sl + v_off);
      km[i] = *reinterpret_cast<const uint32_t*>(sl + km_off);
      vm[i] = *reinterpret_cast<const uint32_t*>(sl + km_off + 4 * kPage);
    }

    // QK: lane (g, n) gets the four limb rows of head g (per set), token n
    float lg[NS][kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      v4i b0, b1;
      if constexpr (D == 128) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          b0[w] = static_cast<int32_t>(kx[i][w] & kLowNibbles);
          b1[w] = static_cast<int32_t>((kx[i][w] >> 4) & kLowNibbles);
        }
      } else {
        b0 = v4i{static_cast<int32_t>(kx[i][0] & kLowNibbles), static_cast<int32_t>(kx[i][1] & kLowNibbles),
                 static_cast<int32_t>((kx[i][0] >> 4) & kLowNibbles),
                 static_cast<int32_t>((kx[i][1] >> 4) & kLowNibbles)};
      }
      const bool ok = !tail || (pv[i] && (p + i) * kPage + n < len);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        v4i c = mfma_i8(aq[st][0], b0, zero4);
        if constexpr (kOps == 2) c = mfma_i8(aq[st][1], b1, c);
        // limbs: c0 * 2^16 + c1 * 2^8 + c2 (c0 * 2^8 + c1 is exact in int32)
        const float tq = __builtin_fmaf(static_cast<float>((c[0] << 8) + c[1]), 256.0f,
                                        static_cast<float>(c[2]));
        const float l2 = qA[st] * __builtin_fmaf(half_hi(km[i]), qS[st], half_lo(km[i]) * tq);
        lg[st][i] = ok ? l2 : kNegInf;
      }
    }

    // online softmax (row = head) and the limbs of w = p * v_scale through LDS
    float alpha[NS], sw[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float mc = fmaxf(fmaxf(lg[st][0], lg[st][1]), fmaxf(lg[st][2], lg[st][3]));
      mc = row_max16(mc);
      const float mnew = fmaxf(m_run[st], mc);
      const float muse = mnew == kNegInf ? 0.0f : mnew;
      alpha[st] = exp2f(m_run[st] - muse);
      m_run[st] = mnew;
      float psum = 0.0f, zsum = 0.0f, wmax = 0.0f, w[kStep];
#pragma unroll
      for (int i = 0; i < kStep; ++i) {
        const float pp = exp2f(lg[st][i] - muse);
        psum += pp;
        if (tail) {
          const bool ok = lg[st][i] != kNegInf;
          zsum += ok ? pp * half_hi(vm[i]) : 0.0f;
          w[i] = ok ? pp * half_lo(vm[i]) : 0.0f;
        } else {
          zsum = __builtin_fmaf(pp, half_hi(vm[i]), zsum);
          w[i] = pp * half_lo(vm[i]);
        }
        wmax = fmaxf(wmax, w[i]);
      }
      l_run[st] = __builtin_fmaf(l_run[st], alpha[st], psum);
      z_run[st] = __builtin_fmaf(z_run[st], alpha[st], zsum);
      wmax = row_max16(wmax);
      int ew = 0;
      frexpf(wmax, &ew);                 // wmax < 2^ew
      ew = ew < -100 ? -100 : ew;        // such a step weighs < 2^-76 of the max
      const float wsc = ldexpf(1.0f, 22 - ew);
      sw[st] = ldexpf(1.0f, ew - 22);
      uint32_t y[kStep];
#pragma unroll
      for (int i = 0; i < kStep; ++i) y[i] = static_cast<uint32_t>(static_cast<int32_t>(rintf(w[i] * wsc)) + 0x8080);
      // limb bytes of the four pages, one word per limb: bytes 2 / 1 / 0 of y
      const uint32_t l0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[3], y[2], 0x0c0c0602u),
                                                __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0602u), 0x05040100u);
      const uint32_t l1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[3], y[2], 0x0c0c0501u),
                                                __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0501u), 0x05040100u) ^ 0x80808080u;
      const uint32_t l2w = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[3], y[2], 0x0c0c0400u),
                                                 __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0400u), 0x05040100u) ^ 0x80808080u;
      uint32_t* wl = &sm.wl[wave][st][0][0][0];
      wl[(0 * 4 + g) * 16 + n] = l0;
      wl[(1 * 4 + g) * 16 + n] = l1;
      wl[(2 * 4 + g) * 16 + n] = l2w;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    v4i apv[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st)
      apv[st] = *reinterpret_cast<const v4i*>(&sm.wl[wave][st][0][0][0] + wl_row);

    // V: per token r of the lane group, transpose across the four pages so a
    // word holds the four pages' codes of one channel pair; nibbles split it.
    uint32_t vt[4][4];   // [r][byte j]
#pragma unroll
    for (int r = 0; r < 4; ++r) transpose_bytes4(vx[0][r], vx[1][r], vx[2][r], vx[3][r], vt[r]);
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) {
      v4i bv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t yv;
        if constexpr (D == 128) yv = (tau & 1) ? (vt[r][tau >> 1] >> 4) : vt[r][tau >> 1];
        else yv = vt[r][tau] >> (4 * (n >> 3));
        bv[r] = static_cast<int32_t>(yv & kLowNibbles);
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const v4i c = mfma_i8(apv[st], bv, zero4);
        const float f = __builtin_fmaf(static_cast<float>((c[0] << 8) + c[1]), 256.0f,
                                       static_cast<float>(c[2]));
        acc[st][tau] = __builtin_fmaf(f, sw[st], acc[st][tau] * alpha[st]);
      }
    }
  }

  // ---- merge the four waves --------------------------------------------------
  __syncthreads();   // setup scratch is reused below
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const float lt = row_sum16(l_run[st]);
    const float zt = row_sum16(z_run[st]);
    const int j = 4 * st + g;            // PV-layout head = row group
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) sm.u.merge.acc[wave][j][pv_channel<D>(n, tau)] = acc[st][tau] + zt;
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
      const float f = exp2f(sm.u.merge.m[w][j] - muse);
      lsum = __builtin_fmaf(sm.u.merge.l[w][j], f, lsum);
      osum = __builtin_fmaf(sm.u.merge.acc[w][j][c], f, osum);
    }
    if (a.nsplit == 1) {
      sm.u.merge.o[j][c] = lsum > 0.0f ? osum / lsum : 0.0f;
    } else {
      const int64_t idx = (hq0 + j) * a.nsplit + s;
      a.part_acc[idx * D + c] = osum;
      if (c == 0) {
        a.part_ml[idx * 2 + 0] = mstar;
        a.part_ml[idx * 2 + 1] = lsum;
      }
    }
  }
  if (a.nsplit != 1) return;
  __syncthreads();
  if (a.block > 0) {
    for (int hh = 1; hh < a.block; hh *= 2) {
      for (int pi = tid; pi < G * D / 2; pi += 64 * kWaves) {
        const int j = pi / (D / 2), q = pi % (D / 2);
        const int i = (q / hh) * (2 * hh) + (q % hh);
        const float u = sm.u.merge.o[j][i], w = sm.u.merge.o[j][i + hh];
        sm.u.merge.o[j][i] = u + w;
        sm.u.merge.o[j][i + hh] = u - w;
      }
      __syncthreads();
    }
  }
  const float sb = a.block > 0 ? block_norm(a.block) : 1.0f;
  for (int e = tid; e < G * D; e += 64 * kWaves)
    a.out[(hq0 + e / D) * D + e % D] = sm.u.merge.o[e / D][e % D] * sb;
}

template <int D, int NS>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.nsplit, a.num_kv_heads, a.batch);
  if (a.in_bf16)
    decode_int4_kernel<D, NS, true><<<grid, 64 * kWaves, 0, s>>>(a);
  else
    decode_int4_kernel<D, NS, false><<<grid, 64 * kWaves, 0, s>>>(a);
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
