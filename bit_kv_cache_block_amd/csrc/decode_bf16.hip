// bf16-KV baseline of the split-K paged decode attention: the same wave
// organisation and online softmax as the INT4 kernel, with bf16 MFMA.  The
// query and the probabilities are each carried as three bf16 limbs (hi, mid,
// lo: 24 significant bits), in the padded columns of the GQA group's tile, so
// the products keep fp32 accuracy against the exact bf16 cache values.
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();

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

template <int D>
__device__ __forceinline__ int pv_channel(int n, int tau) {
  if constexpr (D == 128) return 8 * n + tau;
  else return 8 * (n & 7) + 2 * tau + (n >> 3);
}

__device__ __forceinline__ v8bf as_bf(u32x4 w) { return __builtin_bit_cast(v8bf, w); }

template <int D, int NS, bool QBF16>
__global__ __launch_bounds__(64) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int kSlab = 4 * kPage * D;   // bytes
  constexpr int kNT = D / 16;
  constexpr int kNK = D / 32;            // QK MFMAs per page
  constexpr int kGP = 4 * NS;

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

  // B operand of QK: limb `lam` of head (4st + hs), channels 32mu + 8g .. +7
  u32x4 bq[NS][kNK];
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int mu = 0; mu < kNK; ++mu) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * mu + 8 * g + 2 * i;
        w[i] = static_cast<uint32_t>(bf16_limb(qs[4 * st + hs][c], lam)) |
               (static_cast<uint32_t>(bf16_limb(qs[4 * st + hs][c + 1], lam)) << 16);
      }
      bq[st][mu] = w;
    }

  float m_run[NS], l_run[NS], acc[NS][kNT];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    m_run[st] = kNegInf;
    l_run[st] = 0.0f;
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[st][t] = 0.0f;
  }
  const uint8_t* pool_h = a.pool + static_cast<int64_t>(kvh) * kSlab;
  const int64_t page_stride = static_cast<int64_t>(a.num_kv_heads) * kSlab;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  const int vn = n & (D / 8 - 1);
  const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int p = p0; p < p1; p += 2) {
    u32x4 kx[2][kNK], vx[2][4];
    bool pv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pg = p + i;
      const int pid = pg < p1 ? bt[pg] : -1;
      pv[i] = pid >= 0 && pid < a.num_pages;
      if (pv[i]) {
        const uint8_t* sl = pool_h + static_cast<int64_t>(pid) * page_stride;
#pragma unroll
        for (int mu = 0; mu < kNK; ++mu)
          kx[i][mu] = *reinterpret_cast<const u32x4*>(sl + (n * D + 32 * mu + 8 * g) * 2);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          vx[i][qq] = *reinterpret_cast<const u32x4*>(sl + (kPage * D + (vn * (kPage / 4) + g) * 32) * 2 + 16 * qq);
      } else {
#pragma unroll
        for (int mu = 0; mu < kNK; ++mu) kx[i][mu] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) vx[i][qq] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    float lg[NS][2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        v4f c = zero4;
#pragma unroll
        for (int mu = 0; mu < kNK; ++mu) c = mfma_bf16(as_bf(kx[i][mu]), as_bf(bq[st][mu]), c);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float v = c[rr];
          v += dpp_f<kDppXor1>(v);
          v += dpp_f<kDppXor2>(v);
          const int tok = (p + i) * kPage + 4 * g + rr;
          lg[st][i][rr] = (pv[i] && tok < len) ? v * a.sm_log2 : kNegInf;
        }
      }

    u32x4 apv[NS];
    float alpha_pv[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float mc = kNegInf;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mc = fmaxf(mc, lg[st][i][rr]);
      mc = max_rows(mc);
      const float mnew = fmaxf(m_run[st], mc);
      const float muse = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = exp2f(m_run[st] - muse);
      m_run[st] = mnew;
      float psum = 0.0f;
      uint16_t lb[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float pp = exp2f(lg[st][i][rr] - muse);
          psum += pp;
          lb[i][rr] = bf16_limb(pp, lam);
        }
      l_run[st] = l_run[st] * alpha + psum;
      u32x4 av;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[2 * i] = static_cast<uint32_t>(lb[i][0]) | (static_cast<uint32_t>(lb[i][1]) << 16);
        av[2 * i + 1] = static_cast<uint32_t>(lb[i][2]) | (static_cast<uint32_t>(lb[i][3]) << 16);
      }
      apv[st] = av;
      alpha_pv[st] = lane_read(alpha, 4 * g);
    }

#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) {
      const int jj = (D == 128) ? tau : 2 * tau + (n >> 3);   // channel 8*vn + jj
      u32x4 bv;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // 64 bytes per page = 16 words: channel jj occupies words 2jj, 2jj+1
        const int w0 = 2 * jj;
        bv[2 * i] = vx[i][w0 >> 2][w0 & 3];
        bv[2 * i + 1] = vx[i][(w0 + 1) >> 2][(w0 + 1) & 3];
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const v4f c = mfma_bf16(as_bf(apv[st]), as_bf(bv), zero4);
        const float f = (c[0] + c[1]) + c[2];
        acc[st][tau] = __builtin_fmaf(acc[st][tau], alpha_pv[st], f);
      }
    }
  }

  const int64_t hq0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * G;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const float lt = sum_rows(lam == 0 ? l_run[st] : 0.0f);
    const int jp = 4 * st + g;
    if (jp < G) {
      float* dst = a.part_acc + ((hq0 + jp) * a.nsplit + s) * D;
#pragma unroll
      for (int tau = 0; tau < kNT; ++tau) dst[pv_channel<D>(n, tau)] = acc[st][tau];
    }
    const int jq = 4 * st + hs;
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
    decode_bf16_kernel<D, NS, true><<<grid, 64, 0, s>>>(a);
  else
    decode_bf16_kernel<D, NS, false><<<grid, 64, 0, s>>>(a);
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

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_ns<128>(a, s) : launch_ns<64>(a, s);
}

}  // namespace kvq
