/*
 * kvq_oracle.cpp -- plain CPU oracle (test infrastructure only; see the
 * header for who may use it, the method it follows and the readings taken).
 *
 * Written for clarity, not speed: every step is a direct loop over the
 * definition.  Floating point of the quantizer is fp32 exactly as the
 * method's steps state it (built with -ffp-contract=off and no fast-math);
 * attention is fp64.
 */
#include "kvq_oracle.h"

#include <cfenv>
#include <cmath>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

uint32_t bits_of(float x) { uint32_t u; std::memcpy(&u, &x, 4); return u; }

/* Round a finite non-negative double that is exactly a float value to the
 * floating-point grid with `mant_bits` stored mantissa bits, minimum normal
 * exponent `emin` and exponent bias `bias`; returns the bit pattern without
 * sign.  Round to nearest, ties to even (nearbyint under FE_TONEAREST).
 * Values at or beyond the overflow threshold give infinity. */
uint32_t round_to_grid(double a, int mant_bits, int emin, int emax, int bias) {
  if (a == 0.0) return 0;
  int ex = 0;
  std::frexp(a, &ex);          /* a = fr * 2^ex, fr in [0.5, 1) */
  int e = ex - 1;              /* a in [2^e, 2^(e+1)) */
  if (e < emin) {              /* subnormal: multiples of 2^(emin - mant_bits) */
    double m = std::nearbyint(std::ldexp(a, mant_bits - emin));
    return static_cast<uint32_t>(m);  /* m == 2^mant_bits is the smallest normal */
  }
  double m = std::nearbyint(std::ldexp(a, mant_bits - e));  /* in [2^mb, 2^(mb+1)] */
  if (m == std::ldexp(1.0, mant_bits + 1)) { m = std::ldexp(1.0, mant_bits); e += 1; }
  if (e > emax) return static_cast<uint32_t>((emax + bias + 1)) << mant_bits;  /* inf */
  uint32_t mant = static_cast<uint32_t>(m) - (1u << mant_bits);
  return (static_cast<uint32_t>(e + bias) << mant_bits) | mant;
}

uint16_t f32_to_f16(float x) {
  uint32_t u = bits_of(x);
  uint16_t sign = static_cast<uint16_t>((u >> 16) & 0x8000u);
  if (std::isnan(x)) return sign | 0x7e00u;
  if (std::isinf(x)) return sign | 0x7c00u;
  double a = std::fabs(static_cast<double>(x));
  return sign | static_cast<uint16_t>(round_to_grid(a, 10, -14, 15, 15));
}

float f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int mant = h & 0x3ff;
  double v;
  if (ex == 0) v = std::ldexp(static_cast<double>(mant), -24);
  else if (ex == 31) v = mant ? NAN : INFINITY;
  else v = std::ldexp(static_cast<double>(1024 + mant), ex - 25);
  return static_cast<float>(sign ? -v : v);
}

uint16_t f32_to_bf16(float x) {
  uint32_t u = bits_of(x);
  uint16_t sign = static_cast<uint16_t>((u >> 16) & 0x8000u);
  if (std::isnan(x)) return sign | 0x7fc0u;
  if (std::isinf(x)) return sign | 0x7f80u;
  double a = std::fabs(static_cast<double>(x));
  return sign | static_cast<uint16_t>(round_to_grid(a, 7, -126, 127, 127));
}

float bf16_to_f32(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f; std::memcpy(&f, &u, 4);
  return f;
}

float widen(uint16_t h, int dtype) { return dtype == KVQO_F16 ? f16_to_f32(h) : bf16_to_f32(h); }

int popcount(unsigned v) { int c = 0; while (v) { c += v & 1u; v >>= 1; } return c; }

/* Sylvester Hadamard entry (+1 / -1). */
double hadamard(int i, int j) { return (popcount(static_cast<unsigned>(i & j)) & 1) ? -1.0 : 1.0; }

/* In-place fast Walsh-Hadamard transform of n = 2^k fp32 values; stages
 * h = 1, 2, 4, ... in ascending order, each pair (a[k], a[k+h]) replaced by
 * (a[k] + a[k+h], a[k] - a[k+h]). */
void fwht_f32(float* a, int n) {
  for (int h = 1; h < n; h *= 2)
    for (int i = 0; i < n; i += 2 * h)
      for (int k = i; k < i + h; ++k) {
        float x = a[k];
        float y = a[k + h];
        a[k] = x + y;
        a[k + h] = x - y;
      }
}

/* fp64 block rotation with the explicit matrix: y = blockdiag(H_b/sqrt(b)) x.
 * H_b is symmetric, so this is also the inverse rotation. */
void rotate_f64(const double* x, double* y, int d, int b) {
  if (b <= 1) { for (int i = 0; i < d; ++i) y[i] = x[i]; return; }
  double s = 1.0 / std::sqrt(static_cast<double>(b));
  for (int blk = 0; blk < d; blk += b)
    for (int i = 0; i < b; ++i) {
      double acc = 0.0;
      for (int j = 0; j < b; ++j) acc += hadamard(i, j) * x[blk + j];
      y[blk + i] = acc * s;
    }
}

size_t int4_slab(int p, int d) { return static_cast<size_t>(p) * (d + 8); }
size_t int8_slab(int p, int d) { return static_cast<size_t>(p) * (2 * d + 8); }
size_t bf16_slab(int p, int d) { return static_cast<size_t>(2) * p * d * 2; }

/* Byte address helpers of the INT4 slab (layout text in the header). */
size_t k_code_byte(int p, int d, int t, int c) { (void)p; return static_cast<size_t>(t) * (d / 2) + c / 2; }
size_t v_code_byte(int p, int d, int t, int c) {
  int n = c / 8, j = (c % 8) / 2;
  return static_cast<size_t>(p) * d / 2 + (static_cast<size_t>(n) * p + t) * 4 + j;
}
size_t meta_byte(int p, int d, int kind, int t) {
  return static_cast<size_t>(p) * d + static_cast<size_t>(kind) * 4 * p + static_cast<size_t>(t) * 4;
}
/* Byte address helpers of the grouped INT4 slab (layout text in the header). */
size_t int4g_slab(int p, int d, int group) { return static_cast<size_t>(p) * (d + 8 * (d / group)); }
size_t vg_code_byte(int p, int d, int t, int c) {
  int n = c % (d / 8), j = c / (d / 8);  /* word n*P + t, nibble j */
  return static_cast<size_t>(p) * d / 2 + (static_cast<size_t>(n) * p + t) * 4 + j / 2;
}
size_t metag_byte(int p, int d, int group, int kind, int t, int gi) {
  const int ng = d / group;
  return static_cast<size_t>(p) * d + static_cast<size_t>(kind) * 4 * p * ng +
         (static_cast<size_t>(t) * ng + gi) * 4;
}

/* Byte address helpers of the MXFP4 slab (layout text in the header): codes
 * as in the grouped INT4 slab, then one E8M0 byte per 32-channel block. */
size_t mx_slab(int p, int d) { return static_cast<size_t>(p) * (d + d / 16); }
size_t mx_scale_byte(int p, int d, int kind, int t, int blk) {
  return static_cast<size_t>(p) * d + static_cast<size_t>(kind) * p * (d / 32) +
         static_cast<size_t>(t) * (d / 32) + blk;
}

/* Byte address helpers of the INT8 slab (layout text in the header). */
size_t k8_code_byte(int p, int d, int t, int c) { (void)p; return static_cast<size_t>(t) * d + c; }
size_t v8_code_byte(int p, int d, int t, int c) {
  int n = c / 8, h = (c % 8) / 4, j = c % 4;
  return static_cast<size_t>(p) * d + ((static_cast<size_t>(n) * p + t) * 2 + h) * 4 + j;
}
size_t meta8_byte(int p, int d, int kind, int t) {
  return static_cast<size_t>(2) * p * d + static_cast<size_t>(kind) * 4 * p + static_cast<size_t>(t) * 4;
}
size_t bf16_elem(int p, int d, int kind, int t, int c) {
  if (kind == 0) return static_cast<size_t>(t) * d + c;
  int n = c / 8, j = c % 8, g = t / 4, i = t % 4;
  return static_cast<size_t>(p) * d + ((static_cast<size_t>(n) * (p / 4) + g) * 8 + j) * 4 + i;
}

void put_u16(uint8_t* b, uint16_t v) { b[0] = static_cast<uint8_t>(v & 0xff); b[1] = static_cast<uint8_t>(v >> 8); }
uint16_t get_u16(const uint8_t* b) { return static_cast<uint16_t>(b[0] | (b[1] << 8)); }

bool valid_block(int b, int d) { return b == 0 || b == 1 || ((b & (b - 1)) == 0 && b >= 2 && b <= d && d % b == 0); }

}  // namespace

namespace {

/* Shared body of the two paged decode oracles: `read(page, head, off, kind, c)`
 * returns a decoded fp64 element in the cache's basis; `rot` is the block
 * size used to rotate q in and the output back (0 = none). */
template <class Read>
int32_t decode_paged(Read read, int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                     int32_t rot, const uint16_t* q, int32_t dtype, int32_t num_q_heads,
                     const int32_t* block_table, int32_t max_pages_per_seq,
                     const int32_t* seq_lens, int32_t batch, double sm_scale,
                     const uint8_t* mask, double* out) {
  const int d = head_dim, hq = num_q_heads, p = page_size;
  if (num_kv_heads <= 0 || hq % num_kv_heads != 0) return 1;
  const int group = hq / num_kv_heads;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < hq; ++h) {
      double* o = out + (static_cast<size_t>(b) * hq + h) * d;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      if (mask && !mask[static_cast<size_t>(b) * hq + h]) continue;
      const int len = seq_lens[b];
      if (len <= 0) continue;
      const int kvh = h / group;
      std::vector<double> qv(d), qr(d), s(len), orot(d, 0.0);
      for (int c = 0; c < d; ++c) qv[c] = widen(q[(static_cast<size_t>(b) * hq + h) * d + c], dtype);
      rotate_f64(qv.data(), qr.data(), d, rot);
      // a negative page id marks a page that is not there: its tokens are
      // left out of the softmax, and a row with no token left is zero
      double mx = -INFINITY;
      for (int t = 0; t < len; ++t) {
        const int page = block_table[static_cast<size_t>(b) * max_pages_per_seq + t / p];
        if (page < 0) {
          s[t] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += qr[c] * read(page, kvh, t % p, 0, c);
        s[t] = sm_scale * dot;
        if (s[t] > mx) mx = s[t];
      }
      if (mx == -INFINITY) continue;
      double l = 0.0;
      for (int t = 0; t < len; ++t) { s[t] = s[t] == -INFINITY ? 0.0 : std::exp(s[t] - mx); l += s[t]; }
      for (int t = 0; t < len; ++t) {
        const int page = block_table[static_cast<size_t>(b) * max_pages_per_seq + t / p];
        if (page < 0) continue;
        for (int c = 0; c < d; ++c) orot[c] += s[t] * read(page, kvh, t % p, 1, c);
      }
      for (int c = 0; c < d; ++c) orot[c] /= l;
      rotate_f64(orot.data(), o, d, rot);
    }
  return 0;
}

}  // namespace

extern "C" {

uint16_t kvq_oracle_f32_to_f16(float x) { return f32_to_f16(x); }
float kvq_oracle_f16_to_f32(uint16_t h) { return f16_to_f32(h); }
uint16_t kvq_oracle_f32_to_bf16(float x) { return f32_to_bf16(x); }
float kvq_oracle_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }

float kvq_oracle_block_scale(int32_t b) {
  return static_cast<float>(1.0 / std::sqrt(static_cast<double>(b)));
}

void kvq_oracle_rotate(const float* x, float* y, int32_t d, int32_t b) {
  std::vector<float> a(x, x + d);
  if (b > 1) {
    float s = kvq_oracle_block_scale(b);
    for (int blk = 0; blk < d; blk += b) {
      fwht_f32(&a[blk], b);
      for (int i = 0; i < b; ++i) a[blk + i] = a[blk + i] * s;
    }
  }
  for (int i = 0; i < d; ++i) y[i] = a[i];
}

}  // extern "C"

namespace {

/* Codes of R4 under a given fp16 scale and zero point: (y - zero) * (1 /
 * scale), each fp32 operation rounded once, round half to even, clamped to
 * [0, levels]; a zero scale gives 1/scale = 0.  The scale's sign bit is not
 * part of its value (R14 keeps a mode flag there). */
void encode_codes(const float* y, int32_t d, int levels, uint16_t sh, uint16_t zh, uint8_t* codes) {
  std::fesetround(FE_TONEAREST);
  const float top = static_cast<float>(levels);
  float sf = f16_to_f32(static_cast<uint16_t>(sh & 0x7fffu));
  float zf = f16_to_f32(zh);
  float inv = (sf == 0.0f) ? 0.0f : 1.0f / sf;
  for (int i = 0; i < d; ++i) {
    float diff = y[i] - zf;
    float r = diff * inv;
    float c = std::nearbyint(r);
    if (c < 0.0f) c = 0.0f;
    if (c > top) c = top;
    codes[i] = static_cast<uint8_t>(c);
  }
}

/* The asymmetric quantizer of R2, R4, R5 from a given range [lo, hi]:
 * zero = fp16(lo + 0), scale = fp16(((hi - lo) + 0) / levels), then the
 * codes of R4. */
void quantize_range(const float* y, int32_t d, int levels, float lo, float hi, uint8_t* codes,
                    uint16_t* scale, uint16_t* zero) {
  float zero_f = lo + 0.0f;
  float range = (hi - lo) + 0.0f;
  float step = range / static_cast<float>(levels);
  *scale = f32_to_f16(step);
  *zero = f32_to_f16(zero_f);
  encode_codes(y, d, levels, *scale, *zero, codes);
}

/* Token-wise asymmetric quantization of one vector to `levels` + 1 codes
 * 0..levels (15 for INT4, 255 for INT8): the steps of R2, R4 and R5 over the
 * vector's own range. */
void quantize_levels(const float* y, int32_t d, int levels, uint8_t* codes, uint16_t* scale,
                     uint16_t* zero) {
  float mn = y[0], mx = y[0];
  for (int i = 1; i < d; ++i) {
    if (y[i] < mn) mn = y[i];
    if (y[i] > mx) mx = y[i];
  }
  quantize_range(y, d, levels, mn, mx, codes, scale, zero);
}

/* Criterion of R13 and R14: the sum of squared reconstruction errors of y
 * under (codes, scale, zero), measured on the integer grid 2^-k.  Each
 * element is decoded as code * |scale| + zero (the product is exact, the sum
 * rounded once in fp32), its error y - decoded rounded once in fp32, scaled
 * by 2^k and rounded to the nearest integer (ties to even); the squares are
 * summed exactly in 64-bit integers, so the order of the sum does not
 * matter. */
int64_t grid_sse(const float* y, int32_t d, const uint8_t* codes, uint16_t sh, uint16_t zh, int k) {
  std::fesetround(FE_TONEAREST);
  const float sf = f16_to_f32(static_cast<uint16_t>(sh & 0x7fffu));
  const float zf = f16_to_f32(zh);
  int64_t sse = 0;
  for (int i = 0; i < d; ++i) {
    float decoded = static_cast<float>(codes[i]) * sf;
    decoded = decoded + zf;
    const float err = y[i] - decoded;
    const int64_t e = static_cast<int64_t>(std::nearbyint(std::ldexp(err, k)));
    sse += e * e;
  }
  return sse;
}

/* The grid of R13 and R14 for elements of magnitude at most amax: 2^-k with
 * k = 20 - ex, amax < 2^ex (so every error is below 2^21 grid steps). */
int grid_exponent(float amax) {
  int ex = 0;
  std::frexp(amax, &ex);
  return 20 - ex;
}

/* The eight E2M1 magnitudes, in code order. */
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

}  // namespace

extern "C" {

uint8_t kvq_oracle_e2m1_encode(float v) {
  /* round |v| to the nearest E2M1 magnitude, ties to the even code (the one
     with mantissa bit 0), saturating at 6; the sign bit only on nonzero codes */
  const double a = std::fabs(static_cast<double>(v));
  int best = 7;
  if (a < 6.0) {
    best = 0;
    for (int c = 1; c < 8; ++c) {
      const double dc = std::fabs(a - kE2M1[c]), db = std::fabs(a - kE2M1[best]);
      if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
  }
  return static_cast<uint8_t>(best == 0 ? 0 : ((v < 0.0f ? 8 : 0) | best));
}

double kvq_oracle_e2m1_decode(uint8_t code) {
  const double m = kE2M1[code & 7];
  return (code & 8) ? -m : m;
}

void kvq_oracle_quantize_mx(const float* y, int32_t n, uint8_t* codes, uint8_t* scale_e8m0) {
  /* reading R12: shared exponent X = floor(log2(max|y|)) - 2 (2 = the largest
     E2M1 exponent), 2^X stored as the E8M0 byte X + 127; elements y / 2^X
     rounded to E2M1 */
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = std::fmax(amax, std::fabs(y[i]));
  int x = -127;
  if (amax > 0.0f) {
    int e = 0;
    std::frexp(static_cast<double>(amax), &e);   /* amax in [2^(e-1), 2^e) */
    x = (e - 1) - 2;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
  }
  *scale_e8m0 = static_cast<uint8_t>(x + 127);
  for (int i = 0; i < n; ++i)
    codes[i] = kvq_oracle_e2m1_encode(static_cast<float>(std::ldexp(static_cast<double>(y[i]), -x)));
}

void kvq_oracle_quantize(const float* y, int32_t d, uint8_t* codes, uint16_t* scale,
                         uint16_t* zero) {
  quantize_levels(y, d, 15, codes, scale, zero);
}

void kvq_oracle_quantize_int8(const float* y, int32_t d, uint8_t* codes, uint16_t* scale,
                              uint16_t* zero) {
  quantize_levels(y, d, 255, codes, scale, zero);
}

int64_t kvq_oracle_grid_sse(const float* y, int32_t d, const uint8_t* codes, uint16_t scale,
                            uint16_t zero, int32_t k) {
  return grid_sse(y, d, codes, scale, zero, k);
}

int32_t kvq_oracle_grid_exponent(float amax) { return grid_exponent(amax); }

int32_t kvq_oracle_quantize_search(const float* y, int32_t d, uint8_t* codes, uint16_t* scale,
                                   uint16_t* zero) {
  /* R13: the token-wise INT4 quantizer over the range [mn, mx] shrunk toward
     zero by each factor alpha_j = (16 - j) / 16, j = 0 .. 7 (mn * alpha_j and
     mx * alpha_j, one fp32 rounding each; elements outside are clamped by the
     codes' clamp); the candidate with the smallest grid_sse wins, the
     smaller j on a tie.  j = 0 is the plain quantizer. */
  float mn = y[0], mx = y[0];
  for (int i = 1; i < d; ++i) {
    if (y[i] < mn) mn = y[i];
    if (y[i] > mx) mx = y[i];
  }
  const float amax = std::fmax(std::fabs(mn), std::fabs(mx));
  const int k = grid_exponent(amax);
  std::vector<uint8_t> cand(d);
  int64_t best = 0;
  int best_j = -1;
  for (int j = 0; j < 8; ++j) {
    const float alpha = static_cast<float>(16 - j) / 16.0f;
    uint16_t sh, zh;
    quantize_range(y, d, 15, mn * alpha, mx * alpha, cand.data(), &sh, &zh);
    const int64_t e = grid_sse(y, d, cand.data(), sh, zh, k);
    if (best_j < 0 || e < best) {
      best = e;
      best_j = j;
      std::memcpy(codes, cand.data(), static_cast<size_t>(d));
      *scale = sh;
      *zero = zh;
    }
  }
  return best_j;
}

int32_t kvq_oracle_quantize_hybrid(const float* y, int32_t g, uint8_t* codes, uint16_t* scale,
                                   uint16_t* zero) {
  /* R14: two candidates for the group -- asymmetric (R2) and symmetric:
     scale = fp16(amax / 7) with amax = max |y|, zero = -8 * scale (exact in
     fp16 when finite), so that 0 is the level of code 8 and the levels run
     from -8 scale to 7 scale -- each with the codes of R4; the symmetric one
     wins when its grid_sse is not larger (it needs no zero point of its
     own), and is then marked by the sign bit of the stored scale.  A group
     of zeros, or one whose symmetric scale is 0 or whose -8 * scale is not
     finite in fp16, stays asymmetric. */
  uint16_t sa, za;
  quantize_levels(y, g, 15, codes, &sa, &za);
  *scale = sa;
  *zero = za;
  float mn = y[0], mx = y[0];
  for (int i = 1; i < g; ++i) {
    if (y[i] < mn) mn = y[i];
    if (y[i] > mx) mx = y[i];
  }
  const float amax = std::fmax(std::fabs(mn), std::fabs(mx));
  if (amax == 0.0f) return 0;
  const uint16_t ss = f32_to_f16(amax / 7.0f);
  const float sf = f16_to_f32(ss);
  const float zs_f = -8.0f * sf;
  if (sf == 0.0f || !(std::fabs(zs_f) <= 65504.0f)) return 0;
  const uint16_t zs = f32_to_f16(zs_f);   /* exact: a power-of-two multiple */
  std::vector<uint8_t> cs(g);
  encode_codes(y, g, 15, ss, zs, cs.data());
  const int k = grid_exponent(amax);
  if (grid_sse(y, g, cs.data(), ss, zs, k) <= grid_sse(y, g, codes, sa, za, k)) {
    std::memcpy(codes, cs.data(), static_cast<size_t>(g));
    *scale = static_cast<uint16_t>(ss | 0x8000u);
    *zero = zs;
    return 1;
  }
  return 0;
}

size_t kvq_oracle_int4_slab_bytes(int32_t page_size, int32_t head_dim) { return int4_slab(page_size, head_dim); }
size_t kvq_oracle_bf16_slab_bytes(int32_t page_size, int32_t head_dim) { return bf16_slab(page_size, head_dim); }
size_t kvq_oracle_int8_slab_bytes(int32_t page_size, int32_t head_dim) { return int8_slab(page_size, head_dim); }
size_t kvq_oracle_mxfp4_slab_bytes(int32_t page_size, int32_t head_dim) { return mx_slab(page_size, head_dim); }
size_t kvq_oracle_int4g_slab_bytes(int32_t page_size, int32_t head_dim, int32_t group) {
  return int4g_slab(page_size, head_dim, group);
}

}  // extern "C"

namespace {

/* The INT4 append with the key quantizer `kq` (the plain R2 quantizer, or
 * R13's scale search); values always take the plain one. */
template <class KeyQuant>
int32_t append_int4_with(KeyQuant kq, uint8_t* pool, int32_t num_pages, int32_t page_size,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block,
                         const uint16_t* k, const uint16_t* v, int32_t dtype,
                         int64_t token_stride, const int32_t* slot_mapping, int32_t num_tokens) {
  const int p = page_size, d = head_dim, hkv = num_kv_heads;
  if (!valid_block(block, d) || p % 4 != 0 || d % 8 != 0) return 1;
  const size_t slab = int4_slab(p, d);
  const int64_t capacity = static_cast<int64_t>(num_pages) * p;
#pragma omp parallel for schedule(dynamic, 16)
  for (int t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= capacity) continue;
    const int page = static_cast<int>(slot / p), off = static_cast<int>(slot % p);
    std::vector<float> x(d), y(d);
    std::vector<uint8_t> codes(d);
    for (int h = 0; h < hkv; ++h) {
      uint8_t* s = pool + (static_cast<size_t>(page) * hkv + h) * slab;
      for (int kind = 0; kind < 2; ++kind) {
        const uint16_t* src = (kind == 0 ? k : v) + t * token_stride + static_cast<int64_t>(h) * d;
        for (int c = 0; c < d; ++c) x[c] = widen(src[c], dtype);
        kvq_oracle_rotate(x.data(), y.data(), d, block);
        uint16_t sh, zh;
        if (kind == 0) kq(y.data(), d, codes.data(), &sh, &zh);
        else kvq_oracle_quantize(y.data(), d, codes.data(), &sh, &zh);
        for (int c = 0; c < d; c += 2) {
          uint8_t byte = static_cast<uint8_t>(codes[c] | (codes[c + 1] << 4));
          size_t at = kind == 0 ? k_code_byte(p, d, off, c) : v_code_byte(p, d, off, c);
          s[at] = byte;
        }
        put_u16(s + meta_byte(p, d, kind, off), sh);
        put_u16(s + meta_byte(p, d, kind, off) + 2, zh);
      }
    }
  }
  return 0;
}

}  // namespace

extern "C" {

int32_t kvq_oracle_append_int4(uint8_t* pool, int32_t num_pages, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block,
                               const uint16_t* k, const uint16_t* v, int32_t dtype,
                               int64_t token_stride, const int32_t* slot_mapping,
                               int32_t num_tokens) {
  return append_int4_with(kvq_oracle_quantize, pool, num_pages, page_size, num_kv_heads, head_dim,
                          block, k, v, dtype, token_stride, slot_mapping, num_tokens);
}

int32_t kvq_oracle_append_int4_search(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                      const uint16_t* k, const uint16_t* v, int32_t dtype,
                                      int64_t token_stride, const int32_t* slot_mapping,
                                      int32_t num_tokens) {
  auto search = [](const float* y, int32_t d, uint8_t* codes, uint16_t* scale, uint16_t* zero) {
    kvq_oracle_quantize_search(y, d, codes, scale, zero);
  };
  return append_int4_with(search, pool, num_pages, page_size, num_kv_heads, head_dim, block, k, v,
                          dtype, token_stride, slot_mapping, num_tokens);
}

int32_t kvq_oracle_append_int8(uint8_t* pool, int32_t num_pages, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block,
                               const uint16_t* k, const uint16_t* v, int32_t dtype,
                               int64_t token_stride, const int32_t* slot_mapping,
                               int32_t num_tokens) {
  const int p = page_size, d = head_dim, hkv = num_kv_heads;
  if (!valid_block(block, d) || p % 4 != 0 || d % 8 != 0) return 1;
  const size_t slab = int8_slab(p, d);
  const int64_t capacity = static_cast<int64_t>(num_pages) * p;
#pragma omp parallel for schedule(dynamic, 16)
  for (int t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= capacity) continue;
    const int page = static_cast<int>(slot / p), off = static_cast<int>(slot % p);
    std::vector<float> x(d), y(d);
    std::vector<uint8_t> codes(d);
    for (int h = 0; h < hkv; ++h) {
      uint8_t* s = pool + (static_cast<size_t>(page) * hkv + h) * slab;
      for (int kind = 0; kind < 2; ++kind) {
        const uint16_t* src = (kind == 0 ? k : v) + t * token_stride + static_cast<int64_t>(h) * d;
        for (int c = 0; c < d; ++c) x[c] = widen(src[c], dtype);
        kvq_oracle_rotate(x.data(), y.data(), d, block);
        uint16_t sh, zh;
        kvq_oracle_quantize_int8(y.data(), d, codes.data(), &sh, &zh);
        for (int c = 0; c < d; ++c)
          s[kind == 0 ? k8_code_byte(p, d, off, c) : v8_code_byte(p, d, off, c)] = codes[c];
        put_u16(s + meta8_byte(p, d, kind, off), sh);
        put_u16(s + meta8_byte(p, d, kind, off) + 2, zh);
      }
    }
  }
  return 0;
}

}  // extern "C"

namespace {

/* The grouped INT4 append with the group quantizer `gq` (R10's, or R14's
 * hybrid one). */
template <class GroupQuant>
int32_t append_int4g_with(GroupQuant gq, uint8_t* pool, int32_t num_pages, int32_t page_size,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block, int32_t group,
                          const uint16_t* k, const uint16_t* v, int32_t dtype,
                          int64_t token_stride, const int32_t* slot_mapping, int32_t num_tokens) {
  const int p = page_size, d = head_dim, hkv = num_kv_heads;
  if (!valid_block(block, d) || p % 4 != 0 || d % 16 != 0) return 1;
  if (group < 16 || d % group != 0) return 1;
  const size_t slab = int4g_slab(p, d, group);
  const int64_t capacity = static_cast<int64_t>(num_pages) * p;
#pragma omp parallel for schedule(dynamic, 16)
  for (int t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= capacity) continue;
    const int page = static_cast<int>(slot / p), off = static_cast<int>(slot % p);
    std::vector<float> x(d), y(d);
    std::vector<uint8_t> codes(d);
    for (int h = 0; h < hkv; ++h) {
      uint8_t* s = pool + (static_cast<size_t>(page) * hkv + h) * slab;
      for (int kind = 0; kind < 2; ++kind) {
        const uint16_t* src = (kind == 0 ? k : v) + t * token_stride + static_cast<int64_t>(h) * d;
        for (int c = 0; c < d; ++c) x[c] = widen(src[c], dtype);
        kvq_oracle_rotate(x.data(), y.data(), d, block);
        for (int gi = 0; gi < d / group; ++gi) {
          uint16_t sh, zh;
          gq(&y[gi * group], group, &codes[gi * group], &sh, &zh);   /* R10 / R14 */
          put_u16(s + metag_byte(p, d, group, kind, off, gi), sh);
          put_u16(s + metag_byte(p, d, group, kind, off, gi) + 2, zh);
        }
        for (int c = 0; c < d; ++c) {
          size_t at = kind == 0 ? k_code_byte(p, d, off, c) : vg_code_byte(p, d, off, c);
          bool high = kind == 0 ? (c % 2 == 1) : ((c / (d / 8)) % 2 == 1);
          s[at] = static_cast<uint8_t>(high ? ((s[at] & 0x0f) | (codes[c] << 4)) : ((s[at] & 0xf0) | codes[c]));
        }
      }
    }
  }
  return 0;
}

}  // namespace

extern "C" {

int32_t kvq_oracle_append_int4g(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                int32_t group, const uint16_t* k, const uint16_t* v,
                                int32_t dtype, int64_t token_stride, const int32_t* slot_mapping,
                                int32_t num_tokens) {
  return append_int4g_with(kvq_oracle_quantize, pool, num_pages, page_size, num_kv_heads, head_dim,
                           block, group, k, v, dtype, token_stride, slot_mapping, num_tokens);
}

int32_t kvq_oracle_append_int4g_hybrid(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                       int32_t group, const uint16_t* k, const uint16_t* v,
                                       int32_t dtype, int64_t token_stride,
                                       const int32_t* slot_mapping, int32_t num_tokens) {
  auto hybrid = [](const float* y, int32_t g, uint8_t* codes, uint16_t* scale, uint16_t* zero) {
    kvq_oracle_quantize_hybrid(y, g, codes, scale, zero);
  };
  return append_int4g_with(hybrid, pool, num_pages, page_size, num_kv_heads, head_dim, block, group,
                           k, v, dtype, token_stride, slot_mapping, num_tokens);
}

int32_t kvq_oracle_append_mxfp4(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                const uint16_t* k, const uint16_t* v, int32_t dtype,
                                int64_t token_stride, const int32_t* slot_mapping,
                                int32_t num_tokens) {
  const int p = page_size, d = head_dim, hkv = num_kv_heads;
  if (!valid_block(block, d) || p % 4 != 0 || d % 32 != 0) return 1;
  const size_t slab = mx_slab(p, d);
  const int64_t capacity = static_cast<int64_t>(num_pages) * p;
#pragma omp parallel for schedule(dynamic, 16)
  for (int t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= capacity) continue;
    const int page = static_cast<int>(slot / p), off = static_cast<int>(slot % p);
    std::vector<float> x(d), y(d);
    std::vector<uint8_t> codes(d);
    for (int h = 0; h < hkv; ++h) {
      uint8_t* s = pool + (static_cast<size_t>(page) * hkv + h) * slab;
      for (int kind = 0; kind < 2; ++kind) {
        const uint16_t* src = (kind == 0 ? k : v) + t * token_stride + static_cast<int64_t>(h) * d;
        for (int c = 0; c < d; ++c) x[c] = widen(src[c], dtype);
        kvq_oracle_rotate(x.data(), y.data(), d, block);
        for (int b = 0; b < d / 32; ++b)
          kvq_oracle_quantize_mx(&y[32 * b], 32, &codes[32 * b], &s[mx_scale_byte(p, d, kind, off, b)]);
        for (int c = 0; c < d; ++c) {
          size_t at = kind == 0 ? k_code_byte(p, d, off, c) : vg_code_byte(p, d, off, c);
          bool high = kind == 0 ? (c % 2 == 1) : ((c / (d / 8)) % 2 == 1);
          s[at] = static_cast<uint8_t>(high ? ((s[at] & 0x0f) | (codes[c] << 4)) : ((s[at] & 0xf0) | codes[c]));
        }
      }
    }
  }
  return 0;
}

int32_t kvq_oracle_append_bf16(uint8_t* pool, int32_t num_pages, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim,
                               const uint16_t* k, const uint16_t* v, int32_t dtype,
                               int64_t token_stride, const int32_t* slot_mapping,
                               int32_t num_tokens) {
  const int p = page_size, d = head_dim, hkv = num_kv_heads;
  if (p % 4 != 0 || d % 8 != 0) return 1;
  const size_t slab = bf16_slab(p, d);
  const int64_t capacity = static_cast<int64_t>(num_pages) * p;
#pragma omp parallel for schedule(dynamic, 16)
  for (int t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= capacity) continue;
    const int page = static_cast<int>(slot / p), off = static_cast<int>(slot % p);
    for (int h = 0; h < hkv; ++h) {
      uint8_t* s = pool + (static_cast<size_t>(page) * hkv + h) * slab;
      for (int kind = 0; kind < 2; ++kind) {
        const uint16_t* src = (kind == 0 ? k : v) + t * token_stride + static_cast<int64_t>(h) * d;
        for (int c = 0; c < d; ++c) {
          uint16_t b16 = dtype == KVQO_BF16 ? src[c] : f32_to_bf16(f16_to_f32(src[c]));
          put_u16(s + 2 * bf16_elem(p, d, kind, off, c), b16);
        }
      }
    }
  }
  return 0;
}

double kvq_oracle_int4_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page, int32_t head, int32_t off,
                            int32_t kind, int32_t channel, int32_t* code, uint16_t* scale,
                            uint16_t* zero) {
  const int p = page_size, d = head_dim;
  const uint8_t* s = pool + (static_cast<size_t>(page) * num_kv_heads + head) * int4_slab(p, d);
  size_t at = kind == 0 ? k_code_byte(p, d, off, channel) : v_code_byte(p, d, off, channel);
  int c = (channel % 2 == 0) ? (s[at] & 0xf) : (s[at] >> 4);
  uint16_t sh = get_u16(s + meta_byte(p, d, kind, off));
  uint16_t zh = get_u16(s + meta_byte(p, d, kind, off) + 2);
  if (code) *code = c;
  if (scale) *scale = sh;
  if (zero) *zero = zh;
  return static_cast<double>(c) * static_cast<double>(f16_to_f32(sh)) +
         static_cast<double>(f16_to_f32(zh));
}

double kvq_oracle_int8_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page, int32_t head, int32_t off,
                            int32_t kind, int32_t channel, int32_t* code, uint16_t* scale,
                            uint16_t* zero) {
  const int p = page_size, d = head_dim;
  const uint8_t* s = pool + (static_cast<size_t>(page) * num_kv_heads + head) * int8_slab(p, d);
  int c = s[kind == 0 ? k8_code_byte(p, d, off, channel) : v8_code_byte(p, d, off, channel)];
  uint16_t sh = get_u16(s + meta8_byte(p, d, kind, off));
  uint16_t zh = get_u16(s + meta8_byte(p, d, kind, off) + 2);
  if (code) *code = c;
  if (scale) *scale = sh;
  if (zero) *zero = zh;
  return static_cast<double>(c) * static_cast<double>(f16_to_f32(sh)) +
         static_cast<double>(f16_to_f32(zh));
}

double kvq_oracle_int4g_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                             int32_t head_dim, int32_t group, int32_t page, int32_t head,
                             int32_t off, int32_t kind, int32_t channel, int32_t* code,
                             uint16_t* scale, uint16_t* zero) {
  const int p = page_size, d = head_dim;
  const uint8_t* s = pool + (static_cast<size_t>(page) * num_kv_heads + head) * int4g_slab(p, d, group);
  int c;
  if (kind == 0) c = (channel % 2 == 0) ? (s[k_code_byte(p, d, off, channel)] & 0xf) : (s[k_code_byte(p, d, off, channel)] >> 4);
  else c = ((channel / (d / 8)) % 2 == 0) ? (s[vg_code_byte(p, d, off, channel)] & 0xf) : (s[vg_code_byte(p, d, off, channel)] >> 4);
  const size_t m = metag_byte(p, d, group, kind, off, channel / group);
  uint16_t sh = get_u16(s + m), zh = get_u16(s + m + 2);
  if (code) *code = c;
  if (scale) *scale = sh;
  if (zero) *zero = zh;
  /* the scale's sign bit is the hybrid mode flag (R14), not part of it */
  return static_cast<double>(c) * static_cast<double>(f16_to_f32(static_cast<uint16_t>(sh & 0x7fffu))) +
         static_cast<double>(f16_to_f32(zh));
}

double kvq_oracle_mxfp4_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page, int32_t head, int32_t off, int32_t kind,
                             int32_t channel, int32_t* code, uint8_t* scale_e8m0) {
  const int p = page_size, d = head_dim;
  const uint8_t* s = pool + (static_cast<size_t>(page) * num_kv_heads + head) * mx_slab(p, d);
  int c;
  if (kind == 0) c = (channel % 2 == 0) ? (s[k_code_byte(p, d, off, channel)] & 0xf) : (s[k_code_byte(p, d, off, channel)] >> 4);
  else c = ((channel / (d / 8)) % 2 == 0) ? (s[vg_code_byte(p, d, off, channel)] & 0xf) : (s[vg_code_byte(p, d, off, channel)] >> 4);
  const uint8_t e = s[mx_scale_byte(p, d, kind, off, channel / 32)];
  if (code) *code = c;
  if (scale_e8m0) *scale_e8m0 = e;
  return std::ldexp(kvq_oracle_e2m1_decode(static_cast<uint8_t>(c)), static_cast<int>(e) - 127);
}

double kvq_oracle_bf16_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page, int32_t head, int32_t off,
                            int32_t kind, int32_t channel) {
  const int p = page_size, d = head_dim;
  const uint8_t* s = pool + (static_cast<size_t>(page) * num_kv_heads + head) * bf16_slab(p, d);
  return static_cast<double>(bf16_to_f32(get_u16(s + 2 * bf16_elem(p, d, kind, off, channel))));
}


int32_t kvq_oracle_decode_int4(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block, const uint16_t* q, int32_t dtype,
                               int32_t num_q_heads, const int32_t* block_table,
                               int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                               double sm_scale, const uint8_t* mask, double* out) {
  if (!valid_block(block, head_dim)) return 1;
  auto read = [&](int page, int head, int off, int kind, int c) {
    return kvq_oracle_int4_read(pool, page_size, num_kv_heads, head_dim, page, head, off, kind, c,
                                nullptr, nullptr, nullptr);
  };
  return decode_paged(read, page_size, num_kv_heads, head_dim, block, q, dtype, num_q_heads,
                      block_table, max_pages_per_seq, seq_lens, batch, sm_scale, mask, out);
}

int32_t kvq_oracle_decode_int8(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block, const uint16_t* q, int32_t dtype,
                               int32_t num_q_heads, const int32_t* block_table,
                               int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                               double sm_scale, const uint8_t* mask, double* out) {
  if (!valid_block(block, head_dim)) return 1;
  auto read = [&](int page, int head, int off, int kind, int c) {
    return kvq_oracle_int8_read(pool, page_size, num_kv_heads, head_dim, page, head, off, kind, c,
                                nullptr, nullptr, nullptr);
  };
  return decode_paged(read, page_size, num_kv_heads, head_dim, block, q, dtype, num_q_heads,
                      block_table, max_pages_per_seq, seq_lens, batch, sm_scale, mask, out);
}

int32_t kvq_oracle_decode_int4g(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block, int32_t group, const uint16_t* q,
                                int32_t dtype, int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                double sm_scale, const uint8_t* mask, double* out) {
  if (!valid_block(block, head_dim) || group < 16 || head_dim % group != 0) return 1;
  auto read = [&](int page, int head, int off, int kind, int c) {
    return kvq_oracle_int4g_read(pool, page_size, num_kv_heads, head_dim, group, page, head, off,
                                 kind, c, nullptr, nullptr, nullptr);
  };
  return decode_paged(read, page_size, num_kv_heads, head_dim, block, q, dtype, num_q_heads,
                      block_table, max_pages_per_seq, seq_lens, batch, sm_scale, mask, out);
}

int32_t kvq_oracle_decode_mxfp4(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block, const uint16_t* q, int32_t dtype,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                double sm_scale, const uint8_t* mask, double* out) {
  if (!valid_block(block, head_dim) || head_dim % 32 != 0) return 1;
  auto read = [&](int page, int head, int off, int kind, int c) {
    return kvq_oracle_mxfp4_read(pool, page_size, num_kv_heads, head_dim, page, head, off, kind, c,
                                 nullptr, nullptr);
  };
  return decode_paged(read, page_size, num_kv_heads, head_dim, block, q, dtype, num_q_heads,
                      block_table, max_pages_per_seq, seq_lens, batch, sm_scale, mask, out);
}

int32_t kvq_oracle_decode_bf16(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                               int32_t head_dim, const uint16_t* q, int32_t dtype,
                               int32_t num_q_heads, const int32_t* block_table,
                               int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                               double sm_scale, const uint8_t* mask, double* out) {
  auto read = [&](int page, int head, int off, int kind, int c) {
    return kvq_oracle_bf16_read(pool, page_size, num_kv_heads, head_dim, page, head, off, kind, c);
  };
  return decode_paged(read, page_size, num_kv_heads, head_dim, 0, q, dtype, num_q_heads,
                      block_table, max_pages_per_seq, seq_lens, batch, sm_scale, mask, out);
}

int32_t kvq_oracle_decode_windowed(const uint8_t* int4_pool, const uint8_t* win_pool,
                                   int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block, const uint16_t* q, int32_t dtype,
                                   int32_t num_q_heads, const int32_t* block_table,
                                   int32_t max_pages_per_seq, const int32_t* win_block_table,
                                   int32_t max_win_pages, const int32_t* seq_lens, int32_t batch,
                                   int32_t w_sink, int32_t w_recent, double sm_scale,
                                   const uint8_t* mask, double* out) {
  const int d = head_dim, hq = num_q_heads, p = page_size;
  if (!valid_block(block, d) || num_kv_heads <= 0 || hq % num_kv_heads != 0) return 1;
  if (w_sink < 0 || w_recent < 0) return 1;
  const int group = hq / num_kv_heads;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < hq; ++h) {
      double* o = out + (static_cast<size_t>(b) * hq + h) * d;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      if (mask && !mask[static_cast<size_t>(b) * hq + h]) continue;
      const int len = seq_lens[b];
      if (len <= 0) continue;
      const int kvh = h / group;
      std::vector<double> qv(d), qr(d), s(len), o_int4(d, 0.0), o_win(d, 0.0), tmp(d);
      for (int c = 0; c < d; ++c) qv[c] = widen(q[(static_cast<size_t>(b) * hq + h) * d + c], dtype);
      rotate_f64(qv.data(), qr.data(), d, block);
      /* token t lives in the bf16 window when it is one of the first w_sink
         or of the last w_recent tokens; window position: sinks in order, then
         a ring of w_recent slots indexed by (t - w_sink) mod w_recent */
      auto in_window = [&](int t) { return t < w_sink || t >= len - w_recent; };
      auto win_page_off = [&](int t, int* page, int* off) {
        const int pos = t < w_sink ? t : w_sink + (t - w_sink) % w_recent;
        *page = win_block_table[static_cast<size_t>(b) * max_win_pages + pos / p];
        *off = pos % p;
      };
      /* page of token t in the table that holds it (window or INT4) and its
         offset there; a negative id is a page that is not there, whose
         tokens are left out of the softmax (a row with none left is zero) */
      auto where = [&](int t, int* page, int* off) {
        if (in_window(t)) {
          win_page_off(t, page, off);
        } else {
          *page = block_table[static_cast<size_t>(b) * max_pages_per_seq + t / p];
          *off = t % p;
        }
      };
      double mx = -INFINITY;
      for (int t = 0; t < len; ++t) {
        int page, off;
        where(t, &page, &off);
        if (page < 0) {
          s[t] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        if (in_window(t)) {   /* original basis, un-rotated query */
          for (int c = 0; c < d; ++c)
            dot += qv[c] * kvq_oracle_bf16_read(win_pool, p, num_kv_heads, d, page, kvh, off, 0, c);
        } else {              /* rotated basis, rotated query */
          for (int c = 0; c < d; ++c)
            dot += qr[c] * kvq_oracle_int4_read(int4_pool, p, num_kv_heads, d, page, kvh, off, 0, c,
                                                nullptr, nullptr, nullptr);
        }
        s[t] = sm_scale * dot;
        if (s[t] > mx) mx = s[t];
      }
      if (mx == -INFINITY) continue;
      double l = 0.0;
      for (int t = 0; t < len; ++t) { s[t] = s[t] == -INFINITY ? 0.0 : std::exp(s[t] - mx); l += s[t]; }
      for (int t = 0; t < len; ++t) {
        int page, off;
        where(t, &page, &off);
        if (page < 0) continue;
        if (in_window(t)) {
          for (int c = 0; c < d; ++c)
            o_win[c] += s[t] * kvq_oracle_bf16_read(win_pool, p, num_kv_heads, d, page, kvh, off, 1, c);
        } else {
          for (int c = 0; c < d; ++c)
            o_int4[c] += s[t] * kvq_oracle_int4_read(int4_pool, p, num_kv_heads, d, page, kvh, off, 1, c,
                                                     nullptr, nullptr, nullptr);
        }
      }
      rotate_f64(o_int4.data(), tmp.data(), d, block);   /* back to the original basis */
      for (int c = 0; c < d; ++c) o[c] = (tmp[c] + o_win[c]) / l;
    }
  return 0;
}

int32_t kvq_oracle_decode_int4_bruteforce(const uint8_t* pool, int32_t page_size,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                          const uint16_t* q, int32_t dtype, int32_t num_q_heads,
                                          const int32_t* block_table, int32_t max_pages_per_seq,
                                          const int32_t* seq_lens, int32_t batch, double sm_scale,
                                          double* out) {
  const int d = head_dim, hq = num_q_heads, p = page_size;
  if (!valid_block(block, d) || num_kv_heads <= 0 || hq % num_kv_heads != 0) return 1;
  const int group = hq / num_kv_heads;
  /* the explicit inverse rotation matrix, dense d x d */
  std::vector<double> rinv(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) {
    if (block <= 1) { rinv[static_cast<size_t>(i) * d + i] = 1.0; continue; }
    int blk = i / block;
    for (int j = 0; j < block; ++j)
      rinv[static_cast<size_t>(i) * d + blk * block + j] =
          hadamard(j, i % block) / std::sqrt(static_cast<double>(block));
  }
  for (int b = 0; b < batch; ++b) {
    const int len = seq_lens[b];
    for (int h = 0; h < hq; ++h) {
      double* o = out + (static_cast<size_t>(b) * hq + h) * d;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      if (len <= 0) continue;
      const int kvh = h / group;
      /* gather + un-rotate */
      std::vector<double> kk(static_cast<size_t>(len) * d), vv(static_cast<size_t>(len) * d);
      std::vector<double> rk(d), rv(d);
      for (int t = 0; t < len; ++t) {
        const int page = block_table[static_cast<size_t>(b) * max_pages_per_seq + t / p];
        for (int c = 0; c < d; ++c) {
          rk[c] = kvq_oracle_int4_read(pool, p, num_kv_heads, d, page, kvh, t % p, 0, c, nullptr, nullptr, nullptr);
          rv[c] = kvq_oracle_int4_read(pool, p, num_kv_heads, d, page, kvh, t % p, 1, c, nullptr, nullptr, nullptr);
        }
        for (int i = 0; i < d; ++i) {
          double ak = 0.0, av = 0.0;
          for (int j = 0; j < d; ++j) {
            ak += rinv[static_cast<size_t>(i) * d + j] * rk[j];
            av += rinv[static_cast<size_t>(i) * d + j] * rv[j];
          }
          kk[static_cast<size_t>(t) * d + i] = ak;
          vv[static_cast<size_t>(t) * d + i] = av;
        }
      }
      std::vector<double> qv(d), sc(len);
      for (int c = 0; c < d; ++c) qv[c] = widen(q[(static_cast<size_t>(b) * hq + h) * d + c], dtype);
      double mx = -INFINITY;
      for (int t = 0; t < len; ++t) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += qv[c] * kk[static_cast<size_t>(t) * d + c];
        sc[t] = sm_scale * dot;
        mx = sc[t] > mx ? sc[t] : mx;
      }
      double l = 0.0;
      for (int t = 0; t < len; ++t) { sc[t] = std::exp(sc[t] - mx); l += sc[t]; }
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int t = 0; t < len; ++t) acc += sc[t] * vv[static_cast<size_t>(t) * d + c];
        o[c] = acc / l;
      }
    }
  }
  return 0;
}

int32_t kvq_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void kvq_oracle_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

}  // extern "C"
