/*
 * srft_oracle.c -- plain, slow CPU oracle for the SRFT fixed-rate KV codec (signed int4 or int8
 * codes, per-group absmax scales).
 *
 * TEST INFRASTRUCTURE ONLY, like hq_oracle.c beside it (same library): only the tests, the smoke
 * check and the benchmark's CPU-baseline leg load it; the GPU product never links, loads or calls
 * it, and the two share no code.
 *
 * What it computes follows the technical summary "When quantization is free"
 * (gist.science/ko/paper/2605.05699), section "Methodology":
 *   1. SRFT(x) = pack(F diag(s) x) with F the unitary DFT and s a fixed random sign vector;
 *   2. the fused kernel's steps: load and sign, radix-2 Stockham FFT passes over d/2 complex points,
 *      Hermitian unpack to a real representation, per-channel lambda rescaling, per-group absmax,
 *      rounding to signed int4 / int8, two int4 codes per byte;
 *   3. per-channel plus per-group scaling with 16 groups.
 * The pages fix none of the arithmetic.  The readings taken (stated at each function):
 *   - d = 128 values per vector (one KV head vector); s is the codec's sign diagonal: s_i = -1 iff
 *     bit i mod 32 of word i/32 of Philox4x32-10(key = seed, counter 0) is set (hqo_signs);
 *   - the real length-d DFT runs as a complex length-64 FFT of z_n = x_2n + i x_2n+1, radix-2
 *     Stockham passes (natural-order output), then the Hermitian unpack;
 *   - pack: y_0 = X_0 / sqrt(d), y_1 = X_{d/2} / sqrt(d), y_2k = sqrt(2) Re X_k / sqrt(d),
 *     y_2k+1 = sqrt(2) Im X_k / sqrt(d) (k = 1..63): an orthogonal real d x d map;
 *   - lambda: v_c = y_c / lambda_c, one positive scale per packed coordinate (caller's calibration;
 *     all ones when none is given), applied as one binary32 multiplier per coordinate;
 *   - groups: 16 contiguous groups of 8 packed coordinates; scale Delta_g = binary16(absmax_g / L)
 *     with L = 7 (int4) or 127 (int8), round to nearest even, saturating at 65504; codes
 *     q = clamp(rint(v * (1 / Delta_g)), -L, L), rint half to even; a zero scale gives zero codes;
 *   - a vector with a non-finite packed coordinate gets all-zero codes and every scale 0x7E00 (a
 *     binary16 NaN), so that its decode is NaN;
 *   - storage: codes [vectors][64] bytes (int4: code 2j in the low nibble of byte j, 2j+1 in the
 *     high nibble, two's complement) or [vectors][128] (int8); scales [vectors][16] binary16.
 * Every binary32 step is rounded once in the order written (build with -ffp-contract=off), because
 * the GPU takes the same integer decisions in binary32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D 128
#define NC 64      /* complex FFT length d/2 */
#define GROUPS 16
#define GSIZE 8

void hqo_signs(uint64_t seed, float d[D]); /* hq_oracle.c: the codec's sign diagonal */

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* Twiddle (cos, sin) of the angle 2 pi k / n, as binary32.  Only the first octant comes from the
 * binary64 library cos and sin (angle 2 pi r / n computed in binary64, result rounded to binary32);
 * the rest of the circle follows by the exact symmetries, so that quadrant points are exactly 0 and
 * +-1 and the table is symmetric bit for bit. */
void hqo_srft_twiddle(uint32_t n, uint32_t k, float cs[2]) {
  const double two_pi = 6.283185307179586476925286766559;
  const uint32_t quarter = n / 4, quad = (k % n) / quarter, r = (k % n) % quarter;
  float c0, s0;
  if (2 * r <= quarter) {
    c0 = (float)cos(two_pi * (double)r / (double)n);
    s0 = (float)sin(two_pi * (double)r / (double)n);
  } else {
    c0 = (float)sin(two_pi * (double)(quarter - r) / (double)n);
    s0 = (float)cos(two_pi * (double)(quarter - r) / (double)n);
  }
  switch (quad) { /* rotation by quad quarter turns; 0 - u keeps exact zeros at +0 */
    case 0: cs[0] = c0; cs[1] = s0; break;
    case 1: cs[0] = 0.0f - s0; cs[1] = c0; break;
    case 2: cs[0] = 0.0f - c0; cs[1] = 0.0f - s0; break;
    default: cs[0] = s0; cs[1] = 0.0f - c0; break;
  }
}

/* (a + i b)(c + i e): real part a c - b e, imaginary part a e + b c; each product and each sum
 * rounded once. */
static void cmul(float a, float b, float c, float e, float *re, float *im) {
  float ac = a * c, be = b * e, ae = a * e, bc = b * c;
  *re = ac - be;
  *im = ae + bc;
}

/* Complex FFT of length 64 in binary32, radix-2 Stockham (autosort) passes with sub-transform
 * length Ns = 1, 2, ..., 32: for j = 0..31, v0 = a[j], v1 = a[j + 32],
 * t = v1 * w^((j mod Ns) * 32 / Ns) with w = exp(-+2 pi i / 64), and the outputs v0 + t, v0 - t go
 * to positions (j / Ns) 2 Ns + (j mod Ns) and that + Ns.  Forward (sign -) or inverse (sign +),
 * unnormalised. */
static void fft64(float re[NC], float im[NC], int inverse) {
  float bre[NC], bim[NC];
  for (int ns = 1; ns < NC; ns *= 2) {
    for (int j = 0; j < NC / 2; ++j) {
      float cs[2];
      hqo_srft_twiddle(NC, (uint32_t)((j % ns) * (NC / (2 * ns))), cs);
      float wr = cs[0], wi = inverse ? cs[1] : -cs[1];
      float tr, ti;
      cmul(re[j + NC / 2], im[j + NC / 2], wr, wi, &tr, &ti);
      int o = (j / ns) * 2 * ns + (j % ns);
      bre[o] = re[j] + tr;
      bim[o] = im[j] + ti;
      bre[o + ns] = re[j] - tr;
      bim[o + ns] = im[j] - ti;
    }
    memcpy(re, bre, sizeof(bre));
    memcpy(im, bim, sizeof(bim));
  }
}

/* Per-coordinate multipliers m_c = sigma_c * (1 / lambda_c), each rounded once: sigma_0 = sigma_1
 * = binary32(1 / sqrt(128)) for X_0 and X_64, sigma_c = 1/16 for the others (sqrt(2) / sqrt(128)
 * times the 1/2 the unpack below leaves out).  Returns 0, or -1 for a lambda that is not finite and
 * positive. */
static int multipliers(const float *lam, float m[D]) {
  const float s0 = (float)(1.0 / sqrt(128.0));
  for (int c = 0; c < D; ++c) {
    float l = lam ? lam[c] : 1.0f;
    if (!(l > 0.0f) || !isfinite(l)) return -1;
    float r = 1.0f / l;
    m[c] = (c < 2 ? s0 : 0.0625f) * r;
  }
  return 0;
}

/* v = SRFT(x) / lambda for one vector (binary32): signs, packing of even / odd samples into 64
 * complex values, the FFT, the Hermitian unpack and the multipliers.  Unpack, for k = 1..63 with
 * Z = FFT(z): E = Z_k + conj(Z_{64-k}), G = Z_k - conj(Z_{64-k}), X'_k = E + W^k (-i G) with
 * W = exp(-2 pi i / 128); X'_k is 2 X_k (the unnormalised DFT of x).  X_0 = Re Z_0 + Im Z_0 and
 * X_64 = Re Z_0 - Im Z_0.  Then v_0 = X_0 m_0, v_1 = X_64 m_1, v_2k = Re X'_k m_2k,
 * v_2k+1 = Im X'_k m_2k+1. */
static void forward(const float x[D], const float sgn[D], const float m[D], float v[D]) {
  float re[NC], im[NC];
  for (int n = 0; n < NC; ++n) {
    re[n] = x[2 * n] * sgn[2 * n];
    im[n] = x[2 * n + 1] * sgn[2 * n + 1];
  }
  fft64(re, im, 0);
  v[0] = (re[0] + im[0]) * m[0];
  v[1] = (re[0] - im[0]) * m[1];
  for (int k = 1; k < NC; ++k) {
    float er = re[k] + re[NC - k], ei = im[k] - im[NC - k];  /* Z_k + conj(Z_{64-k}) */
    float gr = re[k] - re[NC - k], gi = im[k] + im[NC - k];  /* Z_k - conj(Z_{64-k}) */
    float cs[2], pr, pi;
    hqo_srft_twiddle(D, (uint32_t)k, cs);
    cmul(gi, -gr, cs[0], -cs[1], &pr, &pi); /* W^k (-i G), -i G = (gi, -gr) */
    v[2 * k] = (er + pr) * m[2 * k];
    v[2 * k + 1] = (ei + pi) * m[2 * k + 1];
  }
}

/* y (packed, before lambda) back to x: for k = 1..63 with Y_k = y_2k + i y_2k+1,
 * Zt_k = (Y_k + conj(Y_{64-k})) + i P with P = W^-k (Y_k - conj(Y_{64-k})); Zt_0 =
 * ((y_0 + y_1) + i (y_0 - y_1)) sqrt(2); z = inverse FFT(Zt) / 16; x_2n = Re z_n s_2n,
 * x_2n+1 = Im z_n s_2n+1.  This is the transpose of the forward map (the 1/16 and sqrt(2) are its
 * scale factors relative to the packed coordinates). */
static void inverse(const float y[D], const float sgn[D], float x[D]) {
  float re[NC], im[NC];
  const float r2 = (float)sqrt(2.0);
  re[0] = (y[0] + y[1]) * r2;
  im[0] = (y[0] - y[1]) * r2;
  for (int k = 1; k < NC; ++k) {
    float ar = y[2 * k], ai = y[2 * k + 1], br = y[2 * (NC - k)], bi = -y[2 * (NC - k) + 1];
    float sr = ar + br, si = ai + bi, dr = ar - br, di = ai - bi;
    float cs[2], pr, pi;
    hqo_srft_twiddle(D, (uint32_t)k, cs);
    cmul(dr, di, cs[0], cs[1], &pr, &pi); /* W^-k (Y_k - conj(Y_{64-k})) */
    re[k] = sr - pi;                        /* + i P: real part -Im P */
    im[k] = si + pr;
  }
  fft64(re, im, 1);
  for (int n = 0; n < NC; ++n) {
    x[2 * n] = (re[n] * 0.0625f) * sgn[2 * n];
    x[2 * n + 1] = (im[n] * 0.0625f) * sgn[2 * n + 1];
  }
}

/* binary16 bits of a finite t >= 0, round to nearest even, saturating at 65504.  Written from the
 * definition: quantum 2^(e - 11) for t in [2^(e-1), 2^e) (11 significant bits), at least 2^-24
 * (subnormals). */
static uint16_t f16_rne_sat(float t) {
  if (t >= 65504.0f) return 0x7BFF;
  if (t == 0.0f) return 0;
  int e;
  frexp((double)t, &e);
  double q = ldexp(1.0, e - 11 < -24 ? -24 : e - 11);
  double r = (double)t / q, ip = floor(r), fr = r - ip;
  if (fr > 0.5 || (fr == 0.5 && fmod(ip, 2.0) == 1.0)) ip += 1.0;
  double h = ip * q; /* exact */
  if (h == 0.0) return 0;
  if (h < ldexp(1.0, -14)) return (uint16_t)(h / ldexp(1.0, -24)); /* subnormal: count of 2^-24 */
  int he;
  double hf = frexp(h, &he); /* h = hf 2^he, hf in [0.5, 1) */
  uint32_t mant = (uint32_t)(ldexp(hf, 11)) - 1024u;
  return (uint16_t)(((uint32_t)(he - 1 + 15) << 10) | mant);
}

static float f16_to_f32(uint16_t h) {
  uint32_t e = (h >> 10) & 31u, m = h & 1023u, s = (uint32_t)(h >> 15);
  double v;
  if (e == 31) return f32_from_bits((s << 31) | 0x7F800000u | (m << 13));
  if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp((double)(m | 1024u), (int)e - 25);
  return (float)(s ? -v : v);
}

static float bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = bits_from_f32(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* Exposed for the pins: v = SRFT(x) / lambda of one vector (lam may be NULL). */
int hqo_srft_forward(const float *x, uint64_t seed, const float *lam, float *v) {
  float sgn[D], m[D];
  if (multipliers(lam, m)) return -1;
  hqo_signs(seed, sgn);
  forward(x, sgn, m, v);
  return 0;
}

/* Exposed for the pins: x = SRFT^-1(y) of one vector (no lambda). */
void hqo_srft_inverse(const float *y, uint64_t seed, float *x) {
  float sgn[D];
  hqo_signs(seed, sgn);
  inverse(y, sgn, x);
}

/* Encode n values (dtype 0: binary32, 1: bfloat16) as n/128 vectors.  bits = 4 or 8.  Returns 0,
 * or -1 on a bad argument. */
int hqo_srft_encode(const void *x, int dtype, uint64_t n, uint64_t seed, const float *lam, int bits,
                    uint8_t *codes, uint16_t *scales) {
  if (n % D || (bits != 4 && bits != 8) || (dtype != 0 && dtype != 1)) return -1;
  float sgn[D], m[D];
  if (multipliers(lam, m)) return -1;
  hqo_signs(seed, sgn);
  const int lim = bits == 4 ? 7 : 127;
  const uint64_t cbytes = bits == 4 ? D / 2 : D;
  for (uint64_t t = 0; t < n / D; ++t) {
    float xin[D], v[D];
    for (int i = 0; i < D; ++i)
      xin[i] = dtype == 0 ? ((const float *)x)[t * D + i] : bf16_to_f32(((const uint16_t *)x)[t * D + i]);
    forward(xin, sgn, m, v);
    int bad = 0;
    for (int c = 0; c < D; ++c) bad |= !isfinite(v[c]);
    int32_t q[D];
    uint16_t *sc = scales + t * GROUPS;
    for (int g = 0; g < GROUPS; ++g) {
      if (bad) {
        sc[g] = 0x7E00;
        for (int c = 0; c < GSIZE; ++c) q[g * GSIZE + c] = 0;
        continue;
      }
      float a = 0.0f;
      for (int c = 0; c < GSIZE; ++c) a = fmaxf(a, fabsf(v[g * GSIZE + c]));
      uint16_t h = f16_rne_sat(a / (float)lim);
      sc[g] = h;
      float delta = f16_to_f32(h);
      float inv = delta > 0.0f ? 1.0f / delta : 0.0f;
      for (int c = 0; c < GSIZE; ++c) {
        float r = nearbyintf(v[g * GSIZE + c] * inv);
        q[g * GSIZE + c] = delta > 0.0f ? (int32_t)fminf(fmaxf(r, (float)-lim), (float)lim) : 0;
      }
    }
    uint8_t *cp = codes + t * cbytes;
    if (bits == 4) {
      for (int j = 0; j < D / 2; ++j) cp[j] = (uint8_t)((q[2 * j] & 15) | ((q[2 * j + 1] & 15) << 4));
    } else {
      for (int c = 0; c < D; ++c) cp[c] = (uint8_t)(int8_t)q[c];
    }
  }
  return 0;
}

/* Decode: y_c = (q_c Delta_g) lambda_c (each product rounded once), then the inverse transform;
 * output binary32 (out_dtype 0) or bfloat16 round to nearest even (1).  An exactly-zero result is
 * +0. */
int hqo_srft_decode(const uint8_t *codes, const uint16_t *scales, uint64_t n, uint64_t seed, const float *lam,
                    int bits, void *out, int out_dtype) {
  if (n % D || (bits != 4 && bits != 8) || (out_dtype != 0 && out_dtype != 1)) return -1;
  for (int c = 0; c < D && lam; ++c)
    if (!(lam[c] > 0.0f) || !isfinite(lam[c])) return -1;
  float sgn[D];
  hqo_signs(seed, sgn);
  const uint64_t cbytes = bits == 4 ? D / 2 : D;
  for (uint64_t t = 0; t < n / D; ++t) {
    const uint8_t *cp = codes + t * cbytes;
    float y[D], xo[D];
    for (int c = 0; c < D; ++c) {
      int32_t q;
      if (bits == 4) {
        int nib = (cp[c / 2] >> (4 * (c & 1))) & 15;
        q = nib >= 8 ? nib - 16 : nib;
      } else {
        q = (int8_t)cp[c];
      }
      float delta = f16_to_f32(scales[t * GROUPS + c / GSIZE]);
      y[c] = ((float)q * delta) * (lam ? lam[c] : 1.0f);
    }
    inverse(y, sgn, xo);
    for (int i = 0; i < D; ++i) {
      float f = xo[i] == 0.0f ? 0.0f : xo[i];
      if (out_dtype == 0) ((float *)out)[t * D + i] = f;
      else ((uint16_t *)out)[t * D + i] = f32_to_bf16_rne(f);
    }
  }
  return 0;
}
