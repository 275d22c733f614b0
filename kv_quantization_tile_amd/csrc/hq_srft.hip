// hq_srft.hip -- the SRFT fixed-rate KV codec: signed int4 (or int8) codes with per-group binary16
// absmax scales, one thread per 128-value vector.
//
// "When quantization is free" technical summary (gist.science/ko/paper/2605.05699), section
// "Methodology": 1. SRFT(x) = pack(F diag(s) x), F the unitary DFT, s fixed random signs; 2. one
// fused kernel -- load and sign in registers, radix-2 Stockham FFT passes over d/2 points, Hermitian
// unpack to reals, per-channel lambda, per-group absmax, rounding to signed int4 / int8, two codes per
// byte; 3. per-channel plus per-group (16 groups) scaling.
//
// Arithmetic, fixed so that codes are reproducible (each binary32 operation rounded once, in this
// order; the library is built without contraction):
//   - s_i = -1 iff bit i mod 32 of word i/32 of Philox4x32-10(key = seed, counter 0) is set (the
//     sign diagonal of the lattice codec, so both codecs see the same signs for the same seed);
//   - z_n = s_2n x_2n + i s_2n+1 x_2n+1 (n = 0..63), Z = FFT_64(z): Stockham passes Ns = 1..32,
//     j = 0..31: t = a[j + 32] w^((j mod Ns) 32 / Ns), outputs a[j] +- t to (j / Ns) 2 Ns + j mod Ns
//     and + Ns; complex products as (ac - be) + i (ae + bc);
//   - unpack: X_0 = Re Z_0 + Im Z_0, X_64 = Re Z_0 - Im Z_0; k = 1..63: E = Z_k + conj Z_{64-k},
//     G = Z_k - conj Z_{64-k}, X'_k = E + W^k (-i G), W = exp(-2 pi i / 128);
//   - v = (X_0, X_64, Re X'_1, Im X'_1, ...) times m_c = sigma_c (1 / lambda_c), sigma = 1/sqrt(128)
//     for the first two and 1/16 for the rest (the packed coordinates of an orthogonal map);
//   - 16 groups of 8: Delta = binary16(absmax / L) (nearest even, saturating at 65504), L = 7 or 127;
//     q = clamp(rint(v (1 / Delta)), -L, L); a vector with a non-finite v gets zero codes and NaN
//     (0x7E00) scales;
//   - decode: y_c = (q Delta) lambda_c, then the transpose: Zt_0 = ((y_0 + y_1) + i (y_0 - y_1))
//     sqrt(2), Zt_k = (Y_k + conj Y_{64-k}) + i W^-k (Y_k - conj Y_{64-k}), z = inverse FFT_64(Zt),
//     x = s (z / 16), exact zeros as +0.
// Twiddles are binary32 roundings of binary64 cos and sin over the first octant, the rest of the
// circle by exact symmetry; they travel in the kernel argument with the multipliers.
// Products by the exact twiddles 1 and -+i are not formed; that changes at most the sign of a zero
// result, which no code and no nonzero output depends on.  The quotients absmax / L and 1 / Delta are
// formed by FMA schemes equal to the correctly rounded quotient (div_l, recip_f16_value).
// Register budget: the 64 complex points are the working set of a thread; the unpacks take k and
// 64 - k together so that inputs die as outputs appear, which keeps a thread near 160 registers
// (three wavefronts per SIMD).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/hq.h"
#include "hq_device.h"

namespace hq_srft {

constexpr int kD = 128;        // values per vector
constexpr int kN = 64;         // complex FFT length
constexpr int kGroups = 16;    // scale groups per vector
constexpr int kBlock = 256;    // one vector per thread

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct Consts {
  float w64c[32], w64s[32];    // cos, sin of 2 pi k / 64
  float w128c[64], w128s[64];  // cos, sin of 2 pi k / 128
  float m[kD];                 // encode multipliers sigma_c / lambda_c
  float lam[kD];               // decode multipliers lambda_c
};

// ---------------------------------------------------------------------------------------------
// Host: the constant tables.

static void twiddle(uint32_t n, uint32_t k, float* c, float* s) {
  const double two_pi = 6.283185307179586476925286766559;
  const uint32_t quarter = n / 4, quad = (k % n) / quarter, r = (k % n) % quarter;
  float c0, s0;
  if (2 * r <= quarter) {
    c0 = (float)std::cos(two_pi * (double)r / (double)n);
    s0 = (float)std::sin(two_pi * (double)r / (double)n);
  } else {
    c0 = (float)std::sin(two_pi * (double)(quarter - r) / (double)n);
    s0 = (float)std::cos(two_pi * (double)(quarter - r) / (double)n);
  }
  switch (quad) {
    case 0: *c = c0; *s = s0; break;
    case 1: *c = 0.0f - s0; *s = c0; break;
    case 2: *c = 0.0f - c0; *s = 0.0f - s0; break;
    default: *c = s0; *s = 0.0f - c0; break;
  }
}

// Fills the tables; false if a lambda is not finite and positive.
static bool make_consts(const float* lambda, Consts* K) {
  for (uint32_t k = 0; k < 32; ++k) twiddle(64, k, &K->w64c[k], &K->w64s[k]);
  for (uint32_t k = 0; k < 64; ++k) twiddle(128, k, &K->w128c[k], &K->w128s[k]);
  const float s0 = (float)(1.0 / std::sqrt(128.0));
  for (int c = 0; c < kD; ++c) {
    const float l = lambda ? lambda[c] : 1.0f;
    if (!(l > 0.0f) || !std::isfinite(l)) return false;
    const volatile float r = 1.0f / l;  // binary32 quotient, then one rounded product
    K->m[c] = (c < 2 ? s0 : 0.0625f) * r;
    K->lam[c] = l;
  }
  return true;
}

// ---------------------------------------------------------------------------------------------
// Device.

// Complex FFT of 64 points held in registers (all indices compile-time), forward (w = e^-) or
// inverse (w = e^+), unnormalised.
template <bool INV>
__device__ __forceinline__ void fft64(float re[kN], float im[kN], const Consts& K) {
#pragma unroll
  for (int lg = 0; lg < 6; ++lg) {
    const int ns = 1 << lg;
    float br[kN], bi[kN];
#pragma unroll
    for (int j = 0; j < kN / 2; ++j) {
      const int k = (j % ns) * (kN / 2 / ns);
      const float ar = re[j + kN / 2], ai = im[j + kN / 2];
      float tr, ti;
      if (k == 0) {
        tr = ar;
        ti = ai;
      } else if (k == 16) {  // w = -i (forward) or +i (inverse)
        tr = INV ? -ai : ai;
        ti = INV ? ar : -ar;
      } else {
        const float c = K.w64c[k], s = INV ? K.w64s[k] : -K.w64s[k];
        tr = ar * c - ai * s;
        ti = ar * s + ai * c;
      }
      const int o = (j / ns) * 2 * ns + (j % ns);
      br[o] = re[j] + tr;
      bi[o] = im[j] + ti;
      br[o + ns] = re[j] - tr;
      bi[o + ns] = im[j] - ti;
    }
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      re[i] = br[i];
      im[i] = bi[i];
    }
  }
}

// The two quotients of the quantiser without the hardware division sequence (whose expansion
// keeps many values live), each equal to the correctly rounded quotient:
//   a / L for L = 7 and 127: q0 = a c with c = RN(1/L), then one correction with the exact remainder
//   fma(-q0, L, a) (Markstein's scheme); checked equal to RN(a / L) for every finite a >= 0;
//   1 / d for d a binary16 value: v_rcp_f32 (within one ulp) and one Newton step
//   fma(fma(-d, y0, 1), y0, y0); checked equal to RN(1 / d) for every positive finite binary16 d and
//   every start within one ulp.
template <int L>
__device__ __forceinline__ float div_l(float a) {
  constexpr float c = 1.0f / (float)L;
  const float q0 = a * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, (float)L, a), c, q0);
}

__device__ __forceinline__ float recip_f16_value(float d) {
  const float y0 = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, y0, 1.0f), y0, y0);
}

// Sign-bit masks of the 128 signs, 32 per word.
__device__ __forceinline__ void sign_words(uint64_t seed, uint32_t w[4]) {
  const hq::U4 p = hq::philox4x32_10(hq::U4{0u, 0u, 0u, 0u}, (uint32_t)seed, (uint32_t)(seed >> 32));
  w[0] = p.x;
  w[1] = p.y;
  w[2] = p.z;
  w[3] = p.w;
}

template <int BITS>
__global__ __launch_bounds__(kBlock) void srft_encode_kernel(const void* __restrict__ x, int f32_in, uint64_t nvec,
                                                             uint64_t seed, Consts K, uint8_t* __restrict__ codes,
                                                             uint16_t* __restrict__ scales) {
  const uint64_t v = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (v >= nvec) return;
  uint32_t sw[4];
  sign_words(seed, sw);
  float re[kN], im[kN];
  if (!f32_in) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + v * kD);
#pragma unroll
    for (int q4 = 0; q4 < 16; ++q4) {
      const uint4 u = src[q4];
      const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 4 * q4 + e;  // complex point n holds x_2n, x_2n+1: the two halves of the word
        const uint32_t bits = sw[n >> 4] >> ((2 * n) & 31);
        const uint32_t word = ws[e] ^ (((bits & 1u) << 15) | ((bits & 2u) << 30));
        re[n] = __uint_as_float(word << 16);
        im[n] = __uint_as_float(word & 0xFFFF0000u);
      }
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + v * kD);
#pragma unroll
    for (int q4 = 0; q4 < 32; ++q4) {
      const uint4 u = src[q4];
      const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int n = 2 * q4 + e;
        const uint32_t bits = sw[n >> 4] >> ((2 * n) & 31);
        re[n] = __uint_as_float(ws[2 * e] ^ ((bits & 1u) << 31));
        im[n] = __uint_as_float(ws[2 * e + 1] ^ ((bits & 2u) << 30));
      }
    }
  }
  fft64<false>(re, im, K);

  // Hermitian unpack into the packed coordinates, times the multipliers; E and G of k and 64 - k
  // are conjugates up to sign, so each pair forms them once.
  float val[kD];
  val[0] = (re[0] + im[0]) * K.m[0];
  val[1] = (re[0] - im[0]) * K.m[1];
#pragma unroll
  for (int k = 1; k <= kN / 2; ++k) {
    const int kk = kN - k;
    const float er = re[k] + re[kk], ei = im[k] - im[kk];
    const float gr = re[k] - re[kk], gi = im[k] + im[kk];
#pragma unroll
    for (int side = 0; side < (k == kN / 2 ? 1 : 2); ++side) {
      const int kx = side ? kk : k;
      // side 1: E_{64-k} = (er, -ei), G_{64-k} = (-gr, gi); -i G = (gi, -gr) resp. (gi, gr)
      const float a = gi, b = side ? gr : -gr;
      const float c = K.w128c[kx], e = -K.w128s[kx];
      const float pr = a * c - b * e, pi = a * e + b * c;
      val[2 * kx] = (er + pr) * K.m[2 * kx];
      val[2 * kx + 1] = ((side ? -ei : ei) + pi) * K.m[2 * kx + 1];
    }
  }

  // 16 groups of 8: binary16 scale of absmax / L, codes rint(v / Delta) clamped to [-L, L].
  constexpr int L = BITS == 4 ? 7 : 127;
  bool bad = false;
  uint32_t sc[kGroups / 2];
  uint32_t cw[BITS == 4 ? 16 : 32];
#pragma unroll
  for (int i = 0; i < (BITS == 4 ? 16 : 32); ++i) cw[i] = 0u;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      bad |= !__builtin_isfinite(val[8 * g + c]);
      a = fmaxf(a, fabsf(val[8 * g + c]));
    }
    const float t = fminf(div_l<L>(a), 65504.0f);
    const _Float16 h = (_Float16)t;
    const float delta = (float)h;
    const float inv = delta > 0.0f ? recip_f16_value(delta) : 0.0f;
    const uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, h);
    if (g & 1) sc[g >> 1] |= hb << 16;
    else sc[g >> 1] = hb;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int idx = 8 * g + c;
      const float r = __builtin_rintf(val[idx] * inv);
      const int32_t q = (int32_t)__builtin_amdgcn_fmed3f(r, (float)-L, (float)L);
      if (BITS == 4) cw[idx >> 3] |= ((uint32_t)q & 15u) << (4 * (idx & 7));
      else cw[idx >> 2] |= ((uint32_t)q & 255u) << (8 * (idx & 3));
    }
  }
  // a non-finite coordinate: zero codes, NaN scales
  const uint32_t keep = bad ? 0u : 0xFFFFFFFFu;
  uint4* cdst = reinterpret_cast<uint4*>(codes + v * (BITS == 4 ? kD / 2 : kD));
#pragma unroll
  for (int i = 0; i < (BITS == 4 ? 4 : 8); ++i)
    cdst[i] = make_uint4(cw[4 * i] & keep, cw[4 * i + 1] & keep, cw[4 * i + 2] & keep, cw[4 * i + 3] & keep);
  uint4* sdst = reinterpret_cast<uint4*>(scales + v * kGroups);
  const uint32_t nan2 = 0x7E007E00u;
  sdst[0] = bad ? make_uint4(nan2, nan2, nan2, nan2) : make_uint4(sc[0], sc[1], sc[2], sc[3]);
  sdst[1] = bad ? make_uint4(nan2, nan2, nan2, nan2) : make_uint4(sc[4], sc[5], sc[6], sc[7]);
}

template <int BITS, bool LAM>
__global__ __launch_bounds__(kBlock) void srft_decode_kernel(const uint8_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scales, uint64_t nvec,
                                                             uint64_t seed, Consts K, void* __restrict__ out,
                                                             int f32_out) {
  // every thread stays to the end (the bf16 store goes through LDS with workgroup barriers); a
  // thread past the last vector decodes the last vector again and stores nothing
  const uint64_t v = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  const uint64_t vl = v < nvec ? v : nvec - 1;
  constexpr int kWords = BITS == 4 ? 16 : 32;
  uint32_t cw[kWords];
  const uint4* csrc = reinterpret_cast<const uint4*>(codes + vl * (BITS == 4 ? kD / 2 : kD));
#pragma unroll
  for (int i = 0; i < kWords / 4; ++i) {
    const uint4 u = csrc[i];
    cw[4 * i] = u.x;
    cw[4 * i + 1] = u.y;
    cw[4 * i + 2] = u.z;
    cw[4 * i + 3] = u.w;
  }
  const uint4* ssrc = reinterpret_cast<const uint4*>(scales + vl * kGroups);
  const uint4 s0 = ssrc[0], s1 = ssrc[1];
  const uint32_t sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  // y_c = (q_c Delta_g) lambda_c, formed where the unpack needs it
  auto y = [&](const int c) __attribute__((always_inline)) -> float {
    const int32_t q = BITS == 4 ? __builtin_amdgcn_sbfe(cw[c >> 3], 4 * (c & 7), 4)
                                : __builtin_amdgcn_sbfe(cw[c >> 2], 8 * (c & 3), 8);
    const int g = c >> 3;
    const float delta = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc[g >> 1] >> (16 * (g & 1))));
    return LAM ? ((float)q * delta) * K.lam[c] : (float)q * delta;  // times 1 is exact
  };
  float re[kN], im[kN];
  const float r2 = 1.41421353816986083984375f;  // binary32 sqrt(2)
  {
    const float y0 = y(0), y1 = y(1);
    re[0] = (y0 + y1) * r2;
    im[0] = (y0 - y1) * r2;
  }
  // k and 64 - k read the same four coordinates: form both together so each is live briefly
#pragma unroll
  for (int k = 1; k <= kN / 2; ++k) {
    const float yk_r = y(2 * k), yk_i = y(2 * k + 1), ym_r = y(2 * (kN - k)), ym_i = y(2 * (kN - k) + 1);
#pragma unroll
    for (int side = 0; side < (k == kN / 2 ? 1 : 2); ++side) {
      const int kx = side ? kN - k : k;
      const float ar = side ? ym_r : yk_r, ai = side ? ym_i : yk_i;
      const float br = side ? yk_r : ym_r, bi = -(side ? yk_i : ym_i);
      const float sr = ar + br, si = ai + bi, dr = ar - br, di = ai - bi;
      const float c = K.w128c[kx], s = K.w128s[kx];
      const float pr = dr * c - di * s, pi = dr * s + di * c;
      re[kx] = sr - pi;
      im[kx] = si + pr;
    }
  }
  fft64<true>(re, im, K);
  uint32_t sw[4];
  sign_words(seed, sw);
  if (!f32_out) {
    uint32_t ow[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const uint32_t bits = sw[n >> 4] >> ((2 * n) & 31);
      const float x0 = __uint_as_float(__float_as_uint(re[n] * 0.0625f) ^ ((bits & 1u) << 31)) + 0.0f;
      const float x1 = __uint_as_float(__float_as_uint(im[n] * 0.0625f) ^ ((bits & 2u) << 30)) + 0.0f;
      // v_cvt_pk_bf16_f32: round to nearest even (a NaN stays a NaN)
      ow[n] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
    }
    // Through LDS, half a vector (128 bytes) per row and 64 rows per wavefront, so that each store
    // instruction writes 8 whole 128-byte lines; row r's 16-byte chunk c sits at slot c ^ (r & 7).
    __shared__ uint4 s_out[kBlock / 64][64 * 8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint64_t wbase = (uint64_t)blockIdx.x * kBlock + (uint64_t)wv * 64;
    uint4* dst = reinterpret_cast<uint4*>(out);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int w = 32 * h + 4 * c;
        s_out[wv][lane * 8 + (c ^ (lane & 7))] = make_uint4(ow[w], ow[w + 1], ow[w + 2], ow[w + 3]);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        const uint64_t vec = wbase + (uint64_t)r;
        if (vec < nvec) dst[vec * 16 + 8 * h + c] = s_out[wv][r * 8 + (c ^ (r & 7))];
      }
      __syncthreads();
    }
  } else {
    if (v >= nvec) return;
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + v * kD);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float xo[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int n = 2 * i + e;
        const uint32_t bits = sw[n >> 4] >> ((2 * n) & 31);
        xo[2 * e] = __uint_as_float(__float_as_uint(re[n] * 0.0625f) ^ ((bits & 1u) << 31)) + 0.0f;
        xo[2 * e + 1] = __uint_as_float(__float_as_uint(im[n] * 0.0625f) ^ ((bits & 2u) << 30)) + 0.0f;
      }
      dst[i] = make_float4(xo[0], xo[1], xo[2], xo[3]);
    }
  }
}

}  // namespace hq_srft

extern "C" {

int hq_srft_encode(const void* x, int32_t dtype, uint64_t n, uint64_t seed, const float* lambda, int32_t bits,
                   void* codes, void* scales, hq_stream_t stream) {
  if (n % hq_srft::kD || n > (1ull << 35) || (dtype != HQ_F32 && dtype != HQ_BF16) || (bits != 4 && bits != 8))
    return HQ_ERR_INVALID_ARG;
  if (n && (!x || !codes || !scales)) return HQ_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)codes | (uintptr_t)scales) & 15u) return HQ_ERR_INVALID_ARG;
  hq_srft::Consts K;
  if (!hq_srft::make_consts(lambda, &K)) return HQ_ERR_INVALID_ARG;
  const uint64_t nvec = n / hq_srft::kD;
  if (nvec == 0) return HQ_OK;
  const dim3 grid((uint32_t)((nvec + hq_srft::kBlock - 1) / hq_srft::kBlock));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int f32_in = dtype == HQ_F32;
  if (bits == 4)
    hipLaunchKernelGGL(hq_srft::srft_encode_kernel<4>, grid, dim3(hq_srft::kBlock), 0, st, x, f32_in, nvec, seed, K,
                       static_cast<uint8_t*>(codes), static_cast<uint16_t*>(scales));
  else
    hipLaunchKernelGGL(hq_srft::srft_encode_kernel<8>, grid, dim3(hq_srft::kBlock), 0, st, x, f32_in, nvec, seed, K,
                       static_cast<uint8_t*>(codes), static_cast<uint16_t*>(scales));
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_ERR_HIP;
}

int hq_srft_decode(const void* codes, const void* scales, uint64_t n, uint64_t seed, const float* lambda,
                   int32_t bits, void* out, int32_t out_dtype, hq_stream_t stream) {
  if (n % hq_srft::kD || n > (1ull << 35) || (out_dtype != HQ_F32 && out_dtype != HQ_BF16) || (bits != 4 && bits != 8))
    return HQ_ERR_INVALID_ARG;
  if (n && (!codes || !scales || !out)) return HQ_ERR_INVALID_ARG;
  if (((uintptr_t)out | (uintptr_t)codes | (uintptr_t)scales) & 15u) return HQ_ERR_INVALID_ARG;
  hq_srft::Consts K;
  if (!hq_srft::make_consts(lambda, &K)) return HQ_ERR_INVALID_ARG;
  const uint64_t nvec = n / hq_srft::kD;
  if (nvec == 0) return HQ_OK;
  const dim3 grid((uint32_t)((nvec + hq_srft::kBlock - 1) / hq_srft::kBlock));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int f32_out = out_dtype == HQ_F32;
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  const uint16_t* sp = static_cast<const uint16_t*>(scales);
  const dim3 block(hq_srft::kBlock);
  if (bits == 4 && lambda)
    hipLaunchKernelGGL((hq_srft::srft_decode_kernel<4, true>), grid, block, 0, st, c, sp, nvec, seed, K, out, f32_out);
  else if (bits == 4)
    hipLaunchKernelGGL((hq_srft::srft_decode_kernel<4, false>), grid, block, 0, st, c, sp, nvec, seed, K, out, f32_out);
  else if (lambda)
    hipLaunchKernelGGL((hq_srft::srft_decode_kernel<8, true>), grid, block, 0, st, c, sp, nvec, seed, K, out, f32_out);
  else
    hipLaunchKernelGGL((hq_srft::srft_decode_kernel<8, false>), grid, block, 0, st, c, sp, nvec, seed, K, out, f32_out);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_ERR_HIP;
}

}  // extern "C"
