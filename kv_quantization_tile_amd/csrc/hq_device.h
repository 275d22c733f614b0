// hq_device.h -- device building blocks of the gfx950 codec kernels.
//
// Thread layout used by every kernel: a workgroup has 256 lanes in 4 wavefronts of 64.  A tile of
// TL values (64, 128 or 256) lives in LPT = TL / 8 consecutive lanes, 8 values per lane: lane
// (wave w, lane l) owns octet o = l % LPT (coordinates 8o..8o+7) of tile TPW w + l / LPT of the
// workgroup's current group of 4 TPW tiles, TPW = 64 / LPT tiles per wavefront.  Three Hadamard
// stages run inside the lane and log2(LPT) across lanes (lane xor 1, 2, 4, ...).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kTile = 128;            // the default tile length; 64 and 256 are the others
constexpr int kChunkValues = 8192;    // a chunk holds kChunkValues / TL tiles
constexpr int kChunkTiles = 64;
constexpr int kBlock = 256;
constexpr int kHeaderBytes = 128;
constexpr uint32_t kMagic = 0x31305148u;  // 'H' 'Q' '0' '1'
constexpr uint32_t kVersion = 1;
constexpr uint32_t kStepBitsMin = (127u - 12u) << 23;
constexpr uint32_t kStepBitsMax = (127u + 12u) << 23;

enum { kLatZ = 0, kLatD4 = 1, kLatE8 = 2, kLatA2 = 3 };
// A2 quantises each pair in stretched coordinates (second coordinate / sqrt 3); its reconstruction
// factor on odd slots is the tile's times this binary32 sqrt(3) (nearest), and its multiplier the
// reciprocal of that.
constexpr uint32_t kA2R3Bits = 0x3FDDB3D7u;


// Three-input XOR in one v_bitop3 (truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): the counter-based generator behind the sign
// diagonal D and the dither.
struct U4 {
  uint32_t x, y, z, w;
};

// Rounds R0 .. R1-1 (the key already bumped R0 times).  Each round's two 32 x 32 -> 64-bit
// products are written as 64-bit multiplies of zero-extended words, which gfx950 computes with one
// v_mad_u64_u32 each instead of a mul_lo / mul_hi pair.  VXOR: each three-way XOR as one
// v_bitop3, for counters that differ in every lane (the dither); otherwise plain XORs, which the
// compiler keeps on the scalar unit where the counter is uniform (the sign diagonal).
template <int R0, int R1, bool VXOR = false>
__device__ __forceinline__ U4 philox_rounds(U4 c, uint32_t& k0, uint32_t& k1) {
#pragma unroll
  for (int r = R0; r < R1; ++r) {
    const uint64_t p0 = (uint64_t)c.x * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c.z * 0xCD9E8D57u;
    if (VXOR)
      c = U4{xor3((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1, xor3((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0};
    else
      c = U4{(uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}
__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
  return philox_rounds<0, 10>(c, k0, k1);
}
// Philox4x32 with 7 rounds when `seven` (the same for every lane), else 10: the 7-round function
// is the first 7 rounds of the 10-round one.  Per-lane counters (the dither's draws).
__device__ __forceinline__ U4 philox4x32_7_or_10(U4 c, uint32_t k0, uint32_t k1, bool seven) {
  c = philox_rounds<0, 7, true>(c, k0, k1);
  if (!seven) c = philox_rounds<7, 10, true>(c, k0, k1);
  return c;
}

// Sign word of octet o: bit i (0..7) set means D_{8o+i} = -1.  D comes from Philox calls with key
// = seed and counters (c, 0, 0, 0): octets 0..15 use call 0, octets 16..31 (tiles of 256) call 1;
// the sign bits are the output words, least significant bit first.
__device__ __forceinline__ uint32_t octet_sign_bits(uint64_t seed, int o) {
  const U4 w = philox4x32_10(U4{(uint32_t)(o >> 4), 0u, 0u, 0u}, (uint32_t)seed, (uint32_t)(seed >> 32));
  const int q = (o >> 2) & 3;
  const uint32_t word = q == 0 ? w.x : q == 1 ? w.y : q == 2 ? w.z : w.w;
  return (word >> ((o & 3) * 8)) & 0xFFu;
}

// ---------------------------------------------------------------------------------------------
// Unnormalised Walsh-Hadamard transform of the TL values held by LPT lanes (8 per lane), stage j
// pairing index i with i + 2^j in the order j = 0..log2(TL)-1; the low element becomes a + b, the
// high a - b.  Stages 0-2 are in registers, the others exchange with lane xor 1, 2, 4, ...
__device__ __forceinline__ void fwht_lane(float a[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float lo = a[i], hi = a[i + h];
      a[i] = lo + hi;
      a[i + h] = lo - hi;
    }
  }
}

// Partner value for the cross-lane stages: ds_swizzle in bit-mask mode (and 0x1F, xor m) inside
// 32 lanes.  It runs in the LDS pipe, so a stage costs one VALU operation per value (the fused
// multiply-add below).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}

// The cross-lane stages.  Each lane computes own + s * partner with s = +1 on the low lane and -1
// on the high lane, as one fused multiply-add: the product by +-1 is exact, so the result is the
// sum or difference rounded once, exactly as the plain butterfly.  The high lane then holds the
// negated value; after the stages lane l holds sigma(l) * y with
// sigma(l) = (-1)^popcount(l mod LPT) (lane_sign_bit), which callers fold into the quantiser's
// multiplier (encode) or into the sign diagonal (decode).
template <int M>
__device__ __forceinline__ void fwht_stage(float a[8], int lane16) {
  const float sgn = (lane16 & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(lane_xor<M>(a[i]), sgn, a[i]);
}

template <int LPT = 16>
__device__ __forceinline__ void fwht_cross(float a[8], int o) {
  fwht_stage<1>(a, o);
  fwht_stage<2>(a, o);
  fwht_stage<4>(a, o);
  if (LPT >= 16) fwht_stage<8>(a, o);
  if (LPT >= 32) fwht_stage<16>(a, o);
}

// The same stages with the per-lane factors of the stages (+-1.0 for lane bits 1, 2, 4, 8, 16)
// given by the caller, which computes them once per kernel instead of once per call.
template <int M>
__device__ __forceinline__ void fwht_stage_s(float a[8], float sgn) {
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(lane_xor<M>(a[i]), sgn, a[i]);
}
template <int LPT = 16>
__device__ __forceinline__ void fwht_cross_s(float a[8], const float* sg) {
  fwht_stage_s<1>(a, sg[0]);
  fwht_stage_s<2>(a, sg[1]);
  fwht_stage_s<4>(a, sg[2]);
  if (LPT >= 16) fwht_stage_s<8>(a, sg[3]);
  if (LPT >= 32) fwht_stage_s<16>(a, sg[4]);
}
// Per-lane factors for fwht_cross_s.  The asm keeps them in registers: left visible, the compiler
// recomputes them at every use (three instructions each) to save the registers.
template <int LPT = 16>
__device__ __forceinline__ void fwht_lane_signs(int o, float* sg) {
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    sg[j] = (o & (1 << j)) ? -1.0f : 1.0f;
    if ((1 << j) < LPT) __asm__ volatile("" : "+v"(sg[j]));
  }
}

template <int LPT = 16>
__device__ __forceinline__ uint32_t lane_sign_bit(int o) { return (uint32_t)__popc(o & (LPT - 1)) & 1u; }

// Sum of squares of the tile as a balanced pairwise tree in index order: squares, pairs inside
// the lane, then lane xor 1, 2, 4, ... (each add is commutative, so both lanes get equal sums).
template <int LPT = 16>
__device__ __forceinline__ float tile_sumsq(const float a[8]) {
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = a[i] * a[i];
  float t = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  t = t + lane_xor<1>(t);
  t = t + lane_xor<2>(t);
  t = t + lane_xor<4>(t);
  if (LPT >= 16) t = t + lane_xor<8>(t);
  if (LPT >= 32) t = t + lane_xor<16>(t);
  return t;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Tile scale s = bfloat16 nearest to sqrt(S / TL), ties to even, decided exactly.  A hardware
// square root r (within one binary32 ulp) gives the candidate c = bf16(r); the true result can only
// be c's neighbour on r's side of c, across the rounding midpoint m between them, and that midpoint
// has 9 significant bits, so S against TL m^2 is an exact binary32 comparison.  S is first brought
// into [2^-60, 2^60] by an exact power-of-two factor so that no square under- or overflows.
template <int TL = 128>
__device__ __forceinline__ uint32_t tile_scale_bits(float S) {
  if (!(S > 0.0f)) return 0u;
  float Ss = S;
  int adj = 0;
  if (S < 0x1p-60f) {
    Ss = S * 0x1p100f;
    adj = 50;
  } else if (S > 0x1p60f) {
    Ss = S * 0x1p-100f;
    adj = -50;
  }
  const float r = __builtin_amdgcn_sqrtf(Ss * (1.0f / (float)TL));
  uint32_t c = f32_to_bf16_rne(r);
  const float cv = bf16_bits_to_f32(c);
  const bool up = r >= cv;
  const uint32_t nb = up ? c + 1u : c - 1u;
  const float m = (cv + bf16_bits_to_f32(nb)) * 0.5f;
  const float tm = (float)TL * (m * m);
  const bool cross = up ? (Ss > tm) : (Ss < tm);
  if (cross || (Ss == tm && (c & 1u))) c = nb;
  return (uint32_t)((int32_t)c - adj * 128);
}


__device__ __forceinline__ uint32_t zigzag(int32_t a) { return ((uint32_t)a << 1) ^ (uint32_t)(a >> 31); }
__device__ __forceinline__ int32_t unzigzag(uint32_t u) { return (int32_t)(u >> 1) ^ -(int32_t)(u & 1u); }

// ---------------------------------------------------------------------------------------------
// Nearest lattice points (Conway-Sloane rules).  Ties: rint is round-half-even; the coordinate
// moved by a parity fix is the largest |v - rint v| (lowest index among equals), moved toward v
// (up when v is an integer).  E8 codes are z = 2 c in 2*E8.
__device__ __forceinline__ void d4_nearest(const float* v, int32_t* x) {
  float a[4];
  uint32_t neg = 0;
  int32_t par = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float r = rintf(v[i]);
    const float e = v[i] - r;
    a[i] = fabsf(e);
    neg |= (__float_as_uint(e) >> 31) << i;
    x[i] = (int32_t)r;
    par += x[i];
  }
  int k = 0;
  float amax = a[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (a[i] > amax) {
      amax = a[i];
      k = i;
    }
  if (par & 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i == k) x[i] += ((neg >> i) & 1u) ? -1 : 1;
  }
}

// E8 = D8 u (D8 + 1/2).  With r = rint v, e = v - r, a = |e|, s = sign of e (+ for e >= 0):
// candidate A (D8) = r, + s at argmax a if sum r is odd; candidate B (D8 + 1/2) = r + s/2, with the
// coordinate of argmin a turned the other way if sum(B - 1/2) is odd.  |v-A|^2 - |v-B|^2 equals
// sum a - 2 + pA (1 - 2 a_max) - pB 2 a_min, so A is kept iff
// ((a0+a1)+(a2+a3))+((a4+a5)+(a6+a7)) [+ (1 - 2 a_max)]  <=  2 [+ 2 a_min]   (binary32, this order).
__device__ __forceinline__ void e8_nearest(const float* v, int32_t* z) {
  float a[8];
  int32_t r[8];
  uint32_t neg = 0;
  int32_t par = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float ri = rintf(v[i]);
    const float e = v[i] - ri;
    a[i] = fabsf(e);
    neg |= (__float_as_uint(e) >> 31) << i;
    r[i] = (int32_t)ri;
    par += r[i];
  }
  const int pa = par & 1;
  const int pb = (pa + __popc(neg)) & 1;
  int ka = 0, kb = 0;
  float amax = a[0], amin = a[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    if (a[i] > amax) {
      amax = a[i];
      ka = i;
    }
    if (a[i] < amin) {
      amin = a[i];
      kb = i;
    }
  }
  const float d = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  const float lhs = pa ? d + (1.0f - 2.0f * amax) : d;
  const float rhs = pb ? 2.0f + 2.0f * amin : 2.0f;
  const bool keep_a = lhs <= rhs;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int32_t s = ((neg >> i) & 1u) ? -1 : 1;
    const int32_t za = 2 * r[i] + ((pa && i == ka) ? 2 * s : 0);
    const int32_t zb = 2 * r[i] + ((pb && i == kb) ? -s : s);
    z[i] = keep_a ? za : zb;
  }
}

// E8 nearest point and bit-stripping in one pass, producing the symbols and the coset bit
// directly (same rule and ties as e8_nearest followed by strip_octet).  With r = rint v, e = v - r,
// sigma_i = [e_i < 0]: the stripped coordinates are u = r for the D8 candidate and
// u = r - sigma = floor v for the D8 + 1/2 candidate; the parity fix moves the first coordinate
// whose |e| equals the maximum (D8) or the minimum (D8 + 1/2) of |e| by one step: +-1 with the sign
// of e for D8, against it for D8 + 1/2.  The stripped coordinates stay in binary32 (integers below
// 2^22, so every step is exact), and zigzag is |2u + 1/2| truncated: 2u for u >= 0, -2u - 1 below.
// 1 - 2 a_max and 2 + 2 a_min are formed by a fused multiply-add: the product by 2 is exact, so
// the single rounding equals that of the separate multiply and add.
template <bool MASK_FIX = false>
__device__ __forceinline__ void e8_symbols(const float* v, uint32_t* sym, uint32_t* coset) {
  float e[8], rf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    rf[i] = rintf(v[i]);
    e[i] = v[i] - rf[i];
  }
  // parity of sum r: the sum of eight integers below 2^18 is exact in binary32
  const float rsum = ((rf[0] + rf[1]) + (rf[2] + rf[3])) + ((rf[4] + rf[5]) + (rf[6] + rf[7]));
  // parity of the number of negative e: sign bit of the XOR of the eight patterns
  const uint32_t xe =
      xor3(xor3(__float_as_uint(e[0]), __float_as_uint(e[1]), __float_as_uint(e[2])),
           xor3(__float_as_uint(e[3]), __float_as_uint(e[4]), __float_as_uint(e[5])),
           __float_as_uint(e[6]) ^ __float_as_uint(e[7]));
  const uint32_t pa = (uint32_t)(int32_t)rsum & 1u, pb = pa ^ (xe >> 31);
  const float amax = fmaxf(fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3]))),
                           fmaxf(fmaxf(fabsf(e[4]), fabsf(e[5])), fmaxf(fabsf(e[6]), fabsf(e[7]))));
  const float amin = fminf(fminf(fminf(fabsf(e[0]), fabsf(e[1])), fminf(fabsf(e[2]), fabsf(e[3]))),
                           fminf(fminf(fabsf(e[4]), fabsf(e[5])), fminf(fabsf(e[6]), fabsf(e[7]))));
  const float d = ((fabsf(e[0]) + fabsf(e[1])) + (fabsf(e[2]) + fabsf(e[3]))) +
                  ((fabsf(e[4]) + fabsf(e[5])) + (fabsf(e[6]) + fabsf(e[7])));
  const float lhs = d + (pa ? __builtin_fmaf(-2.0f, amax, 1.0f) : 0.0f);
  const float rhs = pb ? __builtin_fmaf(2.0f, amin, 2.0f) : 2.0f;
  // rhs - lhs is exact in sign (a difference of distinct finite floats is never zero), so its sign
  // bit is [lhs > rhs]: kb is all ones when the D8 + 1/2 candidate is kept
  const uint32_t kb = (uint32_t)((int32_t)__float_as_uint(rhs - lhs) >> 31);
  const bool keep_a = kb == 0u;
  const float t = keep_a ? amax : amin;
  bool found = keep_a ? (pa == 0u) : (pb == 0u);  // no fix needed: nothing to find
  float u[8];
  if (MASK_FIX) {
    // u_i = rf_i + D_i.  D8 candidate: D = +-1 (toward e) on the fixed coordinate, else 0.  D8 + 1/2:
    // u = floor(v) = rf - [e < 0], moved by 1 against e on the fixed coordinate, so D = -([e < 0]
    // xor hit).  The conditions stay lane masks (scalar work); per coordinate only the compares and
    // two selects of c = 2 D + 1/2 are vector work, and 2 u + 1/2 = fma(2, rf, c) exactly.  Fewer
    // vector instructions and registers, more scalar ones: the choice for kernels whose scalar
    // unit has room.
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool hit = !found && (fabsf(e[i]) == t);
      found = found || hit;
      const bool neg = e[i] < 0.0f;  // e is never -0: it is v - rint(v) in round to nearest
      const bool up = keep_a && hit && !neg;                   // D = +1
      const bool down = keep_a ? (hit && neg) : (neg != hit);  // D = -1
      c[i] = down ? -1.5f : (up ? 2.5f : 0.5f);
    }
    u[7] = rf[7] + (c[7] - 0.5f) * 0.5f;
#pragma unroll
    for (int i = 0; i < 7; ++i) sym[i] = (uint32_t)fabsf(__builtin_fmaf(2.0f, rf[i], c[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float base = keep_a ? rf[i] : floorf(v[i]);
      const bool hit = !found && (fabsf(e[i]) == t);
      found = found || hit;
      // +-1 with the sign of e (D8) or against it (D8 + 1/2): sign bit of e ^ kb on 1.0
      const float step1 = __uint_as_float(((__float_as_uint(e[i]) ^ kb) & 0x80000000u) | 0x3F800000u);
      u[i] = base + (hit ? step1 : 0.0f);
    }
#pragma unroll
    for (int i = 0; i < 7; ++i) sym[i] = (uint32_t)fabsf(__builtin_fmaf(2.0f, u[i], 0.5f));
  }
  const uint32_t x = xor3(xor3(sym[0], sym[1], sym[2]), xor3(sym[3], sym[4], sym[5]), sym[6]);
  // parity of u_0 + .. + u_6: u and zz(u) satisfy [u odd] = bit 1 ^ bit 0 of zz(u)
  const int32_t par = (int32_t)(((x >> 1) ^ x) & 1u);
  sym[7] = zigzag(((int32_t)u[7] - par) >> 1);
  *coset = kb & 1u;
}

// A2 (hexagonal, minimal distance 1) in stretched coordinates w = (v0, v1 / sqrt 3), where it is
// Z^2 u (Z + 1/2)^2 under the squared distance dw0^2 + 3 dw1^2.  With r = rint w and a = |w - r|,
// |w - A|^2 - |w - B|^2 = a0 + 3 a1 - 1 for the rounded point A and the nearest point B of the
// shifted coset, so A is kept iff fma(3, a1, a0) <= 1 (one rounding).  Codes z = 2c: B moves each
// coordinate half a step toward w (up for an exact integer).
__device__ __forceinline__ void a2_nearest(const float* w, int32_t* z) {
  const float r0 = rintf(w[0]), r1 = rintf(w[1]);
  const float e0 = w[0] - r0, e1 = w[1] - r1;
  const bool keep_a = __builtin_fmaf(3.0f, fabsf(e1), fabsf(e0)) <= 1.0f;
  const int32_t s0 = (__float_as_uint(e0) >> 31) ? -1 : 1, s1 = (__float_as_uint(e1) >> 31) ? -1 : 1;
  z[0] = 2 * (int32_t)r0 + (keep_a ? 0 : s0);
  z[1] = 2 * (int32_t)r1 + (keep_a ? 0 : s1);
}

template <int LAT>
__device__ __forceinline__ void nearest_octet(const float* v, int32_t* code) {
  if (LAT == kLatE8) {
    e8_nearest(v, code);
  } else if (LAT == kLatA2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a2_nearest(v + 2 * j, code + 2 * j);
  } else if (LAT == kLatD4) {
    d4_nearest(v, code);
    d4_nearest(v + 4, code + 4);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = (int32_t)rintf(v[i]);
  }
}

template <int LAT>
__device__ __forceinline__ float code_coord(int32_t c) {
  return (LAT == kLatE8 || LAT == kLatA2) ? (float)c * 0.5f : (float)c;
}

// U = b - Q(b) for E8, straight from the nearest-point decision (the rule and arithmetic of
// e8_nearest, evaluated as in e8_symbols): with r = rint b and e = b - r, the chosen point differs
// from r by D, and U = e - D.  D8 candidate: D = 0, or +-1 with the sign of e on the coordinate the
// parity fix moves.  D8 + 1/2 candidate: D = +-1/2 with the sign of e, against it on the coordinate
// that candidate's fix turns.  Every step is exact (e and U lie on the draw's grid).  Requires b
// in [0, 2)^8, which every dither draw is.
__device__ __forceinline__ void e8_dither_u(const float* b, float* u) {
  float e[8], rf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    rf[i] = rintf(b[i]);
    e[i] = b[i] - rf[i];
  }
  // b lies in [0, 2), so each rint is 0.0, 1.0 or 2.0 and only 1.0 has bit 23 (the exponent's low
  // bit) set: the parity of the sum is bit 23 of the XOR of the eight patterns
  const uint32_t xr =
      xor3(xor3(__float_as_uint(rf[0]), __float_as_uint(rf[1]), __float_as_uint(rf[2])),
           xor3(__float_as_uint(rf[3]), __float_as_uint(rf[4]), __float_as_uint(rf[5])),
           __float_as_uint(rf[6]) ^ __float_as_uint(rf[7]));
  const uint32_t xe =
      xor3(xor3(__float_as_uint(e[0]), __float_as_uint(e[1]), __float_as_uint(e[2])),
           xor3(__float_as_uint(e[3]), __float_as_uint(e[4]), __float_as_uint(e[5])),
           __float_as_uint(e[6]) ^ __float_as_uint(e[7]));
  const uint32_t pa = (xr >> 23) & 1u, pb = pa ^ (xe >> 31);
  const float amax = fmaxf(fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3]))),
                           fmaxf(fmaxf(fabsf(e[4]), fabsf(e[5])), fmaxf(fabsf(e[6]), fabsf(e[7]))));
  const float amin = fminf(fminf(fminf(fabsf(e[0]), fabsf(e[1])), fminf(fabsf(e[2]), fabsf(e[3]))),
                           fminf(fminf(fabsf(e[4]), fabsf(e[5])), fminf(fabsf(e[6]), fabsf(e[7]))));
  const float d = ((fabsf(e[0]) + fabsf(e[1])) + (fabsf(e[2]) + fabsf(e[3]))) +
                  ((fabsf(e[4]) + fabsf(e[5])) + (fabsf(e[6]) + fabsf(e[7])));
  const float lhs = d + (pa ? __builtin_fmaf(-2.0f, amax, 1.0f) : 0.0f);
  const float rhs = pb ? __builtin_fmaf(2.0f, amin, 2.0f) : 2.0f;
  const bool keep_a = lhs <= rhs;
  const float t = keep_a ? amax : amin;
  bool found = keep_a ? (pa == 0u) : (pb == 0u);  // no fix needed: nothing to find
  // D relative to the sign of e: on the moved coordinate (hit) and elsewhere
  const float dh = keep_a ? 1.0f : -0.5f, dn = keep_a ? 0.0f : 0.5f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool hit = !found && (fabsf(e[i]) == t);
    found = found || hit;
    const float dm = hit ? dh : dn;
    const float D = __uint_as_float(__float_as_uint(dm) ^ (__float_as_uint(e[i]) & 0x80000000u));
    u[i] = e[i] - D;
  }
}

// Dither flags (the stream header's flags byte): bit 0 dither on; bit 1 the dither's Philox calls
// take 7 rounds instead of 10; bit 2 a 24-bit draw instead of 16-bit halves.
constexpr uint32_t kDitherOn = 1u, kDitherPhilox7 = 2u, kDither24 = 4u;

// Subtractive dither of octet o of tile t: a Philox call with counter (o, t lo, t hi, 1); its eight
// 16-bit halves h (low half first) give b = h / 32768 in [0, 2).  With the 24-bit draw a second
// call (counter word 3 = 2) adds four more words and b_i = (w_i >> 8) / 2^23.  U = b - Q(b) is
// uniform on the Voronoi cell to the draw's resolution.  Exact in binary32.  df is the same in
// every lane, so both branches are uniform.
template <int LAT>
__device__ __forceinline__ void dither_octet(uint64_t seed, uint64_t t, int o, uint32_t df, float* u) {
  const bool seven = (df & kDitherPhilox7) != 0u;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const U4 w = philox4x32_7_or_10(U4{(uint32_t)o, (uint32_t)t, (uint32_t)(t >> 32), 1u}, k0, k1, seven);
  float b[8];
  if (df & kDither24) {
    const U4 v = philox4x32_7_or_10(U4{(uint32_t)o, (uint32_t)t, (uint32_t)(t >> 32), 2u}, k0, k1, seven);
    const uint32_t ww[8] = {w.x, w.y, w.z, w.w, v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (float)(ww[i] >> 8) * (1.0f / 8388608.0f);
  } else {
    // h / 2^15 for a 16-bit half h: the binary32 with exponent 2^8 and h in the low mantissa bits is
    // 256 + h 2^-15, so one subtraction of 256 leaves h 2^-15 exactly
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (i & 1) ? __builtin_amdgcn_alignbit(0x4380u, ww[i >> 1], 16u)
                                    : ((ww[i >> 1] & 0xFFFFu) | 0x43800000u);
      b[i] = __uint_as_float(bits) - 256.0f;
    }
  }
  if (LAT == kLatE8) {
    e8_dither_u(b, u);
    return;
  }
  int32_t q[8];
  nearest_octet<LAT>(b, q);
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = b[i] - code_coord<LAT>(q[i]);
}

// ---------------------------------------------------------------------------------------------
// Bit-stripping and zigzag (see the format description in hq.h).

template <int LAT>
__device__ __forceinline__ bool slot_halved(int s) {
  return LAT == kLatE8 ? (s == 7) : LAT == kLatD4 ? ((s & 3) == 3) : LAT == kLatA2 ? ((s & 1) == 1) : false;
}
template <int LAT>
__device__ __forceinline__ int slot_width(int s, int k) {
  return slot_halved<LAT>(s) ? (k > 0 ? k - 1 : 0) : k;
}
template <int LAT>
__device__ __forceinline__ int octet_rem_bits(int k) {
  const int kh = k > 0 ? k - 1 : 0;
  return LAT == kLatE8 ? 7 * k + kh : LAT == kLatD4 ? 6 * k + 2 * kh : LAT == kLatA2 ? 4 * k + 4 * kh : 8 * k;
}
// Tile record header: 16 scale bits, then the raw coset bits (E8: one per octet, bit o; A2: one
// per pair, bit 4 o + j for pair j of octet o); then the remainders of the TL / 8 octets.
template <int LAT, int TL = kTile>
__device__ __forceinline__ int tile_hdr_bits() {
  return 16 + (LAT == kLatE8 ? TL / 8 : LAT == kLatA2 ? TL / 2 : 0);
}
template <int LAT, int TL = kTile>
__device__ __forceinline__ uint32_t tile_fixed_bits(int k) {
  return (uint32_t)(tile_hdr_bits<LAT, TL>() + (TL / 8) * octet_rem_bits<LAT>(k));
}

template <int LAT>
__device__ __forceinline__ void strip_octet(const int32_t* code, uint32_t* sym, uint32_t* coset) {
  *coset = 0;
  if (LAT == kLatE8) {
    const int32_t p = code[0] & 1;
    int32_t u[8], r = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = (code[i] - p) >> 1;
#pragma unroll
    for (int i = 0; i < 7; ++i) r += u[i];
#pragma unroll
    for (int i = 0; i < 7; ++i) sym[i] = zigzag(u[i]);
    sym[7] = zigzag((u[7] - (r & 1)) >> 1);
    *coset = (uint32_t)p;
  } else if (LAT == kLatA2) {
    uint32_t cs = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t p = code[2 * j] & 1;
      sym[2 * j] = zigzag((code[2 * j] - p) >> 1);
      sym[2 * j + 1] = zigzag((code[2 * j + 1] - p) >> 1);
      cs |= (uint32_t)p << j;
    }
    *coset = cs;
  } else if (LAT == kLatD4) {
#pragma unroll
    for (int b = 0; b < 8; b += 4) {
      const int32_t r = (code[b] + code[b + 1] + code[b + 2]) & 1;
      sym[b] = zigzag(code[b]);
      sym[b + 1] = zigzag(code[b + 1]);
      sym[b + 2] = zigzag(code[b + 2]);
      sym[b + 3] = zigzag((code[b + 3] - r) >> 1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) sym[i] = zigzag(code[i]);
  }
}

template <int LAT>
__device__ __forceinline__ void unstrip_octet(const uint32_t* sym, uint32_t coset, int32_t* code) {
  if (LAT == kLatE8) {
    int32_t u[8], r = 0;
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      u[i] = unzigzag(sym[i]);
      r += u[i];
    }
    u[7] = 2 * unzigzag(sym[7]) + (r & 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = 2 * u[i] + (int32_t)coset;
  } else if (LAT == kLatA2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = 2 * unzigzag(sym[i]) + (int32_t)((coset >> (i / 2)) & 1u);
  } else if (LAT == kLatD4) {
#pragma unroll
    for (int b = 0; b < 8; b += 4) {
      code[b] = unzigzag(sym[b]);
      code[b + 1] = unzigzag(sym[b + 1]);
      code[b + 2] = unzigzag(sym[b + 2]);
      const int32_t r = (code[b] + code[b + 1] + code[b + 2]) & 1;
      code[b + 3] = 2 * unzigzag(sym[b + 3]) + r;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = unzigzag(sym[i]);
  }
}

// ---------------------------------------------------------------------------------------------
// Loads of one lane's 8 values of tile t with the sign diagonal applied (DT 0: fp32, 1: bf16 bits).
// smask[i] is 0x80000000 where D = -1: the sign flip is an xor (fp32) or an add into bit 31 of the
// widened bf16 value, both exact.
template <int DT, int TL = kTile>
__device__ __forceinline__ void load_octet_signed(const void* x, uint64_t t, int o, const uint32_t* smask, float* v) {
  if (DT == 1) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + t * TL + 8 * o);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float((ws[i] << 16) + smask[2 * i]);
      v[2 * i + 1] = __uint_as_float((ws[i] & 0xFFFF0000u) ^ smask[2 * i + 1]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + t * TL + 8 * o);
    const float4 a = p[0], b = p[1];
    const float vv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(__float_as_uint(vv[i]) ^ smask[i]);
  }
}

// Buffer resource over bytes [base, base + bytes) of global memory (raw, no stride): loads past
// the end return zeros, so a ragged last chunk needs no per-tile branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// load_octet_signed through a buffer resource: the lane's octet at byte offset `off` (zeros past
// the resource's end).
template <int DT>
__device__ __forceinline__ void load_octet_signed_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint32_t* smask,
                                                      float* v) {
  if (DT == 1) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float((w[i] << 16) + smask[2 * i]);
      v[2 * i + 1] = __uint_as_float((w[i] & 0xFFFF0000u) ^ smask[2 * i + 1]);
    }
  } else {
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i] ^ smask[i]);
      v[4 + i] = __uint_as_float(b[i] ^ smask[4 + i]);
    }
  }
}

// Broadcast inside the LPT-lane group of a tile: every lane receives the value of lane SRC of its
// own group (ds_swizzle bit-mask mode inside 32 lanes: keep the lane bits above the group, set
// the low bits to SRC).
template <int SRC, int LPT = 16>
__device__ __forceinline__ uint32_t group_bcast(uint32_t v) {
  static_assert(SRC < LPT, "source lane inside the group");
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (0x1F & ~(LPT - 1)) | (SRC << 5));
}

// Loads of one lane's 8 values of tile t (DT 0: fp32, 1: bf16 bits).
template <int DT, int TL = kTile>
__device__ __forceinline__ void load_octet(const void* x, uint64_t t, int o, float* v) {
  if (DT == 1) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + t * TL + 8 * o);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(ws[i] << 16);
      v[2 * i + 1] = __uint_as_float(ws[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + t * TL + 8 * o);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// ---------------------------------------------------------------------------------------------
// Workgroup exclusive prefix sum over 256 lanes (wave scans + LDS of wave totals).
// `scratch` holds at least 4 words.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t s = scratch[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP: four row shifts give the
// prefix inside each row of 16 lanes, then row_bcast:15 adds row 0's (row 2's) total to row 1
// (row 3) and row_bcast:31 adds the total of rows 0-1 to rows 2-3.  Lanes whose source is out of
// range or whose row is masked receive 0 (old = 0, bound_ctrl), so the add leaves them unchanged.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
  return (uint32_t)v;
}

__device__ __forceinline__ uint64_t atomic_load_acq(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_rel(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace hq
