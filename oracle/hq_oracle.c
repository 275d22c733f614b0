/*
 * hq_oracle.c -- plain, slow CPU oracle for the per-tile RHT + lattice + bit-strip + Rice codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  The GPU product path never links, loads or calls it, and the two share no
 * code: this file includes no header of the product and the product includes nothing from here.
 *
 * What it computes follows the HyperQuant technical summaries (gist.science/ko/paper/2606.23406 and
 * gist.science/ja/paper/2606.23406), section "Methodology: the HyperQuant pipeline":
 *   component 1 (per-tile randomized Hadamard transform  RHT_n(x) = H_n D x, tiles of 128, or of
 *   64 or 256: the summary gives 128 as an example size),
 *   component 2 (nearest-point quantisation onto E8 / D4 / A2 / Z with an integer embedding and a
 *   scale),
 *   component 3 (bit-stripping of lattice-fixed bits, then Rice coding; rate within ~0.01 bps),
 *   component 4 (KV bias correction: per-layer +-1 rotation, subtractive dither U ~ Unif(V(L))).
 * Where the pages leave a step open (butterfly order, scale rounding, tie breaks, bit layout,
 * rate-control search, random-number layout) this file takes one plain reading and states it at
 * the function that implements it.  Every floating-point step that decides an integer is done in
 * IEEE binary32 in a fixed order (build with -ffp-contract=off, no fast-math), because the GPU
 * kernel takes those decisions in binary32 too.
 *
 * Parity pins: every function here is checked in tests/ against something other than itself
 * (dense Hadamard matrix, brute-force lattice search, closed forms, the rocRAND Philox source,
 * statistical invariants).  The random-number generator's stream layout and the bitstream layout
 * are this codec's own format choices; their round trips are pinned, their exact bit positions are
 * a definition, not a result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TILE 128            /* the default tile length; 64 and 256 are the other lengths */
#define TILE_MAX 256
#define CHUNK_VALUES 8192   /* a chunk holds 8192 / tile tiles: 128, 64 or 32 */
#define HEADER_BYTES 128
#define HAAR_N 128          /* dimension of the per-layer rotation */
#define MAGIC 0x31305148u /* bytes 'H' 'Q' '0' '1' */
#define VERSION 1

enum { LAT_Z = 0, LAT_D4 = 1, LAT_E8 = 2, LAT_A2 = 3 };

/* A2 works in coordinates where the second coordinate of each pair is divided by sqrt 3 (see
 * a2_nearest): R3 is binary32 sqrt(3) rounded to nearest, 0x3FDDB3D7. */
#define A2_R3_BITS 0x3FDDB3D7u
enum {
  OK = 0,
  ERR_INVALID_ARG = -1,
  ERR_UNSUPPORTED = -2,
  ERR_NONFINITE = -3,
  ERR_CAPACITY = -4,
  ERR_CORRUPT = -5,
  ERR_RATE = -6
};

/* Step range accepted by the codec: 2^-12 .. 2^12 (as binary32 bit patterns). */
#define STEP_BITS_MIN ((uint32_t)(127 - 12) << 23)
#define STEP_BITS_MAX ((uint32_t)(127 + 12) << 23)
#define RC_SAMPLE_TILES 8192   /* pass B (and a fixed step's k choice) */
#define RC_SAMPLE_TILES_A 2048 /* pass A */
#define RC_CANDIDATES 8        /* pass A; pass B evaluates RC_CANDIDATES_B */
#define RC_CANDIDATES_B 4
#define RC_KWIN 4

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* ------------------------------------------------------------------------------------------ */
/* Philox4x32-R, as defined by Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy */
/* as 1, 2, 3" (SC'11): R rounds (10 is the generator's recommended count, 7 the fewest its      */
/* authors report as passing their statistical batteries); each round multiplies counter words  */
/* 0 and 2 by the two round multipliers, xors the high halves with the other counter words and  */
/* the key, and the key is bumped by the two Weyl constants between rounds.  hqo_philox4x32_span */
/* applies rounds r0 .. r1-1 only (the key first bumped r0 times), so a count of R rounds is the */
/* first R rounds of the same function.                                                         */
/* ------------------------------------------------------------------------------------------ */
void hqo_philox4x32_span(const uint32_t ctr_in[4], const uint32_t key_in[2], int r0, int r1, uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < r0; ++round) {
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  for (int round = r0; round < r1; ++round) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}
void hqo_philox4x32_r(const uint32_t ctr_in[4], const uint32_t key_in[2], int rounds, uint32_t out[4]) {
  hqo_philox4x32_span(ctr_in, key_in, 0, rounds, out);
}
void hqo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  hqo_philox4x32_r(ctr_in, key_in, 10, out);
}

/* Sign diagonal D of the RHT (HyperQuant summary, Methodology component 1: "D is a random sign
 * diagonal").  Reading: one D per call, shared by every tile, drawn from Philox calls with
 * key = (seed low word, seed high word) and counters (c,0,0,0), c = 0, 1, ...: the output words of
 * call c are words 4c..4c+3; D_i = -1 iff bit (i mod 32) of word floor(i/32) is set (one call
 * for tiles of 64 or 128, two for 256; shorter tiles use a prefix).  The KV path's per-layer +-1
 * rotation (component 4) is the same kind of diagonal, so it is folded into D by giving each
 * (layer, K|V) call its own seed. */
void hqo_signs_n(uint64_t seed, int tl, float *d) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)}, w[8];
  for (uint32_t c = 0; c < 2; ++c) {
    uint32_t ctr[4] = {c, 0, 0, 0};
    hqo_philox4x32_10(ctr, key, w + 4 * c);
  }
  for (int i = 0; i < tl; ++i) d[i] = ((w[i >> 5] >> (i & 31)) & 1u) ? -1.0f : 1.0f;
}
void hqo_signs(uint64_t seed, float d[TILE]) { hqo_signs_n(seed, TILE, d); }

/* Unnormalised fast Walsh-Hadamard transform, Sylvester (natural) order, in place:
 * y = H_n x with H entries +-1 (n = 64, 128 or 256).  Radix-2 stages j = 0..log2(n)-1; stage j
 * pairs index i (bit j clear) with i + 2^j, the low element becomes a + b and the high element
 * a - b, each rounded once in binary32.  The factor 1/sqrt(n) that makes H orthogonal is carried by
 * the tile scale, and the inverse uses H H = n I. */
void hqo_fwht_n(float *x, int n) {
  for (int h = 1; h < n; h <<= 1) {
    for (int i = 0; i < n; ++i) {
      if (i & h) continue;
      float a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
  }
}
void hqo_fwht128(float x[TILE]) { hqo_fwht_n(x, TILE); }

/* Sum of squares of a tile as a balanced pairwise tree in index order: the n squares (each
 * rounded once), then pairs (2i, 2i+1), then pairs of those, ... log2(n) levels. */
float hqo_sumsq_n(const float *y, int n) {
  float s[TILE_MAX];
  for (int i = 0; i < n; ++i) s[i] = y[i] * y[i];
  for (int len = n; len > 1; len >>= 1)
    for (int i = 0; i < len / 2; ++i) s[i] = s[2 * i] + s[2 * i + 1];
  return s[0];
}
float hqo_sumsq128(const float y[TILE]) { return hqo_sumsq_n(y, TILE); }

/* Round a positive finite double to the nearest bfloat16 (8 significant bits), ties to even,
 * and return the bfloat16 bit pattern.  Written with frexp/ldexp so that it is plainly the
 * definition: scale to an integer with 8 significant bits, round, scale back. */
static uint16_t bf16_rne_from_double(double r) {
  if (r == 0.0) return 0;
  int e;
  double f = frexp(r, &e);            /* r = f 2^e, f in [0.5, 1) */
  double scaled = ldexp(f, 8);        /* [128, 256) */
  double ip = floor(scaled);
  double frac = scaled - ip;
  if (frac > 0.5 || (frac == 0.5 && fmod(ip, 2.0) == 1.0)) ip += 1.0;
  float fv = (float)ldexp(ip, e - 8);  /* at most 9 significant bits: exact in binary32 */
  return (uint16_t)(bits_from_f32(fv) >> 16);
}

/* Tile scale (reading of the scaling factor alpha, HyperQuant summary Methodology component 2):
 * s = bf16_rne( sqrt(S / n) ), the root-mean-square of the unnormalised transformed tile of n
 * values, i.e. the l2 norm of the input tile.  The square root is exact (double sqrt is correctly
 * rounded and S/n is exact in double; no double-rounding case exists because a bfloat16
 * rounding midpoint squared has at most 18 significant bits).  s is stored as 16 bits per tile. */
uint16_t hqo_scale_bits_n(float S, int n) { return bf16_rne_from_double(sqrt((double)S / (double)n)); }
uint16_t hqo_scale_bits(float S) { return hqo_scale_bits_n(S, TILE); }

static float bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = bits_from_f32(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* ------------------------------------------------------------------------------------------ */
/* Nearest lattice points (HyperQuant summary, Methodology component 2: E8, D4 and Z quantisers; */
/* "E8 admits a constant-time closed-form decoder").  The decoders are the Conway-Sloane rules   */
/* (Conway & Sloane, "Fast quantizing and decoding algorithms for lattice quantizers and codes", */
/* IEEE Trans. IT 1982): round every coordinate; if the coordinate sum is odd, move the worst     */
/* rounded coordinate to its second-nearest integer; E8 = D8 u (D8 + 1/2) tries both cosets and  */
/* keeps the nearer.                                                                              */
/* Tie rules (reading): rint = round half to even; "worst" = largest |v - rint v|, lowest index   */
/* among equal values; the move goes toward v (up when v is an integer).                          */
/* ------------------------------------------------------------------------------------------ */

/* D_n for n = 4: x in Z^4 with even coordinate sum. */
static void d4_nearest(const float v[4], int32_t x[4]) {
  float a[4];
  int sgn[4], k = 0, par = 0;
  for (int i = 0; i < 4; ++i) {
    float r = rintf(v[i]);
    float e = v[i] - r;
    a[i] = fabsf(e);
    sgn[i] = signbit(e) ? -1 : 1;
    x[i] = (int32_t)r;
    par += x[i];
  }
  if (par & 1) {
    for (int i = 1; i < 4; ++i)
      if (a[i] > a[k]) k = i;
    x[k] += sgn[k];
  }
}

/* E8 in the integer embedding 2*E8 = { z in Z^8 : all z_i of one parity, sum z = 0 mod 4 }.
 * Candidate A is the nearest D8 point (even embedding 2r), candidate B the nearest point of
 * D8 + 1/2 (odd embedding).  With r = rint(v), e = v - r, a = |e|, s_i = +1 if e_i >= 0 else -1:
 *   A = r, plus s_kA at kA = argmax a if sum r is odd;
 *   B = r + s/2, minus s_kB at kB = argmin a if sum (B - 1/2) is odd (parity pA xor #{s_i<0});
 *   |v-A|^2 - |v-B|^2 = sum a - 2 + pA (1 - 2 a_kA) - pB (2 a_kB)     (exact identity)
 * and A is kept iff  sum a + pA (1 - 2 a_kA) <= 2 + pB (2 a_kB).  The left sum is evaluated as
 * ((a0+a1)+(a2+a3))+((a4+a5)+(a6+a7)), every operation rounded once in binary32. */
static void e8_nearest(const float v[8], int32_t z[8]) {
  float a[8];
  int32_t r[8];
  int sgn[8], pa = 0, nneg = 0;
  for (int i = 0; i < 8; ++i) {
    float ri = rintf(v[i]);
    float e = v[i] - ri;
    a[i] = fabsf(e);
    sgn[i] = signbit(e) ? -1 : 1;
    r[i] = (int32_t)ri;
    pa += r[i];
    nneg += (sgn[i] < 0);
  }
  pa &= 1;
  int pb = (pa + nneg) & 1;
  int ka = 0, kb = 0;
  for (int i = 1; i < 8; ++i) {
    if (a[i] > a[ka]) ka = i;
    if (a[i] < a[kb]) kb = i;
  }
  float d = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  float lhs = pa ? d + (1.0f - 2.0f * a[ka]) : d;
  float rhs = pb ? 2.0f + 2.0f * a[kb] : 2.0f;
  if (lhs <= rhs) {
    for (int i = 0; i < 8; ++i) z[i] = 2 * r[i];
    if (pa) z[ka] += 2 * sgn[ka];
  } else {
    for (int i = 0; i < 8; ++i) z[i] = 2 * r[i] + sgn[i];
    if (pb) z[kb] = 2 * r[kb] - sgn[kb];
  }
}

/* A2, the hexagonal lattice (the summary's 2-dimensional lattice), with minimal distance 1:
 *   A2 = (Z x sqrt3 Z)  u  ((Z + 1/2) x (sqrt3 Z + sqrt3/2)),
 * the union of a rectangular lattice and its shift by a deep hole.  Reading: a pair (v0, v1) is
 * quantised in "stretched" coordinates w = (v0, v1 / sqrt 3), where the lattice is
 * Z^2 u (Z + 1/2)^2 and the squared distance is dw0^2 + 3 dw1^2; the codec's scaling folds the
 * 1/sqrt 3 into the multiplier of odd slots (quantize_tile), so the input here is w.  Candidate A
 * rounds both coordinates (r = rint w, a = |w - r|), candidate B is the nearest point of the shifted
 * set, at distance 1/2 - a_i per coordinate.  Then
 *   |w-A|^2 - |w-B|^2 = a0^2 + 3 a1^2 - (1/2 - a0)^2 - 3 (1/2 - a1)^2 = a0 + 3 a1 - 1,
 * and A is kept iff fl(a0 + 3 a1) <= 1, the sum formed by one fused multiply-add (one rounding).
 * Integer code: z = 2c (the lattice point in stretched coordinates is z/2), so z0 = z1 (mod 2). */
static void a2_nearest(const float w[2], int32_t z[2]) {
  float r[2], a[2];
  int sgn[2];
  for (int i = 0; i < 2; ++i) {
    r[i] = rintf(w[i]);
    float e = w[i] - r[i];
    a[i] = fabsf(e);
    sgn[i] = signbit(e) ? -1 : 1;
  }
  if (fmaf(3.0f, a[1], a[0]) <= 1.0f) {
    for (int i = 0; i < 2; ++i) z[i] = 2 * (int32_t)r[i];
  } else {
    for (int i = 0; i < 2; ++i) z[i] = 2 * (int32_t)r[i] + sgn[i];
  }
}

/* Nearest point for one octet (8 consecutive coordinates) under `lattice`.  Output integer codes:
 * Z: z_i = rint(v_i);  D4: two D4 points;  E8: z in 2*E8 (the lattice point is z/2);
 * A2: four pairs (slots 2j, 2j+1) in stretched coordinates, z = 2c. */
int hqo_nearest_octet(int lattice, const float v[8], int32_t code[8]) {
  switch (lattice) {
    case LAT_Z:
      for (int i = 0; i < 8; ++i) code[i] = (int32_t)rintf(v[i]);
      return OK;
    case LAT_D4:
      d4_nearest(v, code);
      d4_nearest(v + 4, code + 4);
      return OK;
    case LAT_E8:
      e8_nearest(v, code);
      return OK;
    case LAT_A2:
      for (int j = 0; j < 4; ++j) a2_nearest(v + 2 * j, code + 2 * j);
      return OK;
  }
  return ERR_INVALID_ARG;
}

/* The same for `count` consecutive octets (a loop over hqo_nearest_octet, for the tests). */
int hqo_nearest_batch(int lattice, const float *v, uint64_t count, int32_t *code) {
  for (uint64_t i = 0; i < count; ++i) {
    int rc = hqo_nearest_octet(lattice, v + 8 * i, code + 8 * i);
    if (rc) return rc;
  }
  return OK;
}

/* Lattice coordinate (as a float) of an integer code: E8 and A2 codes are twice the lattice
 * point (A2: in stretched coordinates). */
static float code_to_coord(int lattice, int32_t c) {
  return (lattice == LAT_E8 || lattice == LAT_A2) ? (float)c * 0.5f : (float)c;
}

/* Subtractive dither (HyperQuant summary, Methodology component 4: add a fresh U ~ Unif(V(L))
 * before quantising and subtract it after).  Reading: for tile t and octet o, Philox calls with
 * the call's key and counter (o, t low word, t high word, 1) give four 32-bit words w; their eight
 * 16-bit halves (low half first) h_i give b_i = 2 h_i / 2^16 in [0, 2).  [0,2)^8 is a fundamental
 * domain of 2Z^8, a sublattice of E8, D4 x D4, Z^8 and (in stretched coordinates) A2^4, so b is
 * (to the draw's resolution) uniform on a union of whole cells and U = b - Q(b) is uniform on the
 * Voronoi cell V(L) (for A2 in stretched coordinates, i.e. U_1 sqrt 3 is the data-space offset).
 * Every operation here is exact in binary32.
 * The pages fix neither the generator's round count nor the draw's resolution; both are format
 * options in the dither flags (bit 0: dither on; bit 1: the dither's Philox calls take 7 rounds
 * instead of 10; bit 2: 24-bit resolution, from a second call with counter word 3 = 2: b_i =
 * 2 (w_i >> 8) / 2^24 with w_0..w_3 from the first call and w_4..w_7 from the second). */
void hqo_dither_octet_flags(uint64_t seed, uint64_t tile, int octet, int lattice, int flags, float u[8]) {
  const int rounds = (flags & 2) ? 7 : 10;
  uint32_t ctr[4] = {(uint32_t)octet, (uint32_t)tile, (uint32_t)(tile >> 32), 1u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)}, w[8];
  hqo_philox4x32_r(ctr, key, rounds, w);
  float b[8];
  int32_t q[8];
  if (flags & 4) {
    ctr[3] = 2u;
    hqo_philox4x32_r(ctr, key, rounds, w + 4);
    for (int i = 0; i < 8; ++i) b[i] = (float)(w[i] >> 8) * (1.0f / 8388608.0f);
  } else {
    for (int i = 0; i < 8; ++i) {
      uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
      b[i] = (float)h * (1.0f / 32768.0f);
    }
  }
  hqo_nearest_octet(lattice, b, q);
  for (int i = 0; i < 8; ++i) u[i] = b[i] - code_to_coord(lattice, q[i]);
}
void hqo_dither_octet(uint64_t seed, uint64_t tile, int octet, int lattice, float u[8]) {
  hqo_dither_octet_flags(seed, tile, octet, lattice, 1, u);
}

/* Valid dither flags: 0 (off), or bit 0 set with any of bits 1 and 2. */
static int valid_dither(int d) { return d == 0 || (d >= 1 && d <= 7 && (d & 1)); }

/* ------------------------------------------------------------------------------------------ */
/* Per-layer Haar-uniform rotation for KV caches (HyperQuant summary, Methodology component 4: the
 * per-layer rotation is either a full Haar-uniform matrix or the cheap +-1 sign diagonal).  The
 * pages give no construction; the reading taken is the textbook one: G with independent N(0,1)
 * entries, G = Q R with the diagonal of R positive, and Q is Haar-distributed on O(128).
 *   Gaussians: entry e = 128 i + j of G comes from Philox4x32-10 with key = seed and counter
 *   (e / 4, 0, 0, 2); the call's words w0..w3 give two Box-Muller pairs, u(w) = (w + 1/2) 2^-32,
 *   r = sqrt(-2 ln u(w0)), (r cos 2 pi u(w1), r sin 2 pi u(w1)), then the same for (w2, w3); entry
 *   e takes number e mod 4 of those four.  All in binary64.
 *   Q: modified Gram-Schmidt on the columns of G (which makes the diagonal of R positive directly).
 * Output: q[128 i + j] = Q[i][j], binary64. */
static void haar_gaussians(uint64_t seed, double g[HAAR_N * HAAR_N]) {
  const double two_pi = 6.283185307179586476925286766559;
  for (uint32_t c = 0; c < HAAR_N * HAAR_N / 4; ++c) {
    uint32_t ctr[4] = {c, 0u, 0u, 2u}, key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)}, w[4];
    hqo_philox4x32_10(ctr, key, w);
    for (int pair = 0; pair < 2; ++pair) {
      double u1 = ((double)w[2 * pair] + 0.5) * 0x1p-32, u2 = ((double)w[2 * pair + 1] + 0.5) * 0x1p-32;
      double r = sqrt(-2.0 * log(u1));
      g[4 * c + 2 * pair] = r * cos(two_pi * u2);
      g[4 * c + 2 * pair + 1] = r * sin(two_pi * u2);
    }
  }
}

void hqo_haar_gaussians(uint64_t seed, double *g) { haar_gaussians(seed, g); }

void hqo_haar_matrix(uint64_t seed, double *q) {
  double *a = (double *)malloc(sizeof(double) * HAAR_N * HAAR_N);
  haar_gaussians(seed, a);  /* a[i][j]: column j is the vector being orthonormalised */
  for (int j = 0; j < HAAR_N; ++j) {
    for (int p = 0; p < j; ++p) { /* remove the component along the finished column p */
      double dot = 0.0;
      for (int i = 0; i < HAAR_N; ++i) dot += a[i * HAAR_N + p] * a[i * HAAR_N + j];
      for (int i = 0; i < HAAR_N; ++i) a[i * HAAR_N + j] -= dot * a[i * HAAR_N + p];
    }
    double nrm = 0.0;
    for (int i = 0; i < HAAR_N; ++i) nrm += a[i * HAAR_N + j] * a[i * HAAR_N + j];
    nrm = sqrt(nrm);
    for (int i = 0; i < HAAR_N; ++i) a[i * HAAR_N + j] /= nrm;
  }
  memcpy(q, a, sizeof(double) * HAAR_N * HAAR_N);
  free(a);
}

/* ------------------------------------------------------------------------------------------ */
/* Bit-stripping (HyperQuant summary, Methodology component 3: bits that lattice membership fixes */
/* are removed losslessly before coding).  Per octet the integer codes become one raw coset bit   */
/* (E8 only) and eight symbols in slots 0..7; "halved" slots use Rice width max(k-1, 0).          */
/*   E8: p = z0 & 1 (all z_i share it: 7 bits saved), u = (z - p)/2 lies in D8, so u7's parity   */
/*       is fixed by u0..u6 (1 more bit): w = (u7 - (u0+..+u6 & 1))/2; symbols u0..u6, w.        */
/*       8 bits per octet are stripped = log2 [Z^8 : 2 E8].                                       */
/*   D4: per 4-block, w = (x3 - (x0+x1+x2 & 1))/2; symbols x0, x1, x2, w (1 bit stripped).       */
/*   A2: per pair j, p_j = z_2j & 1 is shared by both coordinates (1 bit stripped = log2 [Z^2 :  */
/*       2 A2] in stretched integer form); raw coset bit j of the octet's 4; u = (z - p_j)/2.     */
/*       The odd slots hold the stretched coordinate (1/sqrt 3 ~ 2^-0.79 of the spread of the    */
/*       even ones), so they are "halved" slots too (reading).                                   */
/*   Z : no fixed bits; symbols z0..z7.                                                          */
/* Signed symbols are mapped to unsigned by zigzag: 0,-1,1,-2,.. -> 0,1,2,3,..                    */
/* ------------------------------------------------------------------------------------------ */
static uint32_t zigzag(int32_t a) { return ((uint32_t)a << 1) ^ (uint32_t)(a >> 31); }
static int32_t unzigzag(uint32_t u) { return (int32_t)(u >> 1) ^ -(int32_t)(u & 1u); }

static int slot_halved(int lattice, int slot) {
  if (lattice == LAT_E8) return slot == 7;
  if (lattice == LAT_D4) return (slot & 3) == 3;
  if (lattice == LAT_A2) return slot & 1;
  return 0;
}
static int slot_width(int lattice, int slot, int k) {
  return slot_halved(lattice, slot) ? (k > 0 ? k - 1 : 0) : k;
}

int hqo_strip_octet(int lattice, const int32_t code[8], uint32_t sym[8], int *coset) {
  *coset = 0;
  if (lattice == LAT_Z) {
    for (int i = 0; i < 8; ++i) sym[i] = zigzag(code[i]);
    return OK;
  }
  if (lattice == LAT_D4) {
    for (int b = 0; b < 8; b += 4) {
      int32_t r = (code[b] + code[b + 1] + code[b + 2]) & 1;
      for (int i = 0; i < 3; ++i) sym[b + i] = zigzag(code[b + i]);
      sym[b + 3] = zigzag((code[b + 3] - r) / 2);
    }
    return OK;
  }
  if (lattice == LAT_E8) {
    int32_t p = code[0] & 1, u[8], r = 0;
    for (int i = 0; i < 8; ++i) u[i] = (code[i] - p) / 2;
    for (int i = 0; i < 7; ++i) r += u[i];
    r &= 1;
    for (int i = 0; i < 7; ++i) sym[i] = zigzag(u[i]);
    sym[7] = zigzag((u[7] - r) / 2);
    *coset = p;
    return OK;
  }
  if (lattice == LAT_A2) {
    for (int j = 0; j < 4; ++j) {
      int32_t p = code[2 * j] & 1;
      sym[2 * j] = zigzag((code[2 * j] - p) / 2);
      sym[2 * j + 1] = zigzag((code[2 * j + 1] - p) / 2);
      *coset |= p << j;
    }
    return OK;
  }
  return ERR_INVALID_ARG;
}

int hqo_unstrip_octet(int lattice, const uint32_t sym[8], int coset, int32_t code[8]) {
  if (lattice == LAT_Z) {
    for (int i = 0; i < 8; ++i) code[i] = unzigzag(sym[i]);
    return OK;
  }
  if (lattice == LAT_D4) {
    for (int b = 0; b < 8; b += 4) {
      for (int i = 0; i < 3; ++i) code[b + i] = unzigzag(sym[b + i]);
      int32_t r = (code[b] + code[b + 1] + code[b + 2]) & 1;
      code[b + 3] = 2 * unzigzag(sym[b + 3]) + r;
    }
    return OK;
  }
  if (lattice == LAT_E8) {
    int32_t u[8], r = 0;
    for (int i = 0; i < 7; ++i) { u[i] = unzigzag(sym[i]); r += u[i]; }
    u[7] = 2 * unzigzag(sym[7]) + (r & 1);
    for (int i = 0; i < 8; ++i) code[i] = 2 * u[i] + coset;
    return OK;
  }
  if (lattice == LAT_A2) {
    for (int i = 0; i < 8; ++i) code[i] = 2 * unzigzag(sym[i]) + ((coset >> (i / 2)) & 1);
    return OK;
  }
  return ERR_INVALID_ARG;
}

/* Remainder bits per octet and fixed bits per tile record F of a tile of tl values (tl/8 octets):
 * 16 (scale) + coset bits (E8: one per octet; A2: one per pair) + tl/8 * (sum of slot widths). */
static int octet_rem_bits(int lattice, int k) {
  int b = 0;
  for (int s = 0; s < 8; ++s) b += slot_width(lattice, s, k);
  return b;
}
uint32_t hqo_tile_fixed_bits_n(int lattice, int k, int tl) {
  const uint32_t oct = (uint32_t)tl / 8u;
  const uint32_t coset = lattice == LAT_E8 ? oct : lattice == LAT_A2 ? 4u * oct : 0u;
  return 16u + coset + oct * (uint32_t)octet_rem_bits(lattice, k);
}
uint32_t hqo_tile_fixed_bits(int lattice, int k) { return hqo_tile_fixed_bits_n(lattice, k, TILE); }

static int valid_tile(int tl) { return tl == 64 || tl == 128 || tl == 256; }
static int log2_int(uint64_t v) { int l = 0; while (v > 1) { v >>= 1; ++l; } return l; }

/* ------------------------------------------------------------------------------------------ */
/* Per-tile quantiser (the front half of the encoder).                                          */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
  int lattice, dither, tl;
  uint64_t seed;
  float d[TILE_MAX];
} qctx;

static void qctx_init(qctx *q, int lattice, int dither, uint64_t seed, int tl) {
  q->lattice = lattice;
  q->dither = dither;
  q->seed = seed;
  q->tl = tl;
  hqo_signs_n(seed, tl, q->d);
}

/* Reconstruction factor t and multiplier m of a tile, per slot parity.  Every lattice:
 * t = s * step, m = 1 / t (each rounded once in binary32; m = 0 when s = 0).  A2 odd slots (the
 * second coordinate of a pair): t' = t * R3 and m' = 1 / t', which takes that coordinate into the
 * stretched coordinates of a2_nearest on the way in and back on the way out. */
static void tile_factors(int lattice, float s, float step, float m[2], float t[2]) {
  t[0] = s * step;
  m[0] = (s != 0.0f) ? 1.0f / t[0] : 0.0f;
  if (lattice == LAT_A2) {
    t[1] = t[0] * f32_from_bits(A2_R3_BITS);
    m[1] = (s != 0.0f) ? 1.0f / t[1] : 0.0f;
  } else {
    t[1] = t[0];
    m[1] = m[0];
  }
}

/* Quantise tile `t` (values x[0..tl-1]) at step `step`: returns the scale bits and tl integer
 * codes; returns ERR_NONFINITE if the transformed tile's energy is not finite.
 *   y = H (D x);  S = sumsq(y);  s = bf16(sqrt(S/tl));
 *   m = 1 / (s * step)  (binary32 product then division; m = 0 when s = 0; A2's odd slots use
 *   the m' of tile_factors);
 *   v = y * m  (+ U for the dithered path);  codes = nearest lattice point per octet. */
static int quantize_tile(const qctx *q, uint64_t t, const float *x, float step, uint16_t *scale_out,
                         int32_t *code) {
  float y[TILE_MAX];
  for (int i = 0; i < q->tl; ++i) y[i] = q->d[i] * x[i];
  hqo_fwht_n(y, q->tl);
  float S = hqo_sumsq_n(y, q->tl);
  if (!isfinite(S)) return ERR_NONFINITE;
  uint16_t sb = hqo_scale_bits_n(S, q->tl);
  float s = bf16_to_f32(sb);
  float m[2], tf[2];
  tile_factors(q->lattice, s, step, m, tf);
  for (int o = 0; o < q->tl / 8; ++o) {
    float v[8];
    for (int i = 0; i < 8; ++i) v[i] = y[8 * o + i] * m[i & 1];
    if (q->dither) {
      float u[8];
      hqo_dither_octet_flags(q->seed, t, o, q->lattice, q->dither, u);
      for (int i = 0; i < 8; ++i) v[i] = v[i] + u[i];
    }
    hqo_nearest_octet(q->lattice, v, code + 8 * o);
  }
  *scale_out = sb;
  return OK;
}

/* Inverse of the quantiser for one tile: c = code coordinate; yhat = (c - U) * (s * step);
 * xhat = D (H yhat) / tl (an exact power-of-two factor because H H = tl I).  Reading: a decoded
 * value that is exactly zero is +0 (the pages do not speak of signed zeros; the sign of an exact
 * cancellation depends on the order of the butterflies, not on the data). */
static void dequantize_tile(const qctx *q, uint64_t t, const int32_t *code, uint16_t sb, float step,
                            float *out) {
  float s = bf16_to_f32(sb);
  float m[2], tf[2];
  tile_factors(q->lattice, s, step, m, tf);
  float y[TILE_MAX];
  for (int o = 0; o < q->tl / 8; ++o) {
    float u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (q->dither) hqo_dither_octet_flags(q->seed, t, o, q->lattice, q->dither, u);
    for (int i = 0; i < 8; ++i) {
      float c = code_to_coord(q->lattice, code[8 * o + i]);
      float cu = q->dither ? c - u[i] : c;
      y[8 * o + i] = cu * tf[i & 1];
    }
  }
  hqo_fwht_n(y, q->tl);
  const float inv = 1.0f / (float)q->tl;  /* 2^-6, 2^-7 or 2^-8: exact */
  for (int i = 0; i < q->tl; ++i) {
    float o = q->d[i] * (y[i] * inv);
    out[i] = (o == 0.0f) ? 0.0f : o;
  }
}

static void load_tile(const void *x, int dtype, uint64_t t, int tl, float *out) {
  if (dtype == 0) {
    memcpy(out, (const float *)x + t * (uint64_t)tl, sizeof(float) * (size_t)tl);
  } else {
    const uint16_t *p = (const uint16_t *)x + t * (uint64_t)tl;
    for (int i = 0; i < tl; ++i) out[i] = bf16_to_f32(p[i]);
  }
}

/* Per-value integer codes and per-tile scale bits at a fixed step (diagnostic form of the
 * encoder's front half; the GPU exposes the same thing for code-level parity). */
int hqo_quantize(const void *x, int dtype, uint64_t n, int lattice, int dither, uint64_t seed,
                 float step, int32_t *codes, uint16_t *scales, int tl) {
  if (!valid_tile(tl) || n % (uint64_t)tl || !valid_dither(dither)) return ERR_INVALID_ARG;
  if (lattice < LAT_Z || lattice > LAT_A2) return ERR_INVALID_ARG;
  qctx q;
  qctx_init(&q, lattice, dither, seed, tl);
  uint64_t T = n / (uint64_t)tl;
  for (uint64_t t = 0; t < T; ++t) {
    float xt[TILE_MAX];
    load_tile(x, dtype, t, tl, xt);
    int rc = quantize_tile(&q, t, xt, step, &scales[t], codes + t * (uint64_t)tl);
    if (rc) return rc;
  }
  return OK;
}

/* The binary32 inputs v of the nearest-point step at a fixed step (for locating a code mismatch
 * relative to the Voronoi boundary in the tests). */
int hqo_lattice_inputs(const void *x, int dtype, uint64_t n, int lattice, int dither, uint64_t seed,
                       float step, float *v_out, int tl) {
  if (!valid_tile(tl) || n % (uint64_t)tl || !valid_dither(dither)) return ERR_INVALID_ARG;
  qctx q;
  qctx_init(&q, lattice, dither, seed, tl);
  for (uint64_t t = 0; t < n / (uint64_t)tl; ++t) {
    float y[TILE_MAX];
    load_tile(x, dtype, t, tl, y);
    for (int i = 0; i < tl; ++i) y[i] = q.d[i] * y[i];
    hqo_fwht_n(y, tl);
    float S = hqo_sumsq_n(y, tl);
    if (!isfinite(S)) return ERR_NONFINITE;
    float s = bf16_to_f32(hqo_scale_bits_n(S, tl));
    float m[2], tf[2];
    tile_factors(lattice, s, step, m, tf);
    for (int o = 0; o < tl / 8; ++o) {
      float u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (dither) hqo_dither_octet_flags(seed, t, o, lattice, dither, u);
      for (int i = 0; i < 8; ++i) {
        float v = y[8 * o + i] * m[i & 1];
        v_out[t * (uint64_t)tl + 8 * o + i] = dither ? v + u[i] : v;
      }
    }
  }
  return OK;
}

int hqo_dequantize(const int32_t *codes, const uint16_t *scales, uint64_t n, int lattice,
                   int dither, uint64_t seed, float step, float *out, int tl) {
  if (!valid_tile(tl) || n % (uint64_t)tl || !valid_dither(dither)) return ERR_INVALID_ARG;
  qctx q;
  qctx_init(&q, lattice, dither, seed, tl);
  for (uint64_t t = 0; t < n / (uint64_t)tl; ++t)
    dequantize_tile(&q, t, codes + t * (uint64_t)tl, scales[t], step, out + t * (uint64_t)tl);
  return OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Rate control (HyperQuant summary, Methodology component 3: "the realised rate lands within     */
/* ~0.01 bps of the target").  The pages give no algorithm; reading:                              */
/*  - payload rate = (coset bits + Rice bits) / values; the 16-bit tile scales, the chunk index  */
/*    and padding are side information, reported apart;                                          */
/*  - a jittered stratified sample of N = min(T, 2048) tiles for pass A and min(T, 8192) for pass */
/*    B: stratum i = [floor(iT/N), floor((i+1)T/N)), one tile per stratum chosen by a 32-bit      */
/*    integer hash of i;                                                                          */
/*  - the search variable is b = the binary32 bit pattern of the step (b / 2^23 - 127 is a        */
/*    piecewise-linear log2 of the step);                                                         */
/*  - pass A evaluates 8 candidates b0 + (2j-7) 2^21 (quarter-octave spacing) around the Gaussian */
/*    high-rate guess log2 step = 2.05 - target; pass B 4 candidates (2j-3) 2^18 (1/16 octave)     */
/*    around pass A's answer.  Pass A lands within a few hundredths of an octave of the final     */
/*    answer, well inside pass B's +-3/32 octave, and its result hardly depends on its sample     */
/*    size, so the coarse pass uses the smaller sample;                                           */
/*  - each candidate's Rice parameter is the argmin (ties to the smaller k) over the window        */
/*    kb..kb+3, kb = clamp(-e - 2, 0, 12), e = the step's binary exponent;                        */
/*  - after a pass, the answer is the linear interpolation between the two candidates that        */
/*    bracket the target bit count (first candidate at or below it), or a linear extrapolation    */
/*    from the two end candidates (at most 2^25 beyond them), all in IEEE double, rounded to the  */
/*    nearest integer and clamped to [2^-12, 2^12]; k is taken from the candidate nearest the      */
/*    answer (ties to the lower index).                                                           */
/* ------------------------------------------------------------------------------------------ */
static uint32_t hash32(uint32_t x) {
  x = x * 0x9E3779B1u + 0x7F4A7C15u;
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}

uint64_t hqo_sample_tile(uint64_t i, uint64_t T, uint64_t N) {
  uint64_t lo = (i * T) / N, hi = ((i + 1) * T) / N;
  return lo + (uint64_t)hash32((uint32_t)i) % (hi - lo);
}

static int kwin_base(int64_t b) {
  int e = (int)((b >> 23) & 0xFF) - 127;
  int kb = -e - 2;
  if (kb < 0) kb = 0;
  if (kb > 12) kb = 12;
  return kb;
}

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

static void rc_solve(int nc, const int64_t b[], const double R[], double Tb, double nominal_slope,
                     int64_t *b_out, int *j_near) {
  double x;
  int j = -1;
  for (int i = 0; i < nc; ++i)
    if (R[i] <= Tb) { j = i; break; }
  int64_t lo = 0, hi = 0;
  if (nc == 1) {
    x = (double)b[0];
    lo = hi = b[0];
  } else if (j < 0) {
    double slope = (R[nc - 2] - R[nc - 1]) / (double)(b[nc - 1] - b[nc - 2]);
    if (!(slope > 0.0)) slope = nominal_slope;
    x = (double)b[nc - 1] + (R[nc - 1] - Tb) / slope;
    lo = b[nc - 1];
    hi = b[nc - 1] + ((int64_t)1 << 25);
  } else if (j == 0) {
    double slope = (R[0] - R[1]) / (double)(b[1] - b[0]);
    if (!(slope > 0.0)) slope = nominal_slope;
    x = (double)b[0] - (Tb - R[0]) / slope;
    lo = b[0] - ((int64_t)1 << 25);
    hi = b[0];
  } else {
    x = (double)b[j - 1] + (R[j - 1] - Tb) * (double)(b[j] - b[j - 1]) / (R[j - 1] - R[j]);
    lo = b[j - 1];
    hi = b[j];
  }
  int64_t xb = (int64_t)floor(x + 0.5);
  xb = clamp64(xb, lo, hi);
  xb = clamp64(xb, STEP_BITS_MIN, STEP_BITS_MAX);
  int best = 0;
  for (int i = 1; i < nc; ++i) {
    int64_t di = llabs(b[i] - xb), db = llabs(b[best] - xb);
    if (di < db) best = i;
  }
  *b_out = xb;
  *j_near = best;
}

/* Evaluate the sample at `nc` candidate steps: sumq[c][w] = sum over sample symbols of
 * (symbol >> width) with Rice parameter kb(c) + w.  Returns ERR_NONFINITE on a bad tile. */
static int rc_eval(const qctx *q, const void *x, int dtype, uint64_t T, uint64_t N, int nc,
                   const int64_t b[], int fixed_k, uint64_t sumq[][RC_KWIN]) {
  for (int c = 0; c < nc; ++c)
    for (int w = 0; w < RC_KWIN; ++w) sumq[c][w] = 0;
  for (uint64_t i = 0; i < N; ++i) {
    uint64_t t = hqo_sample_tile(i, T, N);
    float xt[TILE_MAX];
    load_tile(x, dtype, t, q->tl, xt);
    for (int c = 0; c < nc; ++c) {
      uint16_t sb;
      int32_t code[TILE_MAX];
      int rc = quantize_tile(q, t, xt, f32_from_bits((uint32_t)b[c]), &sb, code);
      if (rc) return rc;
      int kb = fixed_k >= 0 ? fixed_k : kwin_base(b[c]);
      for (int o = 0; o < q->tl / 8; ++o) {
        uint32_t sym[8];
        int cos;
        hqo_strip_octet(q->lattice, code + 8 * o, sym, &cos);
        for (int w = 0; w < RC_KWIN; ++w) {
          int k = fixed_k >= 0 ? fixed_k : kb + w;
          for (int s = 0; s < 8; ++s) sumq[c][w] += sym[s] >> slot_width(q->lattice, s, k);
        }
      }
    }
  }
  return OK;
}

/* Total payload bits of a candidate for Rice parameter k. */
/* Lowest reachable payload rate: one unary bit per value plus the raw coset bits (E8: 1/8, A2:
 * 1/2 bit per value). */
static float min_bps(int lattice) {
  return lattice == LAT_E8 ? 1.125f : lattice == LAT_A2 ? 1.5f : 1.0f;
}

static double rc_bits(int lattice, uint64_t N, int k, uint64_t sumq, int tl) {
  double per_tile = (double)(hqo_tile_fixed_bits_n(lattice, k, tl) - 16u) + (double)tl;
  return per_tile * (double)N + (double)sumq;
}

/* Output: chosen step bits, Rice k, and the sample payload estimate (bits/value) by interpolation. */
int hqo_rate(const void *x, int dtype, uint64_t n, int lattice, int dither, uint64_t seed,
             float target_bps, float step, int rice_k, uint32_t *step_bits_out, int *k_out, int tl) {
  if (!valid_tile(tl) || n % (uint64_t)tl || !valid_dither(dither)) return ERR_INVALID_ARG;
  if (lattice < LAT_Z || lattice > LAT_A2) return ERR_INVALID_ARG;
  if (rice_k < -1 || rice_k > 15) return ERR_INVALID_ARG;
  qctx q;
  qctx_init(&q, lattice, dither, seed, tl);
  uint64_t T = n / (uint64_t)tl;
  uint64_t N = T < RC_SAMPLE_TILES ? T : RC_SAMPLE_TILES;
  int64_t b_ans;
  int k_ans;
  if (step > 0.0f) {
    b_ans = (int64_t)bits_from_f32(step);
    if (b_ans < STEP_BITS_MIN || b_ans > STEP_BITS_MAX) return ERR_INVALID_ARG;
    if (rice_k >= 0 || N == 0) {
      *step_bits_out = (uint32_t)b_ans;
      *k_out = rice_k >= 0 ? rice_k : kwin_base(b_ans) + 1;
      return OK;
    }
    /* fixed step, automatic k: one candidate, argmin over the window */
    int64_t b[1] = {b_ans};
    uint64_t sumq[1][RC_KWIN];
    int rc = rc_eval(&q, x, dtype, T, N, 1, b, -1, sumq);
    if (rc) return rc;
    int kb = kwin_base(b_ans), best = 0;
    for (int w = 1; w < RC_KWIN; ++w)
      if (rc_bits(lattice, N, kb + w, sumq[0][w], tl) < rc_bits(lattice, N, kb + best, sumq[0][best], tl))
        best = w;
    *step_bits_out = (uint32_t)b_ans;
    *k_out = kb + best;
    return OK;
  }
  if (!(target_bps >= min_bps(lattice)) || !(target_bps <= 12.0f)) return ERR_RATE;
  int64_t b0 = (int64_t)(127u << 23) + (int64_t)floor((2.05 - (double)target_bps) * 8388608.0 + 0.5);
  if (N == 0) {
    *step_bits_out = (uint32_t)clamp64(b0, STEP_BITS_MIN, STEP_BITS_MAX);
    *k_out = rice_k >= 0 ? rice_k : kwin_base(b0) + 1;
    return OK;
  }
  int64_t centre = b0;
  const uint64_t np[2] = {T < RC_SAMPLE_TILES_A ? T : RC_SAMPLE_TILES_A, N};
  const int ncand[2] = {RC_CANDIDATES, RC_CANDIDATES_B};
  const int half_log2[2] = {21, 18};
  for (int pass = 0; pass < 2; ++pass) {
    const uint64_t Np = np[pass];
    const int nc = ncand[pass];
    const double Tb = (double)target_bps * (double)(Np * (uint64_t)tl);
    const double nominal = (double)(Np * (uint64_t)tl) / 8388608.0;
    int64_t b[RC_CANDIDATES];
    for (int j = 0; j < nc; ++j)
      b[j] = clamp64(centre + (int64_t)(2 * j - (nc - 1)) * ((int64_t)1 << half_log2[pass]),
                     STEP_BITS_MIN, STEP_BITS_MAX);
    uint64_t sumq[RC_CANDIDATES][RC_KWIN];
    int rc = rc_eval(&q, x, dtype, T, Np, nc, b, rice_k, sumq);
    if (rc) return rc;
    double R[RC_CANDIDATES];
    int kc[RC_CANDIDATES];
    for (int j = 0; j < nc; ++j) {
      int kb = rice_k >= 0 ? rice_k : kwin_base(b[j]);
      int best = 0;
      double rb = rc_bits(lattice, Np, rice_k >= 0 ? rice_k : kb, sumq[j][0], tl);
      for (int w = 1; w < RC_KWIN; ++w) {
        double rw = rc_bits(lattice, Np, rice_k >= 0 ? rice_k : kb + w, sumq[j][w], tl);
        if (rw < rb) { rb = rw; best = w; }
      }
      R[j] = rb;
      kc[j] = rice_k >= 0 ? rice_k : kb + best;
    }
    int jn;
    rc_solve(nc, b, R, Tb, nominal, &centre, &jn);
    k_ans = kc[jn];
  }
  b_ans = centre;
  *step_bits_out = (uint32_t)b_ans;
  *k_out = k_ans;
  return OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Bitstream (format version 1; a definition of this codec, the pages give none).               */
/* All multi-byte fields little-endian; bit i of a bit plane is bit (i mod 8) of byte i/8.       */
/*  header (128 B): magic u32 | version u16 | lattice u8 | flags u8 (bit0 dither) | tile u16 |   */
/*    rice k u8 | log2 chunk tiles u8 | step bits u32 | seed u64 | n u64 | tiles u64 |           */
/*    chunks u32 | F u32 (fixed bits per tile record) | fixed_off u64 | unary_off u64 |          */
/*    unary_words u64 | unary_bits u64 | payload_bits u64 | total_bytes u64 | 32 B zero        */
/*  chunk index at byte 128: chunks+1 u32 word offsets (64-bit words) into the unary plane       */
/*  fixed plane at fixed_off = align256(128 + 4 (chunks+1)): chunk c holds tiles 64c..64c+63,    */
/*    8F bytes; tile record t at bit t F: scale bf16 (16) | E8 coset bits, bit o = octet o (16), */
/*    or A2 coset bits, bit 4o + j = pair j of octet o (64) | for octet 0..15, slot 0..7:        */
/*    remainder (slot width bits, least significant first);                                      */
/*    tiles past the end of the tensor are zero bits                                             */
/*  unary plane at unary_off = align256(fixed_off + 8F chunks): chunk c's segment starts at     */
/*    64-bit word index[c]; for each symbol in (tile, octet, slot) order: q = symbol >> width    */
/*    zero bits then a one; the segment is zero-padded to a 64-bit boundary.                     */
/* ------------------------------------------------------------------------------------------ */
static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_u64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) { uint32_t v = 0; for (int i = 3; i >= 0; --i) v = (v << 8) | p[i]; return v; }
static uint64_t get_u64(const uint8_t *p) { uint64_t v = 0; for (int i = 7; i >= 0; --i) v = (v << 8) | p[i]; return v; }

static void put_bit(uint8_t *buf, uint64_t pos, int bit) {
  if (bit) buf[pos >> 3] |= (uint8_t)(1u << (pos & 7));
}
static int get_bit(const uint8_t *buf, uint64_t pos) { return (buf[pos >> 3] >> (pos & 7)) & 1; }
static void put_bits(uint8_t *buf, uint64_t pos, uint32_t val, int nbits) {
  for (int i = 0; i < nbits; ++i) put_bit(buf, pos + (uint64_t)i, (int)((val >> i) & 1u));
}
static uint32_t get_bits(const uint8_t *buf, uint64_t pos, int nbits) {
  uint32_t v = 0;
  for (int i = 0; i < nbits; ++i) v |= (uint32_t)get_bit(buf, pos + (uint64_t)i) << i;
  return v;
}

static uint32_t low_mask(int w) { return w >= 32 ? 0xFFFFFFFFu : ((1u << w) - 1u); }
static uint64_t align256(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

/* Byte layout helpers shared by encoder and decoder of this file. */
typedef struct {
  uint64_t T, chunks, fixed_off, unary_off, ctiles;
  uint32_t F;
  int tl;
} layout;

static layout make_layout(uint64_t n, int lattice, int k, int tl) {
  layout L;
  L.tl = tl;
  L.T = n / (uint64_t)tl;
  L.ctiles = CHUNK_VALUES / (uint64_t)tl;
  L.chunks = (L.T + L.ctiles - 1) / L.ctiles;
  L.F = hqo_tile_fixed_bits_n(lattice, k, tl);
  L.fixed_off = align256(HEADER_BYTES + 4u * (L.chunks + 1));
  L.unary_off = align256(L.fixed_off + L.chunks * L.ctiles * L.F / 8u);
  return L;
}

/* Rice round trip for tests: remainders go to `fixed` at bits w*i.., unary codes to `unary`.
 * Uses the same bit writer and reader as the stream encoder and decoder below. */
int hqo_rice_roundtrip(const uint32_t *vals, uint64_t count, int k, uint32_t *out,
                       uint8_t *fixed, uint8_t *unary, uint64_t unary_cap_bits, uint64_t *unary_len) {
  uint64_t up = 0;
  for (uint64_t i = 0; i < count; ++i) {
    uint32_t q = vals[i] >> k;
    if (up + q + 1 > unary_cap_bits) return ERR_CAPACITY;
    put_bits(fixed, (uint64_t)k * i, vals[i] & low_mask(k), k);
    up += q;
    put_bit(unary, up, 1);
    up += 1;
  }
  *unary_len = up;
  uint64_t rp = 0;
  for (uint64_t i = 0; i < count; ++i) {
    uint32_t q = 0;
    while (!get_bit(unary, rp)) { ++q; ++rp; }
    ++rp;
    out[i] = (q << k) | get_bits(fixed, (uint64_t)k * i, k);
  }
  return OK;
}

int hqo_encode_layout(uint64_t n, int lattice, int k, uint64_t *fixed_off, uint64_t *unary_off,
                      uint32_t *F, int tl) {
  if (!valid_tile(tl)) return ERR_INVALID_ARG;
  layout L = make_layout(n, lattice, k, tl);
  *fixed_off = L.fixed_off;
  *unary_off = L.unary_off;
  *F = L.F;
  return OK;
}

/* Full encoder.  Writes the stream into out[0..cap); returns ERR_CAPACITY with *out_bytes set to
 * the required size when it does not fit.  info[0..3] = step bits, k, payload bits, unary bits. */
int hqo_encode(const void *x, int dtype, uint64_t n, int lattice, int dither, uint64_t seed,
               float target_bps, float step, int rice_k, uint8_t *out, uint64_t cap,
               uint64_t *out_bytes, uint64_t info[4], int tl) {
  if (!valid_tile(tl) || n % (uint64_t)tl || !valid_dither(dither)) return ERR_INVALID_ARG;
  if (lattice < LAT_Z || lattice > LAT_A2) return ERR_INVALID_ARG;
  uint32_t sbits;
  int k;
  int rc = hqo_rate(x, dtype, n, lattice, dither, seed, target_bps, step, rice_k, &sbits, &k, tl);
  if (rc) return rc;
  float st = f32_from_bits(sbits);
  qctx q;
  qctx_init(&q, lattice, dither, seed, tl);
  layout L = make_layout(n, lattice, k, tl);
  int32_t *codes = (int32_t *)malloc(sizeof(int32_t) * (n ? n : 1));
  uint16_t *scales = (uint16_t *)malloc(sizeof(uint16_t) * (L.T ? L.T : 1));
  uint64_t *chunk_bits = (uint64_t *)calloc(L.chunks + 1, sizeof(uint64_t));
  if (!codes || !scales || !chunk_bits) { free(codes); free(scales); free(chunk_bits); return ERR_INVALID_ARG; }
  /* quantise and measure each chunk's unary length */
  for (uint64_t t = 0; t < L.T; ++t) {
    float xt[TILE_MAX];
    load_tile(x, dtype, t, tl, xt);
    rc = quantize_tile(&q, t, xt, st, &scales[t], codes + t * (uint64_t)tl);
    if (rc) { free(codes); free(scales); free(chunk_bits); return rc; }
    for (int o = 0; o < tl / 8; ++o) {
      uint32_t sym[8];
      int cos;
      hqo_strip_octet(lattice, codes + t * (uint64_t)tl + 8 * o, sym, &cos);
      for (int s = 0; s < 8; ++s) chunk_bits[t / L.ctiles] += (sym[s] >> slot_width(lattice, s, k)) + 1u;
    }
  }
  uint64_t words = 0, ubits = 0;
  for (uint64_t c = 0; c < L.chunks; ++c) { words += (chunk_bits[c] + 63u) / 64u; ubits += chunk_bits[c]; }
  uint64_t total = L.unary_off + 8u * words;
  *out_bytes = total;
  uint64_t payload = L.T * (uint64_t)(L.F - 16u) + ubits;
  info[0] = sbits; info[1] = (uint64_t)k; info[2] = payload; info[3] = ubits;
  if (total > cap) { free(codes); free(scales); free(chunk_bits); return ERR_CAPACITY; }
  memset(out, 0, total);
  /* header */
  put_u32(out + 0, MAGIC);
  put_u16(out + 4, VERSION);
  out[6] = (uint8_t)lattice;
  out[7] = (uint8_t)dither;  /* the dither flags */
  put_u16(out + 8, (uint16_t)tl);
  out[10] = (uint8_t)k;
  out[11] = (uint8_t)log2_int(L.ctiles);
  put_u32(out + 12, sbits);
  put_u64(out + 16, seed);
  put_u64(out + 24, n);
  put_u64(out + 32, L.T);
  put_u32(out + 40, (uint32_t)L.chunks);
  put_u32(out + 44, L.F);
  put_u64(out + 48, L.fixed_off);
  put_u64(out + 56, L.unary_off);
  put_u64(out + 64, words);
  put_u64(out + 72, ubits);
  put_u64(out + 80, payload);
  put_u64(out + 88, total);
  /* index, fixed plane, unary plane */
  uint8_t *fixed = out + L.fixed_off, *unary = out + L.unary_off;
  uint64_t wpos = 0;
  for (uint64_t c = 0; c < L.chunks; ++c) {
    put_u32(out + HEADER_BYTES + 4u * c, (uint32_t)wpos);
    uint64_t upos = wpos * 64u;
    for (uint64_t t = c * L.ctiles; t < (c + 1) * L.ctiles && t < L.T; ++t) {
      uint64_t fp = t * (uint64_t)L.F;
      put_bits(fixed, fp, scales[t], 16);
      fp += 16;
      uint64_t coset_pos = fp;
      if (lattice == LAT_E8) fp += (uint64_t)(tl / 8);
      if (lattice == LAT_A2) fp += (uint64_t)(tl / 2);
      for (int o = 0; o < tl / 8; ++o) {
        uint32_t sym[8];
        int cos;
        hqo_strip_octet(lattice, codes + t * (uint64_t)tl + 8 * o, sym, &cos);
        if (lattice == LAT_E8) put_bit(fixed, coset_pos + (uint64_t)o, cos);
        if (lattice == LAT_A2) put_bits(fixed, coset_pos + 4u * (uint64_t)o, (uint32_t)cos, 4);
        for (int s = 0; s < 8; ++s) {
          int w = slot_width(lattice, s, k);
          put_bits(fixed, fp, sym[s] & low_mask(w), w);
          fp += (uint64_t)w;
          upos += sym[s] >> w;
          put_bit(unary, upos, 1);
          upos += 1;
        }
      }
    }
    wpos += (chunk_bits[c] + 63u) / 64u;
  }
  put_u32(out + HEADER_BYTES + 4u * L.chunks, (uint32_t)wpos);
  free(codes); free(scales); free(chunk_bits);
  return OK;
}

/* Full decoder: validates the header and every chunk, then reconstructs.  out_dtype 0 = fp32,
 * 1 = bf16 (round to nearest even). */
/* Stream reader shared by the decoders below: validates the header and index, and hands every tile's
 * integer codes and scale bits to `sink` in tile order (format v1, see hqo_encode_layout). */
typedef void (*tile_sink)(void *ctx, const qctx *q, uint64_t t, const int32_t *code, uint16_t sb, float step);

static int read_stream(const uint8_t *s, uint64_t bytes, uint64_t n, tile_sink sink, void *ctx) {
  if (bytes < HEADER_BYTES) return ERR_CORRUPT;
  if (get_u32(s) != MAGIC || get_u16(s + 4) != VERSION) return ERR_CORRUPT;
  int lattice = s[6], dither = s[7], k = s[10], tl = get_u16(s + 8);
  if (lattice > LAT_A2 || !valid_dither(dither) || !valid_tile(tl) || k > 15) return ERR_CORRUPT;
  if (s[11] != log2_int(CHUNK_VALUES / (uint64_t)tl)) return ERR_CORRUPT;
  if (get_u64(s + 24) != n || n % (uint64_t)tl) return ERR_CORRUPT;
  uint32_t sbits = get_u32(s + 12);
  if (sbits < STEP_BITS_MIN || sbits > STEP_BITS_MAX) return ERR_CORRUPT;
  uint64_t seed = get_u64(s + 16);
  layout L = make_layout(n, lattice, k, tl);
  if (get_u64(s + 32) != L.T || get_u32(s + 40) != (uint32_t)L.chunks || get_u32(s + 44) != L.F ||
      get_u64(s + 48) != L.fixed_off || get_u64(s + 56) != L.unary_off)
    return ERR_CORRUPT;
  uint64_t words = get_u64(s + 64), total = get_u64(s + 88);
  if (total > bytes || L.unary_off + 8u * words != total) return ERR_CORRUPT;
  if (HEADER_BYTES + 4u * (L.chunks + 1) > bytes) return ERR_CORRUPT;
  if (get_u32(s + HEADER_BYTES) != 0 || get_u32(s + HEADER_BYTES + 4u * L.chunks) != words) return ERR_CORRUPT;
  float st = f32_from_bits(sbits);
  qctx q;
  qctx_init(&q, lattice, dither, seed, tl);
  const uint8_t *fixed = s + L.fixed_off, *unary = s + L.unary_off;
  for (uint64_t c = 0; c < L.chunks; ++c) {
    uint32_t w0 = get_u32(s + HEADER_BYTES + 4u * c), w1 = get_u32(s + HEADER_BYTES + 4u * (c + 1));
    if (w1 < w0 || w1 > words) return ERR_CORRUPT;
    uint64_t upos = (uint64_t)w0 * 64u, uend = (uint64_t)w1 * 64u;
    for (uint64_t t = c * L.ctiles; t < (c + 1) * L.ctiles && t < L.T; ++t) {
      uint64_t fp = t * (uint64_t)L.F;
      uint16_t sb = (uint16_t)get_bits(fixed, fp, 16);
      fp += 16;
      uint64_t coset_pos = fp;
      if (lattice == LAT_E8) fp += (uint64_t)(tl / 8);
      if (lattice == LAT_A2) fp += (uint64_t)(tl / 2);
      int32_t code[TILE_MAX];
      for (int o = 0; o < tl / 8; ++o) {
        uint32_t sym[8];
        for (int sl = 0; sl < 8; ++sl) {
          int w = slot_width(lattice, sl, k);
          uint32_t r = get_bits(fixed, fp, w);
          fp += (uint64_t)w;
          uint32_t qv = 0;
          while (1) {
            if (upos >= uend) return ERR_CORRUPT;
            if (get_bit(unary, upos)) break;
            ++qv; ++upos;
            if (qv > (0xFFFFFFFFu >> w)) return ERR_CORRUPT;
          }
          ++upos;
          sym[sl] = (qv << w) | r;
        }
        int cos = lattice == LAT_E8   ? get_bit(fixed, coset_pos + (uint64_t)o)
                  : lattice == LAT_A2 ? (int)get_bits(fixed, coset_pos + 4u * (uint64_t)o, 4)
                                      : 0;
        hqo_unstrip_octet(lattice, sym, cos, code + 8 * o);
      }
      sink(ctx, &q, t, code, sb, st);
    }
    /* the rest of the segment must be padding */
    while (upos < uend) { if (get_bit(unary, upos)) return ERR_CORRUPT; ++upos; }
  }
  return OK;
}

typedef struct { void *out; int out_dtype; } decode_ctx;

static void decode_sink(void *ctx, const qctx *q, uint64_t t, const int32_t *code, uint16_t sb, float step) {
  const decode_ctx *d = (const decode_ctx *)ctx;
  const int tl = q->tl;
  float xt[TILE_MAX];
  dequantize_tile(q, t, code, sb, step, xt);
  if (d->out_dtype == 0) {
    memcpy((float *)d->out + t * (uint64_t)tl, xt, sizeof(float) * (size_t)tl);
  } else {
    uint16_t *o16 = (uint16_t *)d->out + t * (uint64_t)tl;
    for (int i = 0; i < tl; ++i) o16[i] = f32_to_bf16_rne(xt[i]);
  }
}

int hqo_decode(const uint8_t *s, uint64_t bytes, uint64_t n, void *out, int out_dtype) {
  decode_ctx d = {out, out_dtype};
  return read_stream(s, bytes, n, decode_sink, &d);
}

/* The decoder's values before the inverse transform, in binary64: yhat_i = (c_i - U_i) * t with
 * t = s * step the binary32 product both sides use (dequantize_tile; A2's odd slots take its t'),
 * so that the exact reconstruction of tile t is D H yhat / tl.  Test infrastructure for products
 * with the decoded matrix (the fused decode + matrix-vector product). */
static void coords_sink(void *ctx, const qctx *q, uint64_t t, const int32_t *code, uint16_t sb, float step) {
  double *out = (double *)ctx + t * (uint64_t)q->tl;
  float m[2], tf[2];
  tile_factors(q->lattice, bf16_to_f32(sb), step, m, tf);
  for (int o = 0; o < q->tl / 8; ++o) {
    float u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (q->dither) hqo_dither_octet_flags(q->seed, t, o, q->lattice, q->dither, u);
    for (int i = 0; i < 8; ++i) {
      const double c = (double)code_to_coord(q->lattice, code[8 * o + i]);
      out[8 * o + i] = (c - (double)u[i]) * (double)tf[i & 1];
    }
  }
}

int hqo_decode_coords(const uint8_t *s, uint64_t bytes, uint64_t n, double *yhat) {
  return read_stream(s, bytes, n, coords_sink, yhat);
}
