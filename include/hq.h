/*
 * hq.h -- C ABI of the MI355X (gfx950) RHT + lattice + bit-strip + Rice codec.
 *
 * The method is the per-tile pipeline of the HyperQuant technical summary
 * (gist.science/ko/paper/2606.23406; Japanese version gist.science/ja/paper/2606.23406), section
 * "Methodology: the HyperQuant pipeline":
 *   component 1  per-tile randomized Hadamard transform RHT_n(x) = H_n D x (D: random +-1), on
 *                tiles of n = 128 values (the summary's example size), or of 64 or 256,
 *   component 2  nearest-point quantisation onto E8 (or D4, A2, or scalar Z) in an integer
 *                embedding, scaled so the rotated tile matches the lattice,
 *   component 3  stripping of the bits that lattice membership fixes, then Rice coding, with the
 *                realised rate within ~0.01 bits per value of the target,
 *   component 4  for KV caches: a per-layer +-1 rotation (folded into D through the seed) and a
 *                subtractive dither U ~ Uniform(V(lattice)) added before and removed after.
 *
 * Conventions of every entry point:
 *  - Pointers named x, out, stream, workspace are DEVICE pointers (HIP global memory of the current
 *    device); `params`, `info`, `out_bytes` are HOST pointers.  `stream` arguments of type
 *    hq_stream_t are hipStream_t values (0 = the null stream).
 *  - The caller owns every buffer.  The library allocates no device memory and keeps no state
 *    between calls apart from immutable constants and a counter that numbers calls (a workspace
 *    reports the errors recorded under the number of its last call, so nothing has to be cleared
 *    before a call); one workspace serves one call in flight.
 *  - Tensors are flat arrays of n values, n a multiple of the tile length TL (64, 128 or 256; 128
 *    by default); tile t is values [TL t, TL t + TL).
 *  - Every call returns HQ_OK (0) or a negative hq_status code; no exception crosses the ABI.
 *  - Errors found on the device (non-finite input, too small an output buffer, corrupt stream) are
 *    recorded in the workspace; blocking calls return them, hq_status() reads them otherwise.
 *
 * Bitstream (format version 1, little-endian; the pages give no format, this is the codec's own):
 *   header, 128 bytes: u32 magic 'HQ01' | u16 version | u8 lattice | u8 dither flags |
 *     u16 tile TL | u8 rice k | u8 log2 tiles per chunk (log2(8192 / TL)) | u32 step (binary32 bits) |
 *     u64 seed | u64 n | u64 tiles | u32 chunks | u32 F (fixed bits per tile) | u64 fixed_off |
 *     u64 unary_off | u64 unary_words | u64 unary_bits | u64 payload_bits | u64 total_bytes | 32 B 0
 *   chunk index at byte 128: chunks+1 u32 offsets, in 64-bit words, into the unary plane; a chunk
 *     is 8192 values (8192 / TL tiles)
 *   fixed plane at fixed_off = align256(128 + 4 (chunks+1)); chunk c = its tiles' records;
 *     tile record at bit t F (bit i of a plane = bit i%8 of byte i/8): bf16 tile scale (16) |
 *     coset bits (E8: octet o at bit o, TL/8 bits; A2: pair j of octet o at bit 4o+j, TL/2 bits;
 *     none for D4 and Z) | octet 0..TL/8-1, slot 0..7: Rice remainder, width k (full slots) or
 *     max(k-1,0) (halved slots: the parity-fixed slot 7 of E8, 3 and 7 of D4; the stretched odd
 *     slots of A2), LSB first
 *   unary plane at unary_off = align256(fixed_off + chunks (8192 / TL) F / 8): chunk c's segment
 *     starts at word index[c]; each symbol in (tile, octet, slot) order contributes
 *     (symbol >> width) zero bits and a one; segments are zero-padded to 64 bits.
 *   Symbols per octet (8 consecutive coordinates): E8: z in 2E8, p = z0 & 1, u = (z-p)/2,
 *     slots zz(u0..u6), zz((u7 - (u0+..+u6 & 1))/2); D4 (two blocks): zz(x0..x2),
 *     zz((x3 - (x0+x1+x2 & 1))/2); A2 (four pairs, stretched coordinates, z = 2c with
 *     z_2j = z_2j+1 mod 2): p_j = z_2j & 1, slots zz((z_2j - p_j)/2), zz((z_2j+1 - p_j)/2);
 *     Z: zz(z0..z7); zz(a) = (a << 1) ^ (a >> 31).
 *   A2 is the hexagonal lattice with minimal distance 1; each pair (v0, v1) is quantised as
 *     (v0, v1 / sqrt 3) onto Z^2 u (Z+1/2)^2 under the distance dw0^2 + 3 dw1^2: its odd slots use
 *     the multiplier 1 / ((s step) R) and reconstruct with (s step) R, R = binary32 sqrt 3.
 *   Dither flags (0: no dither): bit 0 dither on; bit 1 the dither's Philox4x32 calls take 7 rounds
 *     instead of 10; bit 2 a 24-bit draw instead of 16 bits (valid: 0, 1, 3, 5, 7).  Octet o of
 *     tile t draws b in [0, 2)^8 from Philox with key = seed and counter (o, t lo, t hi, 1): the
 *     eight 16-bit halves (low first) / 2^15; with 24 bits, words w0..w3 of that call and w4..w7
 *     of counter (o, t lo, t hi, 2) give (w_i >> 8) / 2^23.  U = b - Q(b), Q the lattice's
 *     nearest point: uniform on the Voronoi cell to the draw's resolution.  The pages fix neither
 *     the round count nor the resolution; 10 rounds and 16 bits are the defaults.
 */
#ifndef HQ_H_
#define HQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *hq_stream_t; /* a hipStream_t */

typedef enum {
  HQ_OK = 0,
  HQ_ERR_INVALID_ARG = -1, /* null pointer, bad enum, n % TL != 0, n > 2^35, step outside 2^+-12  */
  HQ_ERR_UNSUPPORTED = -2, /* tile size other than 64, 128, 256; or a unary plane of 2^32 words+     */
  HQ_ERR_NONFINITE = -3,   /* a tile whose transformed energy is NaN or Inf                         */
  HQ_ERR_CAPACITY = -4,    /* output buffer too small; *out_bytes holds the size needed            */
  HQ_ERR_CORRUPT = -5,     /* stream fails validation (header, index, segment, terminator count)   */
  HQ_ERR_RATE = -6,        /* target outside [1.125 (E8), 1.5 (A2) or 1.0 (D4, Z), 12] bits / value */
  HQ_ERR_HIP = -7,         /* a HIP runtime call failed                                             */
  HQ_ERR_TIMEOUT = -8,     /* reserved: no longer produced (every cross-workgroup wait now ends)   */
  HQ_ERR_SCRATCH = -9      /* hq_encode_noalloc: n above its static workspace's maximum (2^30 values) */
} hq_status_code;

typedef enum { HQ_Z = 0, HQ_D4 = 1, HQ_E8 = 2, HQ_A2 = 3 } hq_lattice;
typedef enum { HQ_F32 = 0, HQ_BF16 = 1 } hq_dtype;

typedef struct {
  uint32_t tile;       /* values per tile: 64, 128 or 256 (component 1: "tiles, e.g. 128")         */
  int32_t lattice;     /* hq_lattice                                                                */
  float target_bps;    /* payload bits per value (coset + Rice bits / n); used when step == 0       */
  uint64_t seed;       /* Philox key of the sign diagonal D and of the dither                        */
  uint32_t dither;     /* dither flags: 0 off; 1 subtractive dither (component 4); + 2: 7-round     */
                       /* Philox for the draw; + 4: 24-bit draw (3, 5, 7; see the format above)     */
  float step;          /* 0 = choose by rate control; > 0 = fixed lattice step (KV append, tests);
                          -1 (hq_encode only) = the step and k the workspace holds: those that a
                          preceding hq_rate or hq_encode on the same workspace chose            */
  int32_t rice_k;      /* -1 = automatic; 0..15 = fixed Rice parameter                              */
} hq_params;

typedef struct {
  float step;           /* lattice step used                                                         */
  int32_t rice_k;       /* Rice parameter used                                                       */
  uint64_t bytes;       /* stream size                                                              */
  uint64_t payload_bits;/* coset + remainder + unary bits                                            */
  double payload_bps;   /* payload_bits / n: the rate that rate control targets                     */
  double side_bps;      /* (tile scales + header + index + padding) bits / n                          */
  double total_bps;     /* 8 bytes / n                                                              */
} hq_info;

/* Library and format version: returns (major << 16) | format_version.
 * Defined by this codec (the pages give no format); the format is the one described above. */
uint32_t hq_version(void);

/* Human-readable text of a status code (static storage).  Host only; no device call. */
const char *hq_strerror(int code);

/* Bytes of device workspace that hq_encode / hq_rate / hq_decode / hq_codes need for n values
 * (host only; no device call).  The workspace needs no initialisation.
 * The workspace holds the state of components 1-3 of "Methodology: the HyperQuant pipeline"
 * across the kernels of one call: the operating point that rate targeting (component 3) picks, its
 * sample counters, and the encoder's per-chunk offset flags.  HQ_ERR_INVALID_ARG: bytes == NULL or
 * n not a multiple of 64. */
int hq_workspace_size(uint64_t n, const hq_params *params, size_t *bytes);

/* Stream size for n values at a fixed step, Rice k and tile length, without the unary plane (host
 * only): the header, index and fixed plane.  The unary plane adds (symbol >> width) + 1 bits per value,
 * which depends on the data (hq_encode_bound bounds it).  Component 3 of "Methodology: the
 * HyperQuant pipeline" (Rice codes: a fixed-width remainder per symbol).  HQ_ERR_INVALID_ARG for a
 * bad lattice or k, or n % tile != 0; HQ_ERR_UNSUPPORTED for another tile length. */
int hq_stream_fixed_bytes(uint64_t n, int32_t lattice, int32_t rice_k, uint32_t tile, uint64_t *bytes);

/* Worst-case stream size in bytes for n values encoded with `params` (host only; no device call),
 * so that a caller can size the output of an asynchronous hq_encode, or of a KV-cache append at a
 * fixed operating point, before the data exist.  Component 3 of "Methodology: the HyperQuant
 * pipeline" codes lattice symbols with Rice codes and no overload region (the codebook is
 * unbounded), so the size is bounded only through the energy normalisation of component 2: each
 * tile's scale s (the bf16 RMS of its transformed values, 16 bits) makes the lattice inputs w of a
 * tile satisfy sum w^2 <= TL K^2 / step^2, K = 1 + 2^-7 (the bf16 rounding of s and the binary32
 * roundings).  By Cauchy-Schwarz, sum |w| <= TL K / step; a lattice point lies within the covering
 * radius of its input (and the dither of component 4 within the Voronoi cell), and a Rice unary
 * part of a symbol of magnitude u with parameter k is at most u / 2^k + 1 bits.  Summed per tile:
 *   unary bits <= TL + (A TL K / step + (TL / 8) B) / 2^k,
 * A = 2 (E8, D4, Z) or sqrt(14/3) (A2), B per octet: E8 2 sqrt 8 d + 12, D4 8 d + 8, Z 8 d,
 * A2 (4 sqrt 28 / 3) d + 12, where d = 1 without dither and 2 with it; then the stream layout
 * (header, index, fixed plane, 64-bit padding per chunk).  params->step > 0 is used as given;
 * step == 0 or -1 (the step is chosen later) takes the smallest step of the range, 2^-12;
 * params->rice_k == -1 takes the largest bound over k = 0..15.  target_bps and seed play no part.
 * The bound holds for every input whose tiles are each all zero or hold a value of magnitude at
 * least 2^-60 (it then covers the binary32 rounding of the tile energy; a tile whose values all lie
 * below 2^-60 in magnitude can round its energy down and exceed it).  An encode whose stream would
 * exceed the buffer is never written past it: hq_encode then reports HQ_ERR_CAPACITY.
 * HQ_ERR_INVALID_ARG for a null pointer, a bad lattice, dither flags or k, n % tile != 0,
 * n > 2^35 or a step outside [2^-12, 2^12]; HQ_ERR_UNSUPPORTED for another tile length. */
int hq_encode_bound(uint64_t n, const hq_params *params, uint64_t *max_bytes);

/* Rate control alone: component 3 of "Methodology: the HyperQuant pipeline" (rate targeting, the
 * realised rate within ~0.01 bits per value of the target).  Chooses the lattice step and Rice
 * parameter for x so that the payload rate of a jittered stratified sample of min(T, 8192) tiles
 * meets params->target_bps (a coarse pass on min(T, 2048) tiles first).  With info != NULL the call
 * blocks and fills info (payload_bps is the target); with info == NULL it only enqueues work, and a
 * following hq_encode with params->step == -1 on the same workspace and stream encodes at the chosen
 * point (the pair then does exactly what one hq_encode with rate control does).  x must be 16-byte
 * aligned and the workspace 256-byte aligned (HQ_ERR_INVALID_ARG otherwise), as for hq_encode.
 * Errors: HQ_ERR_INVALID_ARG (null or misaligned pointers, bad params, step == -1, a workspace
 * smaller than hq_workspace_size), HQ_ERR_RATE (target outside the lattice's range),
 * HQ_ERR_UNSUPPORTED (tile length); device-side HQ_ERR_NONFINITE / HQ_ERR_TIMEOUT when blocking. */
int hq_rate(const void *x, int32_t dtype, uint64_t n, const hq_params *params, hq_info *info,
            void *workspace, size_t workspace_bytes, hq_stream_t stream);

/* Encode x (n values, dtype hq_dtype) into `out` (device, out_capacity bytes): components 1-4 of
 * "Methodology: the HyperQuant pipeline" (per-tile RHT H D x; nearest point of the scaled lattice;
 * stripping of the bits lattice membership fixes and Rice coding; the subtractive dither of the KV
 * path when params->dither is set).
 * With out_bytes != NULL the call blocks, stores the stream size in *out_bytes (also when the
 * result is HQ_ERR_CAPACITY: the size needed) and fills *info (may be NULL).  With out_bytes == NULL
 * the call only enqueues work on `stream`; the size is in the stream header (total_bytes) and
 * device-side errors are returned later by hq_status(workspace).  Rate control runs when
 * params->step == 0; step > 0 fixes the step; step == -1 takes the operating point that the
 * workspace holds: the one a preceding hq_rate, or a preceding hq_encode with step >= 0, chose on
 * it (repeated step == -1 calls, e.g. appends to a KV cache at one operating point, keep using
 * it).  Every call resets the workspace's status, results and offset flags first; an encode with
 * step == -1 on a workspace that holds no operating point reports HQ_ERR_INVALID_ARG (blocking) or
 * through hq_status.  x, out: 16-byte aligned; workspace: 256-byte aligned, at least
 * hq_workspace_size(n) bytes.  Errors: as hq_rate, plus HQ_ERR_CAPACITY (out too small; nothing
 * is written past out_capacity) and HQ_ERR_UNSUPPORTED (a unary plane of 2^32 words or more). */
int hq_encode(const void *x, int32_t dtype, uint64_t n, const hq_params *params, void *out,
              uint64_t out_capacity, uint64_t *out_bytes, hq_info *info, void *workspace,
              size_t workspace_bytes, hq_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): hq_encode without a workspace argument.  The workspace
 * is a static device array of the library, 1,065,472 bytes on each GPU the library runs on, held
 * until the process ends; it serves n up to 2^30 values (HQ_ERR_SCRATCH above that).  The call
 * allocates nothing.  Arguments, results and errors are those of hq_encode with the same params
 * (the same kernels, the same stream bytes); step == -1 takes the operating point of the previous
 * hq_encode_noalloc on this GPU.  Every call on a GPU shares that GPU's array: each call resets its
 * status, results and offset flags first, and calls that overlap on one GPU (other streams, other
 * host threads) race and may corrupt each other's streams.  With out_bytes == NULL the call only
 * enqueues work; its device-side errors then have no workspace to be read from (the stream
 * header's total_bytes still gives the size, and a stream is complete when that is at most
 * out_capacity), so callers that must learn of non-finite input use the blocking form. */
int hq_encode_noalloc(const void *x, int32_t dtype, uint64_t n, const hq_params *params, void *out,
                      uint64_t out_capacity, uint64_t *out_bytes, hq_info *info, hq_stream_t stream);

/* Decode a stream of `stream_bytes` bytes into out (n values of out_dtype; bf16 is round to nearest
 * even of the fp32 reconstruction): the exact inverse of components 1-4 of "Methodology: the
 * HyperQuant pipeline" (Rice and unstrip are lossless; yhat = (c - U) s step; x = D H yhat / TL,
 * the transform being orthogonal up to the factor TL).  Asynchronous: header and per-chunk
 * validation happen on the device; call hq_status(workspace) to learn of HQ_ERR_CORRUPT.  On a
 * corrupt stream the output contents are unspecified, but no access leaves the given buffers.
 * out: n values, 16-byte aligned; stream_data 16-byte aligned; workspace 256-byte aligned, at least
 * hq_workspace_size(0) bytes.  HQ_ERR_INVALID_ARG on the host for bad pointers, dtype or n. */
int hq_decode(const void *stream_data, uint64_t stream_bytes, void *out, int32_t out_dtype,
              uint64_t n, void *workspace, size_t workspace_bytes, hq_stream_t stream);

/* Waits for `stream` and returns the first device-side error recorded in `workspace` since the last
 * hq_encode / hq_decode / hq_rate / hq_codes / hq_gemv that used it (HQ_OK when none).  Reports
 * the device-side outcome of the calls above (no step of the method of its own). */
int hq_status(void *workspace, hq_stream_t stream);

/* Diagnostic of the last call that used `workspace` (waits for `stream`): which of its bounded
 * cross-workgroup waits ran out of their spin budget and computed the awaited value themselves.
 * No passage of the pages defines these waits: they are this codec's way of running rate targeting
 * (component 3 of "Methodology: the HyperQuant pipeline") and the stream's chunk offsets in single
 * launches.  A fallback gives the same result as the normal path, only later (microseconds to
 * milliseconds), so the flags concern speed, never correctness.  *flags receives bit 0: a
 * look-back computed a predecessor chunk's offset contribution from its input; bit 1: a rate
 * workgroup solved pass A itself instead of waiting for its published centre; bit 2: a rate
 * solver evaluated a pass's whole sample itself.  Errors: HQ_ERR_INVALID_ARG (null pointer),
 * HQ_ERR_HIP. */
int hq_fallbacks(const void *workspace, hq_stream_t stream, uint32_t *flags);

/* Workspace bytes for hq_gemv on a [rows][cols] matrix (host only; enough for any tile length).
 * Holds the rotated activation and the per-tile partial products of the fused product below. */
int hq_gemv_workspace_size(uint64_t rows, uint64_t cols, size_t *bytes);

/* Fused decode + matrix-vector product y = W_hat x, where the stream encodes a row-major
 * [rows][cols] matrix (n = rows * cols; tiles of TL values along cols, so cols % TL == 0) and W_hat
 * is the decoder's reconstruction taken in exact arithmetic.  x: cols values of x_dtype (device),
 * y: rows binary32 values (device).  Since tile (r, j) decodes to D H yhat / TL (component 1's
 * transform is orthogonal up to the factor TL and H is symmetric), its contribution is
 * <yhat, H D x_j> / TL: the activation is rotated once per column tile (binary32, the encoder's
 * butterfly order) and no matrix tile is inverse-transformed.  Per tile, yhat = (c - U) * s * step
 * rounded to binary32, the octet products are a fixed-order chain, the tile sum a fixed tree, and
 * the row sum adds the tiles in column order, so results are deterministic; they differ from an
 * exact product by rounding only (relative to sum |yhat| |x~|, a few hundred units of 2^-24).
 * Components 1-3 of the HyperQuant technical summary (section "Methodology: the HyperQuant
 * pipeline"); fused decode + matrix products are the direction its section "Significance and
 * claims" names for a wall-clock gain.  Asynchronous;
 * stream validation as for hq_decode (a stream whose tile length does not divide cols is corrupt
 * for this call), errors through hq_status(workspace). */
int hq_gemv(const void *stream_data, uint64_t stream_bytes, uint64_t rows, uint64_t cols, const void *x,
            int32_t x_dtype, float *y, void *workspace, size_t workspace_bytes, hq_stream_t stream);

/* The per-layer Haar-uniform rotation of a seed (component 4 of "Methodology: the HyperQuant
 * pipeline": the full-matrix alternative to the +-1 sign diagonal), written to q (HOST pointer, 128 * 128 floats, q[128 i + j] = Q[i][j]).
 * Construction (the pages give none; the textbook one): G with independent N(0,1) entries, entry
 * e = 128 i + j from Philox4x32-10 with key = seed and counter (e / 4, 0, 0, 2), two Box-Muller
 * pairs per call (u(w) = (w + 1/2) 2^-32; r = sqrt(-2 ln u(w0)); (r cos 2pi u(w1), r sin 2pi u(w1)),
 * then (w2, w3)); G = Q R with diag(R) > 0, computed in binary64 and rounded to binary32.
 * Host only, deterministic. */
int hq_haar_matrix(uint64_t seed, float *q);

/* y_v = Q x_v (transpose = 0; the rotation before hq_encode) or Q^T x_v (transpose = 1; after
 * hq_decode) for every 128-value vector v of x.  x, y: DEVICE, n bf16 values each (n % 128 == 0),
 * 16-byte aligned, may not overlap; q: DEVICE, 128 * 128 binary32 as from hq_haar_matrix.
 * On MFMA (bf16 inputs, Q split into two bf16 parts, binary32 accumulation); y is rounded to bf16
 * (nearest even).  Asynchronous on `stream`.  Component 4 of "Methodology: the HyperQuant
 * pipeline" (the per-layer rotation of the KV path, applied before the codec and undone after).
 * HQ_ERR_INVALID_ARG for null or misaligned pointers or n % 128 != 0. */
int hq_rotate(const void *x, uint64_t n, const float *q, int32_t transpose, void *y, hq_stream_t stream);

/* ---------------------------------------------------------------------------------------------
 * SRFT fixed-rate KV codec ("When quantization is free" technical summary,
 * gist.science/ko/paper/2605.05699, section "Methodology" 1-3): per 128-value vector,
 * v = pack(F diag(s) x) / lambda with F the unitary DFT, s the sign diagonal of `seed` (the same
 * signs as the lattice codec's D), pack the orthogonal real form (X_0, X_64, sqrt 2 Re X_1,
 * sqrt 2 Im X_1, ...), lambda a per-coordinate calibration scale; then 16 groups of 8 coordinates,
 * scale Delta = binary16(absmax / L) (L = 7 for int4, 127 for int8; nearest even, saturating at
 * 65504) and codes q = clamp(rint(v * (1 / Delta)), -L, L).  Fixed rate: 4 (or 8) bits per value
 * plus 16 binary16 scales per vector (96 bytes per vector at int4, 2.67x smaller than bf16).
 *
 * codes: DEVICE, n / 2 bytes (bits = 4: codes 2j and 2j + 1 of a vector in the low and high nibble
 * of its byte j, two's complement) or n bytes (bits = 8, int8); scales: DEVICE, n / 128 * 16
 * binary16 values (vector-major).  x / out: DEVICE, n values of `dtype` / `out_dtype` (HQ_F32 or
 * HQ_BF16), n % 128 == 0.  All device pointers 16-byte aligned.  lambda: HOST, 128 binary32 values,
 * each finite and > 0 (HQ_ERR_INVALID_ARG otherwise), or NULL for all ones; encoder and decoder
 * must be given the same lambda and seed.  A vector whose packed coordinates are not all finite is
 * stored with zero codes and NaN (0x7E00) scales and decodes to NaN.  Decode outputs bf16 rounded
 * to nearest even (or binary32), exact zeros as +0.  Both calls are asynchronous on `stream`, use
 * no workspace and allocate nothing. */
int hq_srft_encode(const void *x, int32_t dtype, uint64_t n, uint64_t seed, const float *lambda, int32_t bits,
                   void *codes, void *scales, hq_stream_t stream);
int hq_srft_decode(const void *codes, const void *scales, uint64_t n, uint64_t seed, const float *lambda,
                   int32_t bits, void *out, int32_t out_dtype, hq_stream_t stream);

/* Diagnostic front half of the encoder at a fixed step (components 1 and 2 of "Methodology: the
 * HyperQuant pipeline", with component 4's dither when params->dither is set; the integer codes
 * before component 3's stripping): per-value integer lattice codes (int32;
 * E8 and A2 codes are twice the lattice point (A2 in stretched coordinates), D4 and Z codes are the
 * point) and per-tile bf16 scale bits (uint16).  codes: n values, scales: n / params->tile
 * values, both device buffers, 16-byte aligned.  params->step must be positive (a fixed step);
 * the dither flags apply as for hq_encode.  Asynchronous; non-finite tiles are reported through
 * hq_status.  HQ_ERR_INVALID_ARG for step <= 0, bad params or misaligned pointers. */
int hq_codes(const void *x, int32_t dtype, uint64_t n, const hq_params *params, int32_t *codes,
             uint16_t *scales, void *workspace, size_t workspace_bytes, hq_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HQ_H_ */
