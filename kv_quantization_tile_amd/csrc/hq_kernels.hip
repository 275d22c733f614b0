// hq_kernels.hip -- gfx950 kernels of the RHT + lattice + bit-strip + Rice codec.
//
// Method: HyperQuant technical summary (gist.science/ko/paper/2606.23406), "Methodology: the
// HyperQuant pipeline", components 1-4 (per-tile RHT, lattice quantisation, bit-stripping + Rice
// coding with rate targeting, KV dither).  The byte format is described in include/hq.h.
//
// Kernels of one encode call, all on the caller's stream, with no host round trip in between:
//   init_kernel     clears the workspace flags and counters and seeds the rate search;
//   rate_kernel     the rate search in one launch: its first workgroups evaluate pass A's 8
//                   candidate steps (quarter octaves) on samples of tiles into counters, and
//                   workgroup 0 solves pass A for pass B's centre and publishes it; the workgroups
//                   after them evaluate pass B's 4 candidates (1/16 octave) around that centre, and
//                   the one that completes the last counter set solves pass B for the operating
//                   point;
//   encode_kernel   one workgroup per 8192-value chunk: load, sign, FWHT, scale, lattice, strip,
//                   Rice lengths, workgroup scan, decoupled look-back over chunks for the unary
//                   offsets, and coalesced stores of the chunk's fixed record and unary segment.
// Decode: decode_kernel, one workgroup per chunk, each checking the stream header itself.  The
// fused product: gemv_rotate_kernel (the activation, and the header check), decode_kernel with the
// product in place of the inverse transform, gemv_rows_kernel; decode_check_kernel checks the
// header of an empty product's stream.
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {

constexpr int kFixedWordsMax = 3904;      // 2 F u32 words per chunk; F <= 1952 bits
constexpr int kUnaryWinWords = 768;       // 3 KiB unary staging window = 24576 bits (segments of
                                          // chunks longer than that are written in several windows)
constexpr uint32_t kUnaryWinBits = kUnaryWinWords * 32u;
constexpr uint64_t kFlagAgg = 1ull << 62, kFlagPrefix = 2ull << 62, kValMask = (1ull << 62) - 1;

__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

__device__ __forceinline__ uint32_t low_mask(int w) { return w >= 32 ? 0xFFFFFFFFu : ((1u << w) - 1u); }

// OR `nbits` (<= 32 - 0, value < 2^nbits, nbits <= 16 here) bits into an LDS bit array.
__device__ __forceinline__ void lds_put_bits(uint32_t* s, uint32_t pos, uint32_t val, int nbits) {
  if (nbits == 0 || val == 0) return;
  const uint32_t word = pos >> 5, sh = pos & 31u;
  atomicOr(&s[word], val << sh);
  if (sh + (uint32_t)nbits > 32u) atomicOr(&s[word + 1], val >> (32u - sh));
}

__device__ __forceinline__ uint32_t lds_get_bits(const uint32_t* s, uint32_t pos, int nbits) {
  if (nbits == 0) return 0;
  const uint32_t word = pos >> 5, sh = pos & 31u;
  uint64_t v = s[word];
  if (sh + (uint32_t)nbits > 32u) v |= (uint64_t)s[word + 1] << 32;
  return (uint32_t)(v >> sh) & low_mask(nbits);
}

// Remainder field of one octet in the low RW bits of (lo, hi), slot 0 lowest (least significant
// bit first).  Each slot's low w bits enter at the top of a right-shifting accumulator through one
// funnel shift (alignbit), which also drops the symbol's bits above w; a final shift moves the
// field down.  k is the same in every lane, so the branch is uniform.  Fields up to 64 bits
// (Rice k <= 8).
template <int LAT>
__device__ __forceinline__ void pack_octet_remainders(const uint32_t* sym, int k, uint32_t* lo, uint32_t* hi) {
  const int RW = octet_rem_bits<LAT>(k);
  uint32_t l = 0, h = 0;
  if (RW <= 32) {
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) l = __builtin_amdgcn_alignbit(sym[sl], l, (uint32_t)slot_width<LAT>(sl, k));
    *lo = __builtin_amdgcn_alignbit(0u, l, (uint32_t)(32 - RW));  // shift 32 is 0: RW = 0 leaves l = 0
    *hi = 0u;
  } else {
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const uint32_t w = (uint32_t)slot_width<LAT>(sl, k);
      l = __builtin_amdgcn_alignbit(h, l, w);
      h = __builtin_amdgcn_alignbit(sym[sl], h, w);
    }
    const uint32_t sh = (uint32_t)(64 - RW);  // 1..31
    *lo = __builtin_amdgcn_alignbit(h, l, sh);
    *hi = h >> sh;
  }
}

// OR a field of at most 64 bits (lo, hi) into an LDS bit array at bit position pos.
__device__ __forceinline__ void lds_put_field64(uint32_t* s, uint32_t pos, uint32_t lo, uint32_t hi) {
  const uint32_t word = pos >> 5, sh = pos & 31u;
  const uint32_t w0 = lo << sh;
  const uint32_t w1 = sh ? ((lo >> (32u - sh)) | (hi << sh)) : hi;
  const uint32_t w2 = sh ? (hi >> (32u - sh)) : 0u;
  atomicOr(&s[word], w0);
  atomicOr(&s[word + 1], w1);
  if (w2) atomicOr(&s[word + 2], w2);
}

// Sample tile of stratum i (jittered stratified sampling, see rate control below).
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x = x * 0x9E3779B1u + 0x7F4A7C15u;
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}
// N is min(T, the pass's sample size), a power of two whenever N < T: then the divisions are
// shifts; the stratum width hi - lo is below 2^32, so the pick is a 32-bit remainder.
__device__ __forceinline__ uint64_t sample_tile(uint64_t i, uint64_t T, uint64_t N) {
  uint64_t lo, hi;
  if (N < T && (N & (N - 1)) == 0) {
    const uint32_t sh = (uint32_t)__builtin_ctzll(N);
    lo = (i * T) >> sh;
    hi = ((i + 1) * T) >> sh;
  } else {
    lo = (i * T) / N;
    hi = ((i + 1) * T) / N;
  }
  return lo + (uint64_t)(mix32((uint32_t)i) % (uint32_t)(hi - lo));
}

__host__ __device__ inline int kwin_base(int64_t b) {
  const int e = (int)((b >> 23) & 0xFF) - 127;
  int kb = -e - 2;
  kb = kb < 0 ? 0 : kb;
  return kb > 12 ? 12 : kb;
}

__device__ __forceinline__ int64_t clamp_i64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Records error flags of call `call` in the workspace (see Workspace::err): every writer of a flag
// stores the same value, so plain relaxed stores suffice and nothing needs clearing first.
__device__ __forceinline__ void record_error(Workspace* ws, uint64_t call, uint32_t flags) {
#pragma unroll
  for (int b = 0; b < 8; ++b)
    if ((flags >> b) & 1u) __hip_atomic_store(&ws->err[b], call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Marks that `call` took fallback `kind` (a wait that ran out of its budget; see Workspace::slow).
__device__ __forceinline__ void record_fallback(Workspace* ws, uint64_t call, int kind) {
  __hip_atomic_store(&ws->slow[kind], call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane layout of a tile length TL: LPT lanes per tile, TPW tiles per wavefront, TPR tiles per
// workgroup round, CT tiles per chunk (four rounds, kChunkValues values).
template <int TL>
struct Tiling {
  static_assert(TL == 64 || TL == 128 || TL == 256, "tile length");
  static constexpr int LPT = TL / 8;
  static constexpr int TPW = 64 / LPT;
  static constexpr int TPR = 4 * TPW;
  static constexpr int CT = kChunkValues / TL;
  static_assert(CT == 4 * TPR, "four rounds per chunk");
};

// ---------------------------------------------------------------------------------------------
// Front half shared by the rate, encode and codes kernels: sign, FWHT, tile energy and scale.
// Returns the scale bits; y holds the transformed values (zeroed when the energy is not finite).
template <int DT, int TL>
__device__ __forceinline__ uint32_t transform_octet(const void* x, uint64_t t, bool valid, int o,
                                                     uint32_t sgn, float* y, bool* finite) {
  constexpr int LPT = Tiling<TL>::LPT;
  if (valid) {
    load_octet<DT, TL>(x, t, o, y);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = ((sgn >> i) & 1u) ? -y[i] : y[i];
  fwht_lane(y);
  fwht_cross<LPT>(y, o);
  float S = tile_sumsq<LPT>(y);
  *finite = isfinite(S);
  if (!*finite) {
    S = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.0f;
  }
  return tile_scale_bits<TL>(S);
}

// Per-tile multiplier m = 1 / (s * step) (0 when s = 0), with the lane's sign folded in.  A2's
// odd slots use m' = 1 / ((s * step) * sqrt3) instead (each product and quotient rounded once),
// which takes the pair's second coordinate into the lattice's stretched coordinates.
template <bool ODD>
__device__ __forceinline__ float tile_multiplier(uint32_t sb, float step, uint32_t lane_neg) {
  const float s = bf16_bits_to_f32(sb);
  const float t = ODD ? (s * step) * __uint_as_float(kA2R3Bits) : s * step;
  const float m0 = (s != 0.0f) ? __fdiv_rn(1.0f, t) : 0.0f;
  return lane_neg ? -m0 : m0;
}
__device__ __forceinline__ float tile_multiplier(uint32_t sb, float step, uint32_t lane_neg) {
  return tile_multiplier<false>(sb, step, lane_neg);
}

// v = y * m (+ U); m as above (A2: m' on odd slots); nearest lattice point.
// y holds sigma(lane) times the transformed values (see fwht_cross); the sign is folded into m.
template <int LAT, bool DITHER>
__device__ __forceinline__ void quantize_octet(const float* y, uint32_t sb, float step, const float* u,
                                               int32_t* code, uint32_t lane_neg) {
  const float m = tile_multiplier<false>(sb, step, lane_neg);
  const float m1 = LAT == kLatA2 ? tile_multiplier<true>(sb, step, lane_neg) : m;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = y[i] * ((i & 1) ? m1 : m);
    if (DITHER) v[i] = v[i] + u[i];
  }
  nearest_octet<LAT>(v, code);
}

// Symbols of one octet at multipliers m (even slots) and m1 (odd slots; equal to m except for A2),
// the lane's sign already folded in: v = y * m (+ U), nearest lattice point, bit-stripping.
template <int LAT, bool DITHER, bool MASK_FIX = false>
__device__ __forceinline__ void octet_symbols(const float* y, float m, float m1, const float* u, uint32_t* sym,
                                              uint32_t* coset) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = y[i] * ((i & 1) ? m1 : m);
    if (DITHER) v[i] = v[i] + u[i];
  }
  if (LAT == kLatE8) {
    e8_symbols<MASK_FIX>(v, sym, coset);
  } else {
    int32_t code[8];
    nearest_octet<LAT>(v, code);
    strip_octet<LAT>(code, sym, coset);
  }
}

// ---------------------------------------------------------------------------------------------
// Resets a call's workspace: results, the look-back flags and the rate counters, and numbers the
// workspace with the call (its errors are then those recorded under that number).
// mode kInitProvisional / kInitFinal: the operating point becomes (step_bits, k), and the point tag
// says whether it is complete (kInitFinal) or awaits rate passes (their last solve sets the tag).
// mode kInitKeep (an encode with step == -1): the operating point already in the workspace is
// kept; without a valid tag, or with a step or k out of range, the call records kErrNoPoint and
// the encoder runs at a harmless point (step 1, k 0) so that every access stays in bounds.
__global__ void init_kernel(Workspace* ws, uint64_t* flags, uint64_t nflags, uint32_t* acc, uint32_t nacc,
                            int64_t centre, uint32_t step_bits, int32_t k, int mode, uint64_t call) {
  const uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid == 0) {
    uint32_t status = 0;
    if (mode == kInitKeep) {
      step_bits = ws->step_bits;
      k = ws->rice_k;
      if (ws->point_tag != kPointTag || step_bits < kStepBitsMin || step_bits > kStepBitsMax || k < 0 || k > 15) {
        status = kErrNoPoint;
        step_bits = 127u << 23;
        k = 0;
        ws->point_tag = 0;
      }
    } else {
      ws->point_tag = mode == kInitFinal ? kPointTag : 0u;
      ws->rc_centre = centre;
    }
    ws->call = call;
    if (status) record_error(ws, call, status);
    ws->step_bits = step_bits;
    ws->rice_k = k;
    ws->res_total_bytes = 0;
    ws->res_payload_bits = 0;
    ws->res_unary_bits = 0;
    ws->res_words = 0;
    ws->res_step_bits = step_bits;
    ws->res_k = k;
  }
  for (uint64_t i = gid; i < nflags; i += (uint64_t)gridDim.x * blockDim.x) flags[i] = 0;
  for (uint64_t i = gid; i < nacc; i += (uint64_t)gridDim.x * blockDim.x) acc[i] = 0;
}

// ---------------------------------------------------------------------------------------------
// Rate control.  The pages fix only the outcome (realised rate within ~0.01 bits per value); the
// search is this codec's reading:
//  - sample: N = min(T, 2048) tiles for pass A, min(T, 8192) for pass B, one per stratum
//    [floor(iT/N), floor((i+1)T/N)), picked by a 32-bit hash of i;
//  - the search variable is b, the binary32 bit pattern of the step;
//  - a pass evaluates nc candidates centre + (2j-(nc-1)) 2^h (clamped to [2^-12, 2^12]); for
//    each, the Rice k is the argmin (ties: smaller k) over kb..kb+3, kb = clamp(-exponent - 2, 0, 12);
//  - the solve interpolates linearly (IEEE double) between the two candidates that
//    bracket the target bit count (first candidate at or below it) or extrapolates from the end
//    pair, rounds, clamps, and stores the answer as the next centre together with the k of the
//    candidate nearest to it.  Pass A (8 candidates, h = 21: quarter octaves) starts at
//    2.05 - target octaves; pass B (4 candidates, h = 18: 1/16 octave) refines.  With a fixed step
//    and automatic k one pass (8192 tiles) with the single candidate picks k.
// Bits of candidate j over the Rice window (lane j of the solving wavefront computes its own).
template <int LAT, int TL>
__device__ __forceinline__ void rate_candidate(const uint64_t* sumq, int64_t centre, int j, int nc, int half_log2,
                                               int fixed_k, uint32_t N, int64_t* b_out, double* R_out, int* k_out) {
  const int64_t b = nc == 1 ? centre
                            : clamp_i64(centre + (int64_t)(2 * j - (nc - 1)) * ((int64_t)1 << half_log2), kStepBitsMin,
                                        kStepBitsMax);
  const int kb = fixed_k >= 0 ? fixed_k : kwin_base(b);
  int best = 0;
  double rb = 0.0;
  for (int w = 0; w < kRcKwin; ++w) {
    const int k = fixed_k >= 0 ? fixed_k : kb + w;
    const double per_tile = (double)(tile_fixed_bits<LAT, TL>(k) - 16u) + (double)TL;
    const double bits = per_tile * (double)N + (double)sumq[j * kRcKwin + w];
    if (w == 0 || bits < rb) {
      rb = bits;
      best = w;
    }
  }
  *b_out = b;
  *R_out = rb;
  *k_out = fixed_k >= 0 ? fixed_k : kb + best;
}

// Bracket, interpolate and round: the next centre (or the final step bits) and the k of the
// candidate nearest to it (one lane; b, R, kc per candidate).
__device__ void rate_solve(const int64_t* b, const double* R, const int* kc, int nc, float target, uint32_t N,
                           int tl, int64_t* xb_out, int* k_out) {
  const double Tb = (double)target * (double)((uint64_t)N * (uint64_t)tl);
  const double nominal = (double)((uint64_t)N * (uint64_t)tl) / 8388608.0;
  double xv;
  int64_t lo, hi;
  int jf = -1;
  for (int i = 0; i < nc; ++i)
    if (R[i] <= Tb) {
      jf = i;
      break;
    }
  if (nc == 1) {
    xv = (double)b[0];
    lo = hi = b[0];
  } else if (jf < 0) {
    double slope = (R[nc - 2] - R[nc - 1]) / (double)(b[nc - 1] - b[nc - 2]);
    if (!(slope > 0.0)) slope = nominal;
    xv = (double)b[nc - 1] + (R[nc - 1] - Tb) / slope;
    lo = b[nc - 1];
    hi = b[nc - 1] + ((int64_t)1 << 25);
  } else if (jf == 0) {
    double slope = (R[0] - R[1]) / (double)(b[1] - b[0]);
    if (!(slope > 0.0)) slope = nominal;
    xv = (double)b[0] - (Tb - R[0]) / slope;
    lo = b[0] - ((int64_t)1 << 25);
    hi = b[0];
  } else {
    xv = (double)b[jf - 1] + (R[jf - 1] - Tb) * (double)(b[jf] - b[jf - 1]) / (R[jf - 1] - R[jf]);
    lo = b[jf - 1];
    hi = b[jf];
  }
  int64_t xb = (int64_t)floor(xv + 0.5);
  xb = clamp_i64(xb, lo, hi);
  xb = clamp_i64(xb, kStepBitsMin, kStepBitsMax);
  int best = 0;
  for (int i = 1; i < nc; ++i) {
    const int64_t di = b[i] > xb ? b[i] - xb : xb - b[i];
    const int64_t db = b[best] > xb ? b[best] - xb : xb - b[best];
    if (di < db) best = i;
  }
  *xb_out = xb;
  *k_out = kc[best];
}

// One rate pass: its counters, candidates and workgroups.
struct PassDesc {
  RateAcc* racc;
  int nc, half_log2, fixed_k;
  float target;
  uint32_t N;     // sample tiles
  uint32_t nblk;  // workgroups that add into the counters (workgroup b into set b mod kRcAccSlots)
};

// Arguments of the rate workgroups: the first workgroups of the encoder's launch when the call runs
// rate control, or every workgroup of rate_kernel when hq_rate runs alone.
struct RateArgs {
  const void* x;
  uint64_t T, seed;
  uint32_t df;
  Workspace* ws;
  RatePub* pub;
  PassDesc pa, pb;    // pass A (two passes only), and pass B or the single pass
  int two_pass;
  int64_t centre0;    // pass A's centre, or the fixed step's bits for the single pass
  uint32_t nblk;      // rate workgroups: pa.nblk (pass A: workgroups 0 ..) + pb.nblk (pass B: the next)
  uint32_t spin_budget;
  uint64_t call;
};

struct SolveLds {
  uint64_t sumq[kRcCounters];
  int64_t b[kRcCand];
  double R[kRcCand];
  int k[kRcCand];
};

// LDS of a rate workgroup.
struct RateLds {
  uint32_t red[kRcCounters];
  SolveLds solve;
  int64_t bcast;
};

// Orders one wavefront's LDS writes before its later reads (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Candidate j of a pass around `centre`, as a binary32 bit pattern.
__device__ __forceinline__ int64_t candidate_bits(int64_t centre, int j, int nc, int half_log2) {
  return nc == 1 ? centre
                 : clamp_i64(centre + (int64_t)(2 * j - (nc - 1)) * ((int64_t)1 << half_log2), kStepBitsMin,
                             kStepBitsMax);
}

// One lane's octet of a sample tile: transformed values, dither and tile scale.
struct Sample {
  float y[8], u[8];
  uint32_t sb;
  bool valid;
};

// Sample tile i of a pass of N tiles (nothing past the sample): transform and dither of the lane's
// octet.  Every lane of the wavefront calls it together.  True when the tile's energy is not finite.
template <int LAT, bool DITHER, int DT, int TL>
__device__ __forceinline__ bool sample_prepare(const RateArgs& A, uint32_t N, uint64_t i, int o, uint32_t sgn,
                                               Sample& s) {
  s.valid = i < N;
  const uint64_t t = s.valid ? sample_tile(i, A.T, N) : 0;
  bool finite;
  s.sb = transform_octet<DT, TL>(A.x, t, s.valid, o, sgn, s.y, &finite);
#pragma unroll
  for (int k = 0; k < 8; ++k) s.u[k] = 0.0f;
  if (DITHER) dither_octet<LAT>(A.seed, t, o, A.df, s.u);
  return s.valid && !finite;
}

// Rice quotient sums of the lane's octet at candidate j of a pass around `centre`, over the
// candidate's k window (q[w]; zeros for an invalid sample).  Each lane forms the multiplier of its
// own tile (A2: and of the odd slots); j is the same in every lane.
template <int LAT, bool DITHER, int TL>
__device__ __forceinline__ void sample_eval(const Sample& s, int o, int64_t centre, const PassDesc& pd, int j,
                                            uint32_t q[kRcKwin]) {
  constexpr int LPT = Tiling<TL>::LPT;
  const int64_t b = candidate_bits(centre, j, pd.nc, pd.half_log2);
  const float step = __uint_as_float((uint32_t)b);
  const uint32_t lane_neg = lane_sign_bit<LPT>(o);
  const float m = tile_multiplier<false>(s.sb, step, lane_neg);
  const float m1 = LAT == kLatA2 ? tile_multiplier<true>(s.sb, step, lane_neg) : m;
  uint32_t sym[8], cos;
  octet_symbols<LAT, DITHER>(s.y, m, m1, s.u, sym, &cos);
  const int kb = pd.fixed_k >= 0 ? pd.fixed_k : kwin_base(b);
#pragma unroll
  for (int w = 0; w < kRcKwin; ++w) {
    const int k = pd.fixed_k >= 0 ? pd.fixed_k : kb + w;
    uint32_t t = 0;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) t += sym[sl] >> slot_width<LAT>(sl, k);
    q[w] = s.valid ? t : 0u;
  }
}

// Adds the workgroup's sums into counter set b mod kRcAccSlots of the pass: acc[jj][w] of
// candidate j0 + jj (jj < nj; j0 and nj the same in a wavefront).  Every counter of the set
// receives one contribution, zero or not, so that its count shows when all of the pass's
// workgroups have added.  All lanes of the workgroup call it (two barriers).
template <int NJ>
__device__ uint64_t wg_add_counters(const uint32_t acc[NJ][kRcKwin], int j0, int nj, uint32_t* red, RateAcc* racc,
                                    uint32_t b) {
  const int tid = threadIdx.x;
  if (tid < kRcCounters) red[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int w = 0; w < kRcKwin; ++w)
      if (jj < nj && acc[jj][w]) atomicAdd(&red[(j0 + jj) * kRcKwin + w], acc[jj][w]);
  __syncthreads();
  uint64_t old = 0;
  if (tid < kRcCounters) {
    old = __hip_atomic_fetch_add(&racc->cnt[b % kRcAccSlots][tid], (1ull << kCntShift) + red[tid], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    // the returned value is waited for: the add has been performed before anything that follows
    __asm__ volatile("" ::"v"(old) : "memory");
  }
  return old;  // lane 0: the set's first word before this workgroup's add
}

// Contributions that counter set s of a pass receives from its nblk workgroups.
__device__ __forceinline__ uint32_t set_contribs(uint32_t s, uint32_t nblk) {
  return s < nblk ? (nblk - 1u - s) / (uint32_t)kRcAccSlots + 1u : 0u;
}

// The pass's counters summed over its sets into sumq, as soon as every word holds all of its
// contributions; false if that has not happened after `budget` polls.  One wavefront (all lanes).
__device__ bool pass_sums_wave(const PassDesc& pd, uint32_t budget, uint64_t* sumq) {
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  for (uint32_t spins = 0;; ++spins) {
    uint64_t sum = 0;
    bool done = true;
#pragma unroll
    for (int m = 0; m < kRcAccSlots / 2; ++m) {
      const int s = 2 * m + h;
      const uint64_t w = __hip_atomic_load(&pd.racc->cnt[s][c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      done = done && (uint32_t)(w >> kCntShift) == set_contribs((uint32_t)s, pd.nblk);
      sum += w & ((1ull << kCntShift) - 1ull);
    }
    if (__ballot(!done) == 0) {
      sum += __shfl_xor(sum, 32, 64);
      if (lane < kRcCounters) sumq[lane] = sum;
      wave_lds_sync();
      return true;
    }
    if (spins >= budget) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Every sample tile of a pass evaluated by one wavefront at all of the pass's candidates, summed
// into sumq: the same integer sums that the pass's workgroups add into its counters.  The fallback
// of a wait that has exceeded its budget (written for size, not speed: it runs only then); all
// lanes of the wavefront call it.  acc: kRcCounters words of LDS for this wavefront.
template <int LAT, bool DITHER, int DT, int TL>
__device__ void pass_sums_private(const RateArgs& A, const PassDesc& pd, int64_t centre, uint32_t* acc,
                                  uint64_t* sumq) {
  using TI = Tiling<TL>;
  const int lane = threadIdx.x & 63, o = lane % TI::LPT, tw = lane / TI::LPT;
  const uint32_t sgn = octet_sign_bits(A.seed, o);
  if (lane == 0) record_fallback(A.ws, A.call, kSlowPrivate);
  if (lane < kRcCounters) acc[lane] = 0u;
  wave_lds_sync();
#pragma unroll 1
  for (uint32_t i0 = 0; i0 < pd.N; i0 += (uint32_t)TI::TPW) {
    Sample s;
    sample_prepare<LAT, DITHER, DT, TL>(A, pd.N, (uint64_t)i0 + tw, o, sgn, s);
#pragma unroll 1
    for (int j = 0; j < pd.nc; ++j) {
      uint32_t q[kRcKwin];
      sample_eval<LAT, DITHER, TL>(s, o, centre, pd, j, q);
#pragma unroll
      for (int w = 0; w < kRcKwin; ++w)
        if (q[w]) atomicAdd(&acc[j * kRcKwin + w], q[w]);
    }
  }
  wave_lds_sync();
  if (lane < kRcCounters) sumq[lane] = acc[lane];
  wave_lds_sync();
}

// The candidates of a pass evaluated from its summed counters and solved by one wavefront (all
// lanes call it): the next centre, or the final step bits, and the Rice k.  Wave-uniform results.
template <int LAT, int TL>
__device__ void solve_sums_wave(const PassDesc& pd, int64_t centre, SolveLds* L, int64_t* xb_out, int* k_out) {
  const int lane = threadIdx.x & 63;
  if (lane < pd.nc) {
    int64_t b;
    double R;
    int kk;
    rate_candidate<LAT, TL>(L->sumq, centre, lane, pd.nc, pd.half_log2, pd.fixed_k, pd.N, &b, &R, &kk);
    L->b[lane] = b;
    L->R[lane] = R;
    L->k[lane] = kk;
  }
  wave_lds_sync();
  int64_t xb = 0;
  int kres = 0;
  if (lane == 0) rate_solve(L->b, L->R, L->k, pd.nc, pd.target, pd.N, TL, &xb, &kres);
  *xb_out = (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)xb);  // step bits: 32-bit, positive
  *k_out = __builtin_amdgcn_readfirstlane(kres);
}

// Solve of a pass by one wavefront from its counters, or, when they are not complete within the
// budget, from its own evaluation of the whole sample (the same sums, hence the same result).
template <int LAT, bool DITHER, int DT, int TL>
__device__ void solve_pass_wave(const RateArgs& A, const PassDesc& pd, int64_t centre, uint32_t budget, RateLds* L,
                                int64_t* xb, int* k) {
  if (!pass_sums_wave(pd, budget, L->solve.sumq))
    pass_sums_private<LAT, DITHER, DT, TL>(A, pd, centre, L->red, L->solve.sumq);
  solve_sums_wave<LAT, TL>(pd, centre, &L->solve, xb, k);
}

// Polls a published word with lane 0 (bit 63 set once published): the word, or false after
// `budget` polls.  Wave-uniform result.
__device__ bool wait_pub(const uint64_t* word, uint32_t budget, uint64_t* val) {
  uint32_t got = 0, lo = 0, hi = 0;
  if ((threadIdx.x & 63) == 0) {
    for (uint32_t spins = 0;; ++spins) {
      const uint64_t v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v >> 63) {
        got = 1;
        lo = (uint32_t)v;
        hi = (uint32_t)(v >> 32);
        break;
      }
      if (spins >= budget) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  got = __builtin_amdgcn_readfirstlane(got);
  *val = ((uint64_t)__builtin_amdgcn_readfirstlane(hi) << 32) | __builtin_amdgcn_readfirstlane(lo);
  return got != 0u;
}

// Publishes a word in every copy (lanes 0 .. kPubCopies-1 of the calling wavefront store one each).
__device__ __forceinline__ void publish(uint64_t* words, uint64_t v) {
  const int lane = threadIdx.x & 63;
  if (lane < kPubCopies)
    __hip_atomic_store(&words[lane * kPubStride], (1ull << 63) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rate workgroup b (0 <= b < A.nblk).  Workgroups 0 .. pa.nblk-1 run pass A: sample tiles
// b TPW .. b TPW + TPW - 1, two of its 8 candidates per wavefront (the four wavefronts take the
// same tiles); none of them waits, except workgroup 0, which then solves pass A as soon as its
// counters are complete and publishes the result, pass B's centre.  The next pb.nblk workgroups
// run pass B (or the single pass): sample tiles from 4 j TPW (j = b - pa.nblk), TPW per
// wavefront, every candidate, at the published centre (a workgroup that does not see it within
// its budget solves pass A itself); the last of them to add its sums solves pass B, stores the
// operating point in the workspace (the encoder, the next launch, reads it there) and leaves.
// Only pass B's workgroups wait, for pass A's, which come before them in the grid: no wait
// depends on how many workgroups the GPU holds at once.
template <int LAT, bool DITHER, int DT, int TL>
__device__ void rate_workgroup(const RateArgs& A, uint32_t b, RateLds& L) {
  using TI = Tiling<TL>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, o = lane % TI::LPT, tw = lane / TI::LPT;
  const uint32_t sgn = octet_sign_bits(A.seed, o);
  // waits for another workgroup's result: far beyond any wait in normal operation (the fallback
  // computes the awaited value itself, at the cost of evaluating a whole sample in one wavefront)
  const uint32_t budget = A.spin_budget > 0xFFFFFFFFu / 256u ? 0xFFFFFFFFu : A.spin_budget * 256u;
  if (b < A.pa.nblk) {  // pass A (uniform in the workgroup)
    const PassDesc& pa = A.pa;
    Sample sa;
    if (sample_prepare<LAT, DITHER, DT, TL>(A, pa.N, (uint64_t)b * TI::TPW + tw, o, sgn, sa) && o == 0 &&
        wave == 0)
      record_error(A.ws, A.call, kErrNonfinite);
    uint32_t acc[2][kRcKwin];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) sample_eval<LAT, DITHER, TL>(sa, o, A.centre0, pa, 2 * wave + jj, acc[jj]);
    wg_add_counters<2>(acc, 2 * wave, 2, L.red, pa.racc, b);
    if (b == 0 && wave == 0) {
      int64_t c;
      int k;
      solve_pass_wave<LAT, DITHER, DT, TL>(A, pa, A.centre0, budget, &L, &c, &k);
      publish(A.pub->centre, (uint64_t)(uint32_t)c);
    }
    return;
  }
  const PassDesc& pb = A.pb;
  const uint32_t j = b - A.pa.nblk;  // pass B workgroup
  uint64_t old0 = 0;
  Sample sb;
  if (sample_prepare<LAT, DITHER, DT, TL>(A, pb.N, ((uint64_t)j * 4 + wave) * TI::TPW + tw, o, sgn, sb) &&
      o == 0)
    record_error(A.ws, A.call, kErrNonfinite);
  int64_t centre = A.centre0;
  if (A.two_pass) {
    if (wave == 0) {
      uint64_t v = 0;
      int64_t c;
      int k;
      if (wait_pub(&A.pub->centre[(j % kPubCopies) * kPubStride], budget, &v)) {
        c = (int64_t)(uint32_t)v;
      } else {  // not published within the budget: pass A solved here
        if (lane == 0) record_fallback(A.ws, A.call, kSlowCentre);
        solve_pass_wave<LAT, DITHER, DT, TL>(A, A.pa, A.centre0, budget, &L, &c, &k);
      }
      if (lane == 0) L.bcast = c;
    }
    __syncthreads();
    centre = L.bcast;
    uint32_t acc[kRcCandB][kRcKwin];  // pass B's four candidates, independent of one another
#pragma unroll
    for (int jj = 0; jj < kRcCandB; ++jj) sample_eval<LAT, DITHER, TL>(sb, o, centre, pb, jj, acc[jj]);
    old0 = wg_add_counters<kRcCandB>(acc, 0, kRcCandB, L.red, pb.racc, j);
  } else {  // the single pass: one candidate
    uint32_t acc[1][kRcKwin];
    sample_eval<LAT, DITHER, TL>(sb, o, centre, pb, 0, acc[0]);
    old0 = wg_add_counters<1>(acc, 0, 1, L.red, pb.racc, j);
  }
  // the workgroup that completes the first word of its counter set (the word counts its own
  // contributions) counts the set in; the one that counts the last set in solves pass B (16
  // workgroups meet at that count rather than all of them: contended atomics on one word queue)
  if (tid == 0) {
    const uint32_t s = j % kRcAccSlots;
    const uint32_t nsets = pb.nblk < (uint32_t)kRcAccSlots ? pb.nblk : (uint32_t)kRcAccSlots;
    bool last = false;
    if ((uint32_t)(old0 >> kCntShift) + 1u == set_contribs(s, pb.nblk))
      last = __hip_atomic_fetch_add(&A.pub->done_b[0], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == nsets;
    L.bcast = last ? 1 : 0;
  }
  __syncthreads();
  if (L.bcast && wave == 0) {
    int64_t xb;
    int k;
    solve_pass_wave<LAT, DITHER, DT, TL>(A, pb, centre, budget, &L, &xb, &k);
    if (lane == 0) {
      Workspace* ws = A.ws;
      ws->rc_centre = xb;
      ws->step_bits = (uint32_t)xb;
      ws->rice_k = k;
      ws->res_step_bits = (uint32_t)xb;
      ws->res_k = k;
      ws->point_tag = kPointTag;
    }
  }
}

template <int LAT, bool DITHER, int DT, int TL>
__global__ __launch_bounds__(kBlock) void rate_kernel(RateArgs A) {
  __shared__ RateLds L;
  rate_workgroup<LAT, DITHER, DT, TL>(A, blockIdx.x, L);
}

// ---------------------------------------------------------------------------------------------
// Header of the stream (see hq.h), written by the workgroup that completes the last chunk.
// Symbols of one lane's octet in round r of chunk c, computed from the input again (load, sign,
// FWHT, tile scale, multiplier, dither, lattice).  Used only for octets whose unary code is longer
// than one word and for segments larger than the staging window; every lane of the wavefront must
// call it together (the FWHT and the tile energy exchange values between lanes).
template <int LAT, bool DITHER, int DT, int TL>
__device__ __forceinline__ void round_symbols(const void* x, uint64_t T, uint64_t seed, uint32_t df, uint32_t c, int r,
                                              int wave, int tw, int o, uint32_t sgn, uint32_t lane_neg, float step,
                                              uint32_t* sym) {
  using TI = Tiling<TL>;
  const uint64_t t = (uint64_t)c * TI::CT + (uint32_t)TI::TPR * r + (uint32_t)TI::TPW * wave + tw;
  // the sign masks are rebuilt here (the asm hides that they equal the caller's), so that callers
  // do not keep their own eight masks alive for this rarely taken path
  __asm__ volatile("" : "+v"(sgn));
  uint32_t smask[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) smask[i] = ((sgn >> i) & 1u) << 31;
  float y[8];
  if (t < T) {
    load_octet_signed<DT, TL>(x, t, o, smask, y);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.0f;
  }
  fwht_lane(y);
  fwht_cross<TI::LPT>(y, o);
  const float S = tile_sumsq<TI::LPT>(y);
  const bool fin = isfinite(S);
  if (!fin) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.0f;
  }
  const uint32_t sb = tile_scale_bits<TL>(fin ? S : 0.0f);
  const float m = tile_multiplier<false>(sb, step, lane_neg);
  const float m1 = LAT == kLatA2 ? tile_multiplier<true>(sb, step, lane_neg) : m;
  float u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (DITHER) dither_octet<LAT>(seed, t, o, df, u);
  uint32_t cos;
  octet_symbols<LAT, DITHER>(y, m, m1, u, sym, &cos);
}

__device__ void write_header(uint8_t* out, uint64_t cap, int lattice, uint32_t dflags, int k, uint32_t step_bits,
                             uint64_t seed, uint64_t n, uint64_t T, uint32_t chunks, uint32_t F,
                             uint64_t fixed_off, uint64_t unary_off, uint64_t words, uint64_t ubits,
                             uint64_t payload, uint64_t total, uint32_t tile, uint32_t log2_ct) {
  if (cap < (uint64_t)kHeaderBytes) return;
  uint32_t h[32];
  h[0] = kMagic;
  h[1] = kVersion | ((uint32_t)lattice << 16) | ((dflags & 0xFFu) << 24);
  h[2] = tile | ((uint32_t)k << 16) | (log2_ct << 24);
  h[3] = step_bits;
  h[4] = (uint32_t)seed; h[5] = (uint32_t)(seed >> 32);
  h[6] = (uint32_t)n; h[7] = (uint32_t)(n >> 32);
  h[8] = (uint32_t)T; h[9] = (uint32_t)(T >> 32);
  h[10] = chunks;
  h[11] = F;
  h[12] = (uint32_t)fixed_off; h[13] = (uint32_t)(fixed_off >> 32);
  h[14] = (uint32_t)unary_off; h[15] = (uint32_t)(unary_off >> 32);
  h[16] = (uint32_t)words; h[17] = (uint32_t)(words >> 32);
  h[18] = (uint32_t)ubits; h[19] = (uint32_t)(ubits >> 32);
  h[20] = (uint32_t)payload; h[21] = (uint32_t)(payload >> 32);
  h[22] = (uint32_t)total; h[23] = (uint32_t)(total >> 32);
  for (int i = 24; i < 32; ++i) h[i] = 0;
  uint32_t* o32 = reinterpret_cast<uint32_t*>(out);
  for (int i = 0; i < 32; ++i) o32[i] = h[i];
}

// Decoupled look-back (Merrill & Garland, "Single-pass parallel prefix scan with decoupled
// look-back", 2016) over chunks, run by one wavefront: each round reads the flags of 64
// predecessors at once, sums the aggregates up to the nearest inclusive prefix, and retries the
// window while a predecessor there has not published.  Chunk c is workgroup c.  A predecessor that
// has not published after `budget` spin rounds has its aggregate computed here from its input
// (agg_of, the whole wavefront: the same value its own workgroup will publish), so every wait ends
// whether or not the hardware has started that workgroup: forward progress does not depend on
// the order workgroups are dispatched in.  Each flag word carries its own value (flag in bits
// 62-63; the 64-bit word count in bits 0-33 and the padding-bit count in bits 34-61, summed
// field-wise), so relaxed agent-scope atomics suffice and no cache write-back or invalidation is
// needed.
template <class AggOf>
__device__ uint64_t lookback_wave(uint64_t* flags, uint32_t c, uint64_t agg, uint32_t budget, AggOf agg_of) {
  const int lane = threadIdx.x & 63;
  if (c == 0) {
    if (lane == 0) __hip_atomic_store(&flags[0], kFlagPrefix | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  if (lane == 0) __hip_atomic_store(&flags[c], kFlagAgg | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t excl = 0;
  int64_t base = (int64_t)c - 1;
  uint32_t spins = 0;
  while (true) {
    const int64_t j = base - lane;
    uint64_t sv = j >= 0 ? __hip_atomic_load(&flags[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : kFlagPrefix;
    const uint64_t f = sv & ~kValMask;
    const uint64_t pmask = __ballot(f == kFlagPrefix);
    const uint64_t zmask = __ballot(f == 0);
    const int first_p = pmask ? __ffsll((unsigned long long)pmask) - 1 : 64;
    const uint64_t need = first_p >= 63 ? ~0ull : ((2ull << first_p) - 1ull);
    uint64_t miss = zmask & need;
    if (miss) {
      if (spins++ < budget) {
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      // fallback: the missing aggregates of this window, computed from the predecessors' input
      while (miss) {
        const int l = __ffsll((unsigned long long)miss) - 1;
        miss &= miss - 1;
        const uint64_t a = agg_of((uint32_t)(base - l));
        if (lane == l) sv = kFlagAgg | a;
      }
      spins = 0;
    }
    uint64_t v = lane <= first_p ? (sv & kValMask) : 0ull;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    excl += v;
    if (first_p < 64) break;
    base -= 64;
  }
  if (lane == 0)
    __hip_atomic_store(&flags[c], kFlagPrefix | (excl + agg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return excl;
}

constexpr int kPadShift = 34;
constexpr uint64_t kWordsMask = (1ull << kPadShift) - 1;

// Look-back aggregate of chunk p (64-bit words of its unary segment, and its padding bits) computed
// by one wavefront from the chunk's input: the unary bits of its 4 x 4 (wavefront, round) tile
// groups, each recomputed by round_symbols.  Every lane of the wavefront calls it together.
template <int LAT, bool DITHER, int DT, int TL>
__device__ __forceinline__ uint64_t chunk_aggregate(const void* x, uint64_t T, uint64_t seed, uint32_t df,
                                                                uint32_t p, int k, uint32_t step_bits, uint32_t sgn,
                                                                uint32_t lane_neg) {
  using TI = Tiling<TL>;
  const int lane = threadIdx.x & 63, o = lane % TI::LPT, tw = lane / TI::LPT;
  const float step = __uint_as_float(step_bits);
  uint32_t bits = 0;
#pragma unroll 1
  for (int g = 0; g < 16; ++g) {
    const int gw = g >> 2, gr = g & 3;
    uint32_t sy[8];
    round_symbols<LAT, DITHER, DT, TL>(x, T, seed, df, p, gr, gw, tw, o, sgn, lane_neg, step, sy);
    const uint64_t t = (uint64_t)p * TI::CT + (uint32_t)TI::TPR * gr + (uint32_t)TI::TPW * gw + tw;
    if (t < T) {
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) bits += (sy[sl] >> slot_width<LAT>(sl, k)) + 1u;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) bits += __shfl_xor(bits, m, 64);
  const uint64_t w = (bits + 63u) / 64u;
  return w | ((64ull * w - bits) << kPadShift);
}

struct EncParams {
  const void* x;
  uint64_t n, T;
  uint32_t chunks;
  uint64_t seed;
  uint32_t dflags;  // dither flags (0 without dither)
  uint8_t* out;
  uint64_t cap;
  Workspace* ws;
  uint64_t* flags;
  uint32_t spin_budget;
  uint64_t call;
};

// The encoder's LDS: the chunk's fixed record, the unary staging window, per-round wavefront totals,
// the offsets of rounds written terminator by terminator, and the chunk's prefix.
struct EncLds {
  uint4 fixed4[kFixedWordsMax / 4];
  uint4 unary4[kUnaryWinWords / 4];
  uint4 wtot4[4];
  uint32_t off[4][kBlock];
  uint64_t prefix;
};

// One chunk of the encode (the body of encode_kernel; the LDS is the kernel's).
template <int LAT, bool DITHER, int DT, int TL>
__device__ __forceinline__ void encode_chunk(const EncParams& P, EncLds& lds) {
  using TI = Tiling<TL>;
  constexpr int LPT = TI::LPT;
  uint4* s_fixed4 = lds.fixed4;
  uint4* s_unary4 = lds.unary4;
  uint4* s_wtot4 = lds.wtot4;
  auto& s_off = lds.off;
  uint64_t& s_prefix = lds.prefix;
  uint32_t* s_fixed = reinterpret_cast<uint32_t*>(s_fixed4);
  uint32_t* s_unary = reinterpret_cast<uint32_t*>(s_unary4);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, o = lane % LPT, tw = lane / LPT;
  Workspace* ws = P.ws;
  const uint32_t c = blockIdx.x;
  const uint32_t step_bits = ws->step_bits;
  const int k = ws->rice_k;
  const float step = __uint_as_float(step_bits);
  const uint32_t F = tile_fixed_bits<LAT, TL>(k);
  const int RW = octet_rem_bits<LAT>(k);
  const int hdr = tile_hdr_bits<LAT, TL>();
  const uint32_t fixed_words = (uint32_t)TI::CT * F / 32u;  // a chunk's record, 16-byte multiple
  const uint64_t chunk_bytes = 4ull * fixed_words;
  const uint64_t fixed_off = align256(kHeaderBytes + 4ull * (P.chunks + 1));
  const uint64_t unary_off = align256(fixed_off + (uint64_t)P.chunks * chunk_bytes);
  const uint4 z4 = make_uint4(0, 0, 0, 0);
  for (uint32_t i = tid; i < fixed_words / 4; i += kBlock) s_fixed4[i] = z4;
  for (uint32_t i = tid; i < kUnaryWinWords / 4; i += kBlock) s_unary4[i] = z4;
  __syncthreads();

  // alignment padding of the stream (after the index, after the fixed plane) is zero bytes
  if (c == 0) {
    const uint64_t pads[2][2] = {{kHeaderBytes + 4ull * (P.chunks + 1), fixed_off},
                                 {fixed_off + (uint64_t)P.chunks * chunk_bytes, unary_off}};
    for (int pz = 0; pz < 2; ++pz)
      for (uint64_t b = pads[pz][0] + 4ull * tid; b < pads[pz][1]; b += 4ull * kBlock)
        if (b + 4 <= P.cap) *reinterpret_cast<uint32_t*>(P.out + b) = 0u;
  }

  if (c >= P.chunks) {  // empty tensor: one workgroup writes the header and the index
    if (P.chunks == 0 && tid == 0) {
      const uint64_t total = unary_off;
      write_header(P.out, P.cap, LAT, P.dflags, k, step_bits, P.seed, P.n, P.T, 0, F, fixed_off, unary_off, 0, 0,
                   0, total, TL, __builtin_ctz(TI::CT));
      if (P.cap >= kHeaderBytes + 4) reinterpret_cast<uint32_t*>(P.out)[kHeaderBytes / 4] = 0;
      if (total > P.cap) record_error(ws, P.call, kErrCapacity);
      ws->res_total_bytes = total;
      ws->res_payload_bits = 0;
      ws->res_unary_bits = 0;
      ws->res_words = 0;
      ws->res_step_bits = step_bits;
      ws->res_k = k;
    }
    return;
  }

  const uint32_t sgn = octet_sign_bits(P.seed, o);
  uint32_t smask[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) smask[i] = ((sgn >> i) & 1u) << 31;
  const uint32_t lane_neg = lane_sign_bit<LPT>(o);

  // phase 1: every round's transform and tile energy.  The chunk's input is read through a buffer
  // resource over its valid tiles, so tiles past the end load as zeros without per-tile branches.
  float y[4][8];
  float S[4];
  {
    constexpr uint32_t kEsz = DT == 1 ? 2u : 4u;
    const uint64_t t0 = (uint64_t)c * TI::CT;
    const uint64_t left = P.T - t0;
    const uint32_t vbytes = (uint32_t)(left < (uint64_t)TI::CT ? left : (uint64_t)TI::CT) * (uint32_t)TL * kEsz;
    const __amdgpu_buffer_rsrc_t rin =
        byte_range(reinterpret_cast<const uint8_t*>(P.x) + t0 * (uint64_t)TL * kEsz, vbytes);
    float sg[5];
    fwht_lane_signs<LPT>(o, sg);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t tc = (uint32_t)TI::TPR * r + (uint32_t)TI::TPW * wave + tw;
      load_octet_signed_buf<DT>(rin, (tc * (uint32_t)TL + 8u * (uint32_t)o) * kEsz, smask, y[r]);
      fwht_lane(y[r]);
      fwht_cross_s<LPT>(y[r], sg);
      S[r] = tile_sumsq<LPT>(y[r]);
    }
  }
  // one scale and one division per lane (round o mod 4; A2: lanes with bit 2 of o set divide for
  // the odd slots), broadcast inside the tile's lane group
  uint32_t sb_mine;
  float m_mine;
  {
    const int rr = o & 3;
    const float Sr = rr == 0 ? S[0] : rr == 1 ? S[1] : rr == 2 ? S[2] : S[3];
    const bool fin = isfinite(Sr);
    const uint64_t t = (uint64_t)c * TI::CT + (uint32_t)TI::TPR * rr + (uint32_t)TI::TPW * wave + tw;
    if (!fin && t < P.T && o < 4) record_error(ws, P.call, kErrNonfinite);
    sb_mine = tile_scale_bits<TL>(fin ? Sr : 0.0f);
    m_mine = (LAT == kLatA2 && (o & 4)) ? tile_multiplier<true>(sb_mine, step, 0u)
                                        : tile_multiplier<false>(sb_mine, step, 0u);
  }
  uint32_t sbr[4];
  float mr[4], mr1[4];
  sbr[0] = group_bcast<0, LPT>(sb_mine); sbr[1] = group_bcast<1, LPT>(sb_mine);
  sbr[2] = group_bcast<2, LPT>(sb_mine); sbr[3] = group_bcast<3, LPT>(sb_mine);
  mr[0] = __uint_as_float(group_bcast<0, LPT>(__float_as_uint(m_mine)));
  mr[1] = __uint_as_float(group_bcast<1, LPT>(__float_as_uint(m_mine)));
  mr[2] = __uint_as_float(group_bcast<2, LPT>(__float_as_uint(m_mine)));
  mr[3] = __uint_as_float(group_bcast<3, LPT>(__float_as_uint(m_mine)));
  if (LAT == kLatA2) {
    mr1[0] = __uint_as_float(group_bcast<4, LPT>(__float_as_uint(m_mine)));
    mr1[1] = __uint_as_float(group_bcast<5, LPT>(__float_as_uint(m_mine)));
    mr1[2] = __uint_as_float(group_bcast<6, LPT>(__float_as_uint(m_mine)));
    mr1[3] = __uint_as_float(group_bcast<7, LPT>(__float_as_uint(m_mine)));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) mr1[r] = mr[r];
  }

  // phase 2: quantise, strip, pack the fixed record, Rice lengths and unary patterns
  uint32_t sym[4][8];
  uint32_t L[4], pat[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t tc = (uint32_t)TI::TPR * r + (uint32_t)TI::TPW * wave + tw;
    const uint64_t t = (uint64_t)c * TI::CT + tc;
    const bool valid = t < P.T;
    if (__ballot(!isfinite(S[r]))) {  // uniform test: the common case skips the block entirely
      // (the empty asm keeps the branch: without it the compiler runs the block with an empty
      // execution mask, eight instructions per round)
      __asm__ volatile("");
      if (!isfinite(S[r])) {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[r][i] = 0.0f;
      }
    }
    float u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (DITHER) dither_octet<LAT>(P.seed, t, o, P.dflags, u);
    uint32_t cos;
    // without dither the encoder's scalar unit has room for the mask form of the E8 fix-up (measured:
    // faster here; slower in the dithered encoder and in the rate passes)
    octet_symbols<LAT, DITHER, !DITHER>(y[r], lane_neg ? -mr[r] : mr[r], lane_neg ? -mr1[r] : mr1[r], u, sym[r],
                                        &cos);
    const uint64_t bal = __ballot(valid && cos != 0u);
    uint32_t len = 8;
    if (valid) {
      const uint32_t rec = tc * F;
      if (o == 0) {
        if (LAT == kLatE8 && LPT <= 16) {
          // the scale and the tile's coset bits as one field of 16 + LPT <= 32 bits
          const uint32_t v = sbr[r] | (((uint32_t)(bal >> (LPT * tw)) & low_mask(LPT)) << 16);
          const uint32_t sh = rec & 31u;
          atomicOr(&s_fixed[rec >> 5], v << sh);
          if (sh + 16u + (uint32_t)LPT > 32u) atomicOr(&s_fixed[(rec >> 5) + 1], __builtin_amdgcn_alignbit(0u, v, 32u - sh));
        } else {
          lds_put_bits(s_fixed, rec, sbr[r], 16);
          if (LAT == kLatE8) lds_put_bits(s_fixed, rec + 16, (uint32_t)(bal >> (LPT * tw)) & low_mask(LPT), LPT);
        }
      }
      // A2: the octet's four pair cosets, bits 4 o .. 4 o + 3 after the scale (never across a word)
      if (LAT == kLatA2) lds_put_bits(s_fixed, rec + 16 + 4u * (uint32_t)o, cos, 4);
      uint32_t pos = rec + hdr + (uint32_t)o * RW;
      if (RW <= 32) {  // uniform: the field is one word, ORed into at most two
        uint32_t lo, hi;
        pack_octet_remainders<LAT>(sym[r], k, &lo, &hi);
        const uint32_t sh = pos & 31u;
        atomicOr(&s_fixed[pos >> 5], lo << sh);
        if (sh + (uint32_t)RW > 32u) atomicOr(&s_fixed[(pos >> 5) + 1], __builtin_amdgcn_alignbit(0u, lo, 32u - sh));
      } else if (k <= 8) {
        uint32_t lo, hi;
        pack_octet_remainders<LAT>(sym[r], k, &lo, &hi);
        lds_put_field64(s_fixed, pos, lo, hi);
      } else {
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int w = slot_width<LAT>(sl, k);
          lds_put_bits(s_fixed, pos, sym[r][sl] & low_mask(w), w);
          pos += w;
        }
      }
      // unary code of the octet relative to its start: the terminator of slot s sits at
      // c_s = sum over s' <= s of (q_s' + 1), minus 1; bits at c >= 32 only matter when L > 32,
      // and such octets are written terminator by terminator below
      uint32_t cpos = 0xFFFFFFFFu, pt = 0;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        cpos += (sym[r][sl] >> slot_width<LAT>(sl, k)) + 1u;
        pt |= 1u << (cpos & 31u);
      }
      len = cpos + 1u;
      pat[r] = pt;
    } else {
      pat[r] = 0;
    }
    L[r] = valid ? len : 0u;
  }

  // unary offsets inside the chunk (octet index 256 r + tid is the symbol order): wavefront scans
  // of every round, then one exchange of the 16 wavefront totals
  uint32_t incl[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) incl[r] = wave_incl_scan(L[r]);
  if (lane == 63) {
    uint32_t* wt = reinterpret_cast<uint32_t*>(s_wtot4);
#pragma unroll
    for (int r = 0; r < 4; ++r) wt[4 * r + wave] = incl[r];
  }
  __syncthreads();
  uint32_t off[4], B = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint4 t4 = s_wtot4[r];
    const uint32_t before = (wave > 0 ? t4.x : 0u) + (wave > 1 ? t4.y : 0u) + (wave > 2 ? t4.z : 0u);
    off[r] = B + before + incl[r] - L[r];
    B += (t4.x + t4.y) + (t4.z + t4.w);
  }
  const uint64_t W = (B + 63u) / 64u;

  // unary segment, staged through LDS in windows of kUnaryWinBits.  Common case: the segment fits
  // one window and each octet's code (at most 32 bits) is ORed in as one pattern, now: its position
  // inside the chunk does not depend on the chunk's prefix.  Otherwise the symbols of the rounds
  // concerned are computed again after the look-back and written terminator by terminator; those
  // rounds' offsets wait in LDS (nothing of a round stays in registers across the look-back).
  const bool multi = B > kUnaryWinBits;
  if (!multi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t p0 = off[r];
      if (L[r] != 0u && L[r] <= 32u) {
        const uint32_t sh = p0 & 31u;
        atomicOr(&s_unary[p0 >> 5], pat[r] << sh);
        if (sh + L[r] > 32u) atomicOr(&s_unary[(p0 >> 5) + 1], __builtin_amdgcn_alignbit(0u, pat[r], 32u - sh));
      }
    }
  }
  uint32_t slow = 0;  // rounds (bit r) in which some lane of this wavefront writes terminators
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (__ballot(multi ? L[r] != 0u : L[r] > 32u)) {
      slow |= 1u << r;
      s_off[r][tid] = off[r];
    }

  if (wave == 0) {
    const uint64_t agg = W | ((64ull * W - B) << kPadShift);
    // the look-back's fallback: a predecessor's aggregate computed by this wavefront
    auto agg_of = [&](uint32_t p) -> uint64_t {
      if (lane == 0) record_fallback(ws, P.call, kSlowLookback);
      return chunk_aggregate<LAT, DITHER, DT, TL>(P.x, P.T, P.seed, P.dflags, p, k, step_bits, sgn, lane_neg);
    };
    const uint64_t ex = lookback_wave(P.flags, c, agg, P.spin_budget, agg_of);
    if (lane == 0) s_prefix = ex;
  } else {
    // the chunk's fixed record (its place does not depend on the prefix), by the other
    // wavefronts while wavefront 0 looks back
    const uint64_t fbase = fixed_off + (uint64_t)c * chunk_bytes;
    if (fbase + chunk_bytes <= P.cap) {
      uint4* dst = reinterpret_cast<uint4*>(P.out + fbase);
      for (uint32_t i = tid - 64u; i < fixed_words / 4; i += kBlock - 64u) dst[i] = s_fixed4[i];
    } else if (tid == 64) {
      record_error(ws, P.call, kErrCapacity);
    }
  }
  __syncthreads();
  const uint64_t prefix = s_prefix & kWordsMask;
  const uint64_t prefix_pad = s_prefix >> kPadShift;
  if (tid == 0) {
    if (prefix + W > 0xFFFFFFFFull) record_error(ws, P.call, kErrRange);  // u32 chunk index
    if (kHeaderBytes + 4ull * c + 4 <= P.cap)
      reinterpret_cast<uint32_t*>(P.out + kHeaderBytes)[c] = (uint32_t)prefix;
    else
      record_error(ws, P.call, kErrCapacity);
  }

  const uint64_t ubase = unary_off + 8ull * prefix;
  const bool fits = ubase + 8ull * W <= P.cap;
  const uint32_t seg_words = (uint32_t)(2u * W);
  for (uint32_t wb = 0; wb < B; wb += kUnaryWinBits) {
    if (wb) {
      __syncthreads();
      for (uint32_t i = tid; i < kUnaryWinWords / 4; i += kBlock) s_unary4[i] = z4;
      __syncthreads();
    }
#pragma unroll 1
    for (int r = 0; r < 4; ++r) {
      if (!((slow >> r) & 1u)) continue;  // uniform in the wavefront
      const uint32_t offr = s_off[r][tid];
      uint32_t sy[8];
      round_symbols<LAT, DITHER, DT, TL>(P.x, P.T, P.seed, P.dflags, c, r, wave, tw, o, sgn, lane_neg, step, sy);
      // the octet's unary length again, from the recomputed symbols (0 past the last tile)
      uint32_t Lr = 0;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) Lr += (sy[sl] >> slot_width<LAT>(sl, k)) + 1u;
      if ((uint64_t)c * TI::CT + (uint32_t)TI::TPR * r + (uint32_t)TI::TPW * wave + tw >= P.T) Lr = 0;
      if (multi ? Lr != 0u : Lr > 32u) {
        uint32_t p = offr;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          p += sy[sl] >> slot_width<LAT>(sl, k);
          const uint32_t rel = p - wb;
          if (p >= wb && rel < kUnaryWinBits) atomicOr(&s_unary[rel >> 5], 1u << (rel & 31u));
          p += 1;
        }
      }
    }
    __syncthreads();
    const uint32_t w0 = wb >> 5;
    const uint32_t nw = min((uint32_t)kUnaryWinWords, seg_words - w0);
    if (fits) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(P.out + ubase) + w0;
      for (uint32_t i = tid; i < nw; i += kBlock) dst[i] = s_unary[i];
    }
  }
  if (!fits && tid == 0) record_error(ws, P.call, kErrCapacity);

  if (c == P.chunks - 1 && tid == 0) {
    const uint64_t words = prefix + W;
    const uint64_t total = unary_off + 8ull * words;
    const uint64_t ubits = 64ull * words - (prefix_pad + (64ull * W - B));
    const uint64_t payload = P.T * (uint64_t)(F - 16u) + ubits;
    write_header(P.out, P.cap, LAT, P.dflags, k, step_bits, P.seed, P.n, P.T, P.chunks, F, fixed_off, unary_off,
                 words, ubits, payload, total, TL, __builtin_ctz(TI::CT));
    if (kHeaderBytes + 4ull * P.chunks + 4 <= P.cap)
      reinterpret_cast<uint32_t*>(P.out + kHeaderBytes)[P.chunks] = (uint32_t)words;
    if (total > P.cap) record_error(ws, P.call, kErrCapacity);
    ws->res_total_bytes = total;
    ws->res_payload_bits = payload;
    ws->res_unary_bits = ubits;
    ws->res_words = words;
    ws->res_step_bits = step_bits;
    ws->res_k = k;
  }
}

// Occupancy: seven waves per SIMD without dither (71 registers, and a 22.3 KiB LDS footprint so
// that seven workgroups fit a CU's 160 KiB; measured 86.5 -> 82.8 us on the 14336 x 4096 weight
// against six), five with it (the register budgets the hot path fits in); the look-back's rare
// fallback must fit the same budget.
template <int LAT, bool DITHER, int DT, int TL>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(DITHER ? 5 : 7))) void encode_kernel(
    EncParams P) {
  __shared__ EncLds lds;
  encode_chunk<LAT, DITHER, DT, TL>(P, lds);
}

// ---------------------------------------------------------------------------------------------
// Diagnostic codes kernel: front half at a fixed step, integer codes and scale bits out.
template <int LAT, bool DITHER, int DT, int TL>
__global__ __launch_bounds__(kBlock) void codes_kernel(const void* __restrict__ x, uint64_t T, uint64_t seed,
                                                       uint32_t df, uint32_t step_bits, int32_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales, Workspace* ws, uint64_t call) {
  using TI = Tiling<TL>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, o = lane % TI::LPT, tw = lane / TI::LPT;
  const uint64_t t = (uint64_t)blockIdx.x * TI::TPR + wave * TI::TPW + tw;
  const bool valid = t < T;
  const uint32_t sgn = octet_sign_bits(seed, o);
  float y[8];
  bool finite;
  const uint32_t sb = transform_octet<DT, TL>(x, t, valid, o, sgn, y, &finite);
  if (valid && !finite && o == 0) record_error(ws, call, kErrNonfinite);
  float u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (DITHER) dither_octet<LAT>(seed, t, o, df, u);
  int32_t code[8];
  quantize_octet<LAT, DITHER>(y, sb, __uint_as_float(step_bits), u, code, lane_sign_bit<TI::LPT>(o));
  if (valid) {
    int4* dst = reinterpret_cast<int4*>(codes + t * TL + 8 * o);
    dst[0] = make_int4(code[0], code[1], code[2], code[3]);
    dst[1] = make_int4(code[4], code[5], code[6], code[7]);
    if (o == 0) scales[t] = (uint16_t)sb;
  }
}

// ---------------------------------------------------------------------------------------------
// Decoder.
// The stream header's validity and the fields the decoder needs.
// Fields of a stream header that the decoder needs.
struct DecInfo {
  uint32_t tile, lattice, dither, F, chunks, step_bits;
  int k;
  uint64_t seed, tiles, fixed_off, unary_off, words;
};

// Validates the stream header of `in` (in_bytes bytes) for n values and, for a matrix product, a row
// length cols of whole tiles (0 for a plain decode), with the first and last chunk index entries,
// and fills *d.  Scalar loads: every lane computes the same.  False for a corrupt stream.
__device__ __forceinline__ bool read_header(const uint8_t* __restrict__ in, uint64_t in_bytes, uint64_t n,
                                            uint64_t cols, DecInfo* d) {
  // a chunk is kChunkValues values at every tile length: the chunk count, and with it the first and
  // last index entries, follow from n, so their loads go out with the header's
  const uint32_t chunks = (uint32_t)((n + kChunkValues - 1) / kChunkValues);
  if (in_bytes < (uint64_t)kHeaderBytes + 4ull * ((uint64_t)chunks + 1)) return false;
  const uint32_t* __restrict__ h = reinterpret_cast<const uint32_t*>(in);
  const uint32_t* __restrict__ idx = reinterpret_cast<const uint32_t*>(in + kHeaderBytes);
  const uint32_t i_first = idx[0], i_last = idx[chunks];
  const uint64_t hn = ((uint64_t)h[7] << 32) | h[6];
  const uint32_t htile = h[2] & 0xFFFFu;
  const bool tile_ok = htile == 64u || htile == 128u || htile == 256u;
  const uint32_t tile = tile_ok ? htile : 128u;
  const uint32_t ct = (uint32_t)kChunkValues / tile;  // tiles per chunk
  const uint64_t T = n / tile;
  const int lattice = (int)((h[1] >> 16) & 0xFF), flags = (int)(h[1] >> 24), k = (int)((h[2] >> 16) & 0xFF);
  const bool flags_ok = flags == 0 || (flags <= 7 && (flags & 1));  // dither flags
  if (!(tile_ok && h[0] == kMagic && (h[1] & 0xFFFFu) == kVersion && lattice <= kLatA2 && flags_ok && k <= 15 &&
        (h[2] >> 24) == (uint32_t)__builtin_ctz(ct) && h[3] >= kStepBitsMin && h[3] <= kStepBitsMax && hn == n &&
        (n % tile) == 0 && (cols % tile) == 0))
    return false;
  const int kh = k > 0 ? k - 1 : 0;
  const int rem = lattice == kLatE8 ? 7 * k + kh
                  : lattice == kLatD4 ? 6 * k + 2 * kh
                  : lattice == kLatA2 ? 4 * k + 4 * kh
                                      : 8 * k;
  const uint32_t oct = tile / 8u;
  const uint32_t F = 16u + (lattice == kLatE8 ? oct : lattice == kLatA2 ? 4u * oct : 0u) + oct * (uint32_t)rem;
  const uint64_t fixed_off = align256(kHeaderBytes + 4ull * (chunks + 1));
  const uint64_t unary_off = align256(fixed_off + (uint64_t)chunks * ct * F / 8ull);
  const uint64_t words = ((uint64_t)h[17] << 32) | h[16];
  const uint64_t total = ((uint64_t)h[23] << 32) | h[22];
  if (!((((uint64_t)h[9] << 32) | h[8]) == T && h[10] == chunks && h[11] == F &&
        (((uint64_t)h[13] << 32) | h[12]) == fixed_off && (((uint64_t)h[15] << 32) | h[14]) == unary_off &&
        total <= in_bytes && words <= (1ull << 32) && unary_off + 8ull * words == total))
    return false;
  if (!(i_first == 0u && (uint64_t)i_last == words)) return false;
  d->tile = tile;
  d->lattice = (uint32_t)lattice;
  d->dither = (uint32_t)flags;
  d->k = k;
  d->step_bits = h[3];
  d->F = F;
  d->chunks = chunks;
  d->seed = ((uint64_t)h[5] << 32) | h[4];
  d->tiles = T;
  d->fixed_off = fixed_off;
  d->unary_off = unary_off;
  d->words = words;
  return true;
}

// The header check of a matrix product, whose later kernels read the header's fields from the
// workspace: read_header, and lane 0 of the calling workgroup numbers the workspace with the call,
// publishes the fields (or the error) there.
__device__ bool check_header(const uint8_t* __restrict__ in, uint64_t in_bytes, uint64_t n, uint64_t cols,
                             Workspace* ws, bool publish, uint64_t call, DecInfo* d) {
  const bool ok = read_header(in, in_bytes, n, cols, d);
  if (publish && threadIdx.x == 0) {
    ws->call = call;
    ws->dec_valid = 0;
    if (!ok) record_error(ws, call, kErrCorrupt);
    if (ok) {
      ws->dec_tile = d->tile;
      ws->dec_lattice = d->lattice;
      ws->dec_dither = d->dither;
      ws->dec_k = d->k;
      ws->dec_step_bits = d->step_bits;
      ws->dec_F = d->F;
      ws->dec_chunks = d->chunks;
      ws->dec_seed = d->seed;
      ws->dec_tiles = d->tiles;
      ws->dec_fixed_off = d->fixed_off;
      ws->dec_unary_off = d->unary_off;
      ws->dec_words = d->words;
      ws->dec_valid = 1;
    }
  }
  return ok;
}

// The header check alone (a matrix product of an empty matrix).
__global__ void decode_check_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes, uint64_t n, Workspace* ws,
                                    uint64_t call) {
  DecInfo d;
  check_header(in, in_bytes, n, 0, ws, true, call, &d);
}

constexpr int kMaxSymsPerChunk = kChunkValues;

// One slot's remainder from an octet field held in (lo, hi) (at most 64 bits); off and w are the
// same in every lane.
__device__ __forceinline__ uint32_t field_slot(uint32_t lo, uint32_t hi, int off, int w) {
  if (w == 0) return 0u;
  if (off >= 32) return __builtin_amdgcn_ubfe(hi, (uint32_t)(off - 32), (uint32_t)w);
  if (off + w <= 32) return __builtin_amdgcn_ubfe(lo, (uint32_t)off, (uint32_t)w);
  return __builtin_amdgcn_alignbit(hi, lo, (uint32_t)off) & low_mask(w);
}

// Bit field of `nbits` (<= 32) bits at bit position pos of a plane in global memory; both words
// are read unconditionally (callers guarantee the second is inside the stream).
__device__ __forceinline__ uint32_t plane_bits(const uint32_t* __restrict__ pl, uint32_t pos, int nbits) {
  const uint32_t word = pos >> 5;
  return __builtin_amdgcn_alignbit(pl[word + 1], pl[word], pos & 31u) & low_mask(nbits);
}

typedef float hq_f2 __attribute__((ext_vector_type(2)));
typedef uint32_t hq_u4 __attribute__((ext_vector_type(4)));
typedef __bf16 hq_b2 __attribute__((ext_vector_type(2)));

// Twice the un-zigzagged value of a symbol: 2 unzz(s) = s ^ -(s & 1) (s for even s, -s - 1 for odd).
__device__ __forceinline__ int32_t twice_unzz(uint32_t s) {
  return (int32_t)(s ^ (uint32_t)__builtin_amdgcn_sbfe((int32_t)s, 0u, 1u));
}

// Decode of one chunk's tiles: the first round's record words are requested, the terminator
// positions of the chunk's unary segment are found (unary_positions), then the rounds run.
// Each lane rebuilds one octet per round: Rice symbols (unary part from consecutive terminator
// positions, remainders from the fixed record read in place), lattice codes, rescale (and dither
// removal), inverse FWHT, sign and 1/TL, store.  The fixed-record words of round r + 1 are loaded
// while round r is computed.  Every read of the record stays inside the stream: a chunk's record
// has room for all its 8192 / TL tiles, and at most two words past its end lie in the unary plane,
// which holds at least one word per symbol's chunk once the chunk's terminator count has been
// checked.  The first round, requested before that check, reads only the first quarter of the
// chunk's records.
// Extra arguments of the fused decode + matrix-vector product: the rotated activation (one
// TL-value tile per column tile of the matrix), the matrix's columns, and the per-tile partial
// products.
struct GemvArgs {
  const float* xt;
  uint64_t cols;  // the matrix's columns: cols / TL column tiles
  float* tp;
};

// Terminator positions of a chunk's unary segment (nW32 words at seg) into the workgroup's table,
// which holds kMaxSymsPerChunk 16-bit entries or half as many 32-bit ones.  Thread i takes words
// [i m, i m + m) (m = ceil(nW32 / 256)), counts their set bits, a workgroup scan gives each thread
// the index of its first symbol, and, once the total is checked to equal the chunk's symbol count
// nsym (so every write below stays inside the table), it writes the position of each set bit:
//   MODE 0 (nW32 <= kPos16Words, so every position fits 16 bits): every terminator, 16-bit;
//   MODE 1 / 2: the terminators of symbols [0, 4096) / [4096, 8192) as 32-bit entries at index
//   g - 4096 (MODE - 1); MODE 2 also puts terminator 4095's position into *s_boundary.
// Returns false (for the whole workgroup) on a count mismatch, after flagging the stream corrupt.
constexpr uint32_t kPos16Words = 2048;       // 65536 bits
constexpr uint32_t kPosHalf = kMaxSymsPerChunk / 2;
template <int MODE>
__device__ __forceinline__ bool unary_positions(const uint32_t* __restrict__ seg, uint32_t nW32, uint32_t nsym,
                                                uint32_t* s_pos, uint32_t* s_boundary, Workspace* ws,
                                                uint64_t call) {
  uint32_t* s_wsum = s_pos;  // the four wavefront totals, read before any position is written
  uint16_t* t16 = reinterpret_cast<uint16_t*>(s_pos);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t m = (nW32 + kBlock - 1) / kBlock;
  const uint32_t j0 = min((uint32_t)tid * m, nW32), j1 = min(j0 + m, nW32);
  // segments of up to 1024 words (4 bits per symbol): the run is loaded once, all words at once,
  // and kept in registers for the scatter
  const bool small = MODE == 0 && m <= 4u;
  uint32_t wd[4] = {0u, 0u, 0u, 0u};
  uint32_t cnt = 0;
  if (small) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (j0 + (uint32_t)i < j1) wd[i] = seg[j0 + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt += (uint32_t)__popc(wd[i]);
  } else {
    for (uint32_t j = j0; j < j1; ++j) cnt += (uint32_t)__popc(seg[j]);
  }
  const uint32_t incl = wave_incl_scan(cnt);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  const uint32_t t0 = s_wsum[0], t1 = s_wsum[1], t2 = s_wsum[2], t3 = s_wsum[3];
  const uint32_t total = (t0 + t1) + (t2 + t3);
  __syncthreads();  // every lane has the totals before the table is overwritten
  if (total != nsym) {  // uniform: the whole workgroup leaves
    if (tid == 0 && MODE != 2) record_error(ws, call, kErrCorrupt);
    return false;
  }
  uint32_t g = (wave > 0 ? t0 : 0u) + (wave > 1 ? t1 : 0u) + (wave > 2 ? t2 : 0u) + incl - cnt;
  if (small) {
    // two set bits per pass (the second write only where that bit exists): half the passes of a
    // one-bit loop for one more compare
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t bits = wd[i];
      const uint32_t bitbase = (j0 + (uint32_t)i) * 32u;
      const uint32_t gnext = g + (uint32_t)__popc(bits);
      while (bits) {
        const uint32_t b1 = bits & (bits - 1u);
        t16[g] = (uint16_t)(bitbase + (uint32_t)__builtin_ctz(bits));
        if (b1) t16[g + 1] = (uint16_t)(bitbase + (uint32_t)__builtin_ctz(b1));
        g += 2;
        bits = b1 & (b1 - 1u);
      }
      g = gnext;
    }
  } else {
    for (uint32_t j = j0; j < j1; ++j) {
      uint32_t bits = seg[j];
      const uint32_t bitbase = j * 32u;
      while (bits) {
        const uint32_t pos = bitbase + (uint32_t)__builtin_ctz(bits);
        if (MODE == 0) {
          t16[g] = (uint16_t)pos;
        } else {
          const uint32_t gl = g - (MODE == 2 ? kPosHalf : 0u);  // wraps above the half when below it
          if (gl < kPosHalf) s_pos[gl] = pos;
          if (MODE == 2 && g == kPosHalf - 1u) *s_boundary = pos;
        }
        ++g;
        bits &= bits - 1u;
      }
    }
  }
  __syncthreads();
  return true;
}

template <int LAT, int DT_OUT, bool GEMV, int TL, int KC = -1>
__device__ __forceinline__ void decode_chunk_body(const uint8_t* __restrict__ in, void* __restrict__ out,
                                                  Workspace* ws, uint64_t call, uint32_t c, uint32_t tiles_c,
                                                  const uint32_t* __restrict__ seg, uint32_t nW32, uint32_t* s_pos,
                                                  uint32_t* s_boundary, float4* s_fac, GemvArgs g) {
  using TI = Tiling<TL>;
  constexpr int LPT = TI::LPT;
  constexpr float kInvTile = 1.0f / (float)TL;  // exact power of two
  // the E8 coset bit of a tile of 256 lies beyond the 32-bit window that holds the scale
  constexpr bool kCosetWord = LAT == kLatA2 || (LAT == kLatE8 && LPT > 16);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, o = lane % LPT, tw = lane / LPT;
  // KC >= 0: the stream's Rice parameter as a compile-time constant (the header check has
  // verified that the record length matches it)
  // the stream's fields, read from its (validated, read-only) header where they are needed
  const uint32_t* __restrict__ hw = reinterpret_cast<const uint32_t*>(in);
  const int k = KC >= 0 ? KC : (int)((hw[2] >> 16) & 0xFFu);
  const uint32_t F = KC >= 0 ? tile_fixed_bits<LAT, TL>(KC) : hw[11];
  const uint32_t df = hw[1] >> 24;  // dither flags of the stream
  const bool dither = df != 0u;
  const uint64_t seed = ((uint64_t)hw[5] << 32) | hw[4];
  const float step = __uint_as_float(hw[3]);
  const int RW = octet_rem_bits<LAT>(k);
  const uint32_t hdr = (uint32_t)tile_hdr_bits<LAT, TL>();
  const uint32_t* __restrict__ fw =
      reinterpret_cast<const uint32_t*>(in + (((uint64_t)hw[13] << 32) | hw[12]) + (uint64_t)c * ((uint64_t)TI::CT * F / 8ull));
  // output factor per coordinate: +-1/TL with the sign of D and of the lane's butterfly sign; the
  // fused multiply-add with +0 below is exact and turns an exact zero into +0
  // These factors and the cross-lane butterflies' +-1 depend only on the octet index o: a table of
  // them per o (lanes 0 .. LPT-1 fill it; the barriers of unary_positions publish it) is read
  // again in every round, which costs three LDS reads instead of about 40 vector instructions of
  // re-deriving them from o (the registers to keep them would cost a wave per SIMD).
  if (tid < LPT) {
    const uint32_t sgn = octet_sign_bits(seed, tid) ^ (lane_sign_bit<LPT>(tid) ? 0xFFu : 0u);
    float f[12];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = ((sgn >> i) & 1u) ? -kInvTile : kInvTile;
#pragma unroll
    for (int j = 0; j < 4; ++j) f[8 + j] = (tid & (1 << j)) ? -1.0f : 1.0f;
    s_fac[3 * tid] = make_float4(f[0], f[1], f[2], f[3]);
    s_fac[3 * tid + 1] = make_float4(f[4], f[5], f[6], f[7]);
    s_fac[3 * tid + 2] = make_float4(f[8], f[9], f[10], f[11]);
  }
  bool bad = false;
  // record words of a round: the tile header (scale, then E8 coset bits), the word with the octet's
  // coset bits when they are not in that window (A2's four; E8 at 32 lanes per tile), and the
  // octet's field
  const uint32_t cbit = LAT == kLatA2 ? 4u * (uint32_t)o : (uint32_t)o;  // coset bits after the scale
  uint32_t hA, hB, hC, f0, f1, f2;
  auto issue = [&](int r) {
    const uint32_t rec = ((uint32_t)TI::TPR * r + (uint32_t)TI::TPW * wave + tw) * F;
    const uint32_t P = rec + hdr + (uint32_t)o * (uint32_t)RW;
    hA = fw[rec >> 5];
    hB = fw[(rec >> 5) + 1];
    hC = kCosetWord ? fw[(rec + 16u + cbit) >> 5] : 0u;
    f0 = fw[P >> 5];
    f1 = fw[(P >> 5) + 1];
    f2 = RW > 32 ? fw[(P >> 5) + 2] : 0u;
  };
  // q of a corrupt segment can exceed what q << w holds only when the segment is that long
  const bool check_q = nW32 > (0xFFFFFFFFu >> 15) / 32u;
  // segments longer than kPos16Words words (q beyond 16-bit positions: a tiny step at a small k,
  // or a corrupt stream): the table holds 32-bit positions of half the chunk's symbols at a time
  const bool wide = nW32 > kPos16Words;  // uniform
  auto do_round = [&](int r) {
    const uint32_t tc = (uint32_t)TI::TPR * r + (uint32_t)TI::TPW * wave + tw;
    const bool valid = tc < tiles_c;
    const uint64_t t = (uint64_t)c * TI::CT + tc;
    const uint32_t rec = tc * F;
    const uint32_t P = rec + hdr + (uint32_t)o * (uint32_t)RW;
    const uint32_t a0 = hA, a1 = hB, a2w = hC, x0 = f0, x1 = f1, x2 = f2;
    if (r < 3) issue(r + 1);
    float yv[8];
    // a tile past the chunk's end is decoded like the others from what lies in its record's place
    // (inside the stream: every chunk has room for all its tiles) and dropped at the store; the
    // matrix-vector product needs its zeros
    if (!GEMV || valid) {
      // the 32 bits at rec are the scale (low half) and, for E8 with at most 16 octets, the
      // coset bits of the tile's octets (high half)
      const uint32_t th = __builtin_amdgcn_alignbit(a1, a0, rec & 31u);
      const uint32_t sb = th & 0xFFFFu;
      const uint32_t coset = kCosetWord      ? (a2w >> ((rec + 16u + cbit) & 31u)) & (LAT == kLatA2 ? 0xFu : 1u)
                             : LAT == kLatE8 ? (th >> (16 + o)) & 1u
                                             : 0u;
      const uint32_t sh = P & 31u;
      const uint32_t lo = __builtin_amdgcn_alignbit(x1, x0, sh), hi = __builtin_amdgcn_alignbit(x2, x1, sh);
      // unary parts: q = p - p_prev - 1 = (p_prev ^ ~0) + p; the symbol before the chunk's first
      // sits at -1
      const uint32_t g0 = ((uint32_t)LPT * tc + (uint32_t)o) * 8u;  // symbol index of slot 0: tc TL + 8 o
      uint32_t pprev, pp[8];
      if (!wide) {
        // the octet's eight 16-bit positions in one 16-byte read (the asm keeps it whole: split into
        // narrower pieces the reads conflict in more banks)
        const uint16_t* t16 = reinterpret_cast<const uint16_t*>(s_pos);
        const uint32_t pv = t16[g0 ? g0 - 1 : 0];
        pprev = g0 ? pv : 0xFFFFFFFFu;
        hq_u4 pw = *reinterpret_cast<const hq_u4*>(t16 + g0);
        __asm__ volatile("" : "+v"(pw));
        pp[0] = pw.x & 0xFFFFu; pp[1] = pw.x >> 16; pp[2] = pw.y & 0xFFFFu; pp[3] = pw.y >> 16;
        pp[4] = pw.z & 0xFFFFu; pp[5] = pw.z >> 16; pp[6] = pw.w & 0xFFFFu; pp[7] = pw.w >> 16;
      } else {
        // 32-bit entries of the current half of the chunk's symbols (rounds 0-1: [0, 4096), 2-3:
        // [4096, 8192)); the terminator before the second half is in *s_boundary
        const uint32_t gl = g0 - (r >= 2 ? kPosHalf : 0u);
        const uint32_t pv = gl ? s_pos[gl - 1] : *s_boundary;
        pprev = g0 ? pv : 0xFFFFFFFFu;
        hq_u4 pa = *reinterpret_cast<const hq_u4*>(s_pos + gl);
        hq_u4 pb = *reinterpret_cast<const hq_u4*>(s_pos + gl + 4);
        __asm__ volatile("" : "+v"(pa), "+v"(pb));
        pp[0] = pa.x; pp[1] = pa.y; pp[2] = pa.z; pp[3] = pa.w;
        pp[4] = pb.x; pp[5] = pb.y; pp[6] = pb.z; pp[7] = pb.w;
      }
      uint32_t q[8];
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        q[sl] = (pprev ^ 0xFFFFFFFFu) + pp[sl];
        pprev = pp[sl];
      }
      // q << w can only lose bits in a segment that long (uniform, and rare: the branch is skipped)
      if (__builtin_expect(check_q, 0) && valid) {
#pragma unroll
        for (int sl = 0; sl < 8; ++sl)
          if (q[sl] > (0xFFFFFFFFu >> slot_width<LAT>(sl, k))) bad = true;
      }
      uint32_t sym[8];
      if (RW <= 32) {  // uniform: every slot is one bit-field extract of lo
        int off = 0;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int w = slot_width<LAT>(sl, k);
          sym[sl] = (q[sl] << w) | __builtin_amdgcn_ubfe(lo, (uint32_t)off, (uint32_t)w);
          off += w;
        }
      } else if (k <= 8) {
        int off = 0;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int w = slot_width<LAT>(sl, k);
          sym[sl] = (q[sl] << w) | field_slot(lo, hi, off, w);
          off += w;
        }
      } else {
        uint32_t pos = P;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int w = slot_width<LAT>(sl, k);
          sym[sl] = (q[sl] << w) | plane_bits(fw, pos, w);
          pos += (uint32_t)w;
        }
      }
      const float tsc = bf16_bits_to_f32(sb) * step;
      if (LAT == kLatE8) {
        // z_i = 2 u_i + p for i < 7; the parity of u_0 + .. + u_6 is bit 1 of z_0 ^ .. ^ z_6;
        // z_7 = 2 (2 unzz(s_7) + par) + p
        int32_t z[8];
        uint32_t xz = 0;
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          z[i] = twice_unzz(sym[i]) + (int32_t)coset;
          xz ^= (uint32_t)z[i];
        }
        z[7] = 2 * twice_unzz(sym[7]) + (int32_t)((xz & 2u) | coset);
        if (dither) {
          float u[8];
          dither_octet<LAT>(seed, t, o, df, u);
#pragma unroll
          // z / 2 is exact, so the fused form rounds the difference once, as z / 2 - u does
          for (int i = 0; i < 8; ++i) yv[i] = __builtin_fmaf((float)z[i], 0.5f, -u[i]) * tsc;
        } else {
          // (z / 2) * tsc equals z * (tsc / 2): both are the same real product rounded once
          const float f = tsc * 0.5f;
#pragma unroll
          for (int i = 0; i < 8; ++i) yv[i] = (float)z[i] * f;
        }
      } else if (LAT == kLatA2) {
        // odd slots: the stretched coordinate, reconstructed with (s * step) * sqrt3
        int32_t code[8];
        unstrip_octet<LAT>(sym, coset, code);
        const float tsc1 = tsc * __uint_as_float(kA2R3Bits);
        float u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (dither) dither_octet<LAT>(seed, t, o, df, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float cc = code_coord<LAT>(code[i]);
          yv[i] = (dither ? cc - u[i] : cc) * ((i & 1) ? tsc1 : tsc);
        }
      } else {
        int32_t code[8];
        unstrip_octet<LAT>(sym, coset, code);
        if (dither) {
          float u[8];
          dither_octet<LAT>(seed, t, o, df, u);
#pragma unroll
          for (int i = 0; i < 8; ++i) yv[i] = (code_coord<LAT>(code[i]) - u[i]) * tsc;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) yv[i] = (float)code[i] * tsc;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[i] = 0.0f;
    }
    if constexpr (GEMV) {
      // the tile's share of its row: <yhat, x~_j> / TL (the lane's butterfly sign plays no part:
      // yhat is not transformed here); the octet partial is a fixed-order chain, the tile sum a
      // fixed xor tree
      const uint32_t j = (uint32_t)(t % (g.cols / TL));
      const float4* xp = reinterpret_cast<const float4*>(g.xt + (uint64_t)j * TL + 8 * o);
      const float4 a = valid ? xp[0] : make_float4(0, 0, 0, 0), b = valid ? xp[1] : make_float4(0, 0, 0, 0);
      float part = yv[0] * a.x;
      part = __builtin_fmaf(yv[1], a.y, part);
      part = __builtin_fmaf(yv[2], a.z, part);
      part = __builtin_fmaf(yv[3], a.w, part);
      part = __builtin_fmaf(yv[4], b.x, part);
      part = __builtin_fmaf(yv[5], b.y, part);
      part = __builtin_fmaf(yv[6], b.z, part);
      part = __builtin_fmaf(yv[7], b.w, part);
      part = part + lane_xor<1>(part);
      part = part + lane_xor<2>(part);
      part = part + lane_xor<4>(part);
      if (LPT >= 16) part = part + lane_xor<8>(part);
      if (LPT >= 32) part = part + lane_xor<16>(part);
      if (valid && o == 0) g.tp[t] = part * kInvTile;
      return;
    }
    fwht_lane(yv);
    // the table's address is made opaque per round so that its entries are read here, not kept
    uint32_t fo = 3u * (uint32_t)o;
    __asm__ volatile("" : "+v"(fo));
    const float4 c0 = s_fac[fo], c1 = s_fac[fo + 1], sg4 = s_fac[fo + 2];
    const float sg[5] = {sg4.x, sg4.y, sg4.z, sg4.w, (o & 16) ? -1.0f : 1.0f};
    fwht_cross_s<LPT>(yv, sg);
    if (valid) {
      const float cmul[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      float xo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xo[i] = __builtin_fmaf(yv[i], cmul[i], 0.0f);
      if (DT_OUT == 1) {
        hq_b2 pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = __builtin_convertvector((hq_f2){xo[2 * i], xo[2 * i + 1]}, hq_b2);
        uint4 st;
        st.x = __builtin_bit_cast(uint32_t, pk[0]);
        st.y = __builtin_bit_cast(uint32_t, pk[1]);
        st.z = __builtin_bit_cast(uint32_t, pk[2]);
        st.w = __builtin_bit_cast(uint32_t, pk[3]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + t * TL + 8 * o) = st;
      } else {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + t * TL + 8 * o);
        dst[0] = make_float4(xo[0], xo[1], xo[2], xo[3]);
        dst[1] = make_float4(xo[4], xo[5], xo[6], xo[7]);
      }
    }
    };
  // the first round's record words are in flight while the positions are found
  issue(0);
  const uint32_t nsym = tiles_c * (uint32_t)TL;
  if (!(wide ? unary_positions<1>(seg, nW32, nsym, s_pos, s_boundary, ws, call)
              : unary_positions<0>(seg, nW32, nsym, s_pos, s_boundary, ws, call)))
    return;
  do_round(0);
  do_round(1);
  if (wide) {
    __syncthreads();  // every read of the first half is done before the table is rewritten
    if (!unary_positions<2>(seg, nW32, nsym, s_pos, s_boundary, ws, call)) return;
  }
  do_round(2);
  do_round(3);
  if (bad) record_error(ws, call, kErrCorrupt);
}

// One workgroup per chunk.  A plain decode validates the stream header in every workgroup (scalar
// loads of 128 bytes; workgroup 0 numbers the workspace with the call), a matrix product takes the
// fields its rotation kernel checked and published.  Then the chunk's index entries are checked,
// and decode_chunk of the stream's lattice and tile length finds the terminator positions
// (unary_positions) and decodes the tiles.
template <int DT_OUT, bool GEMV>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(7, 8))) void decode_kernel(
    const uint8_t* __restrict__ in, uint64_t in_bytes, uint64_t n, void* __restrict__ out, Workspace* ws,
    GemvArgs gv, uint64_t call) {
  // 16 KiB of terminator positions (8192 16-bit or 4096 32-bit entries) and the boundary word: the
  // register budget of seven waves per SIMD, not LDS, sets the occupancy (72 registers and a few
  // words of spill; measured faster than six waves without the spill: 57.5 -> 54.9 us on the
  // weight's stream)
  __shared__ uint4 s_pos4[kMaxSymsPerChunk / 8];
  __shared__ uint32_t s_boundary;
  __shared__ float4 s_fac[3 * 32];  // per octet index: 8 output factors, 4 butterfly signs
  uint32_t* s_pos = reinterpret_cast<uint32_t*>(s_pos4);
  const int tid = threadIdx.x;
  const uint32_t c = blockIdx.x;
  // a chunk holds kChunkValues values at every tile length, so n gives the chunk count: while the
  // header is in flight the chunk's index entries can be requested too (when the stream is long
  // enough to hold the index at all)
  const uint32_t chunks_n = (uint32_t)((n + kChunkValues - 1) / kChunkValues);
  const uint32_t* idx = reinterpret_cast<const uint32_t*>(in + kHeaderBytes);
  const bool idx_in = in_bytes >= (uint64_t)kHeaderBytes + 4ull * ((uint64_t)chunks_n + 1) && c < chunks_n;
  const uint32_t w0 = idx_in ? idx[c] : 0u, w1 = idx_in ? idx[c + 1] : 0u;
  if (GEMV) {
    if (!ws->dec_valid) return;
  } else {
    DecInfo d;
    const bool ok = read_header(in, in_bytes, n, 0, &d);
    if (tid == 0) {
      if (c == 0) __hip_atomic_store(&ws->call, call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!ok) record_error(ws, call, kErrCorrupt);
    }
    if (!ok) return;
  }
  // the stream's fields, read again from its validated header (read-only, so the compiler may
  // reload them instead of keeping them in registers)
  const uint32_t* __restrict__ hw = reinterpret_cast<const uint32_t*>(in);
  const uint32_t chunks = hw[10];
  if (c >= chunks) return;
  const uint64_t T = ((uint64_t)hw[9] << 32) | hw[8];
  const uint32_t tile = hw[2] & 0xFFFFu;
  const uint32_t lattice = (hw[1] >> 16) & 0xFFu;
  const int hk = (int)((hw[2] >> 16) & 0xFFu);
  const uint64_t words = ((uint64_t)hw[17] << 32) | hw[16];
  const uint64_t unary_off = ((uint64_t)hw[15] << 32) | hw[14];
  const uint32_t ct = (uint32_t)kChunkValues / tile;
  const uint32_t tiles_c = (uint32_t)min((uint64_t)ct, T - (uint64_t)c * ct);
  if (w1 < w0 || (uint64_t)w1 > words || (uint64_t)(w1 - w0) * 64ull > 0xFFFFFFFFull) {
    if (tid == 0) record_error(ws, call, kErrCorrupt);
    return;
  }
  const uint32_t* __restrict__ seg = reinterpret_cast<const uint32_t*>(in + unary_off + 8ull * w0);
  const uint32_t nW32 = 2u * (w1 - w0);
  // uniform dispatch on the stream's lattice and tile length
#define HQ_DEC_ARGS in, out, ws, call, c, tiles_c, seg, nW32, s_pos, &s_boundary, s_fac, gv
#define HQ_DEC_LAT(TLV)                                                                  \
  switch (lattice) {                                                                     \
    case kLatE8: decode_chunk_body<kLatE8, DT_OUT, GEMV, TLV>(HQ_DEC_ARGS); break;       \
    case kLatA2: decode_chunk_body<kLatA2, DT_OUT, GEMV, TLV>(HQ_DEC_ARGS); break;       \
    case kLatD4: decode_chunk_body<kLatD4, DT_OUT, GEMV, TLV>(HQ_DEC_ARGS); break;       \
    default: decode_chunk_body<kLatZ, DT_OUT, GEMV, TLV>(HQ_DEC_ARGS); break;            \
  }
  if (tile == 128u && lattice == kLatE8 && hk <= 3) {
    switch (hk) {
      case 0: decode_chunk_body<kLatE8, DT_OUT, GEMV, 128, 0>(HQ_DEC_ARGS); break;
      case 1: decode_chunk_body<kLatE8, DT_OUT, GEMV, 128, 1>(HQ_DEC_ARGS); break;
      case 2: decode_chunk_body<kLatE8, DT_OUT, GEMV, 128, 2>(HQ_DEC_ARGS); break;
      default: decode_chunk_body<kLatE8, DT_OUT, GEMV, 128, 3>(HQ_DEC_ARGS); break;
    }
  } else if (tile == 64u) {
    HQ_DEC_LAT(64)
  } else if (tile == 256u) {
    HQ_DEC_LAT(256)
  } else {
    HQ_DEC_LAT(128)
  }
#undef HQ_DEC_LAT
#undef HQ_DEC_ARGS
}

// ---------------------------------------------------------------------------------------------
// Fused decode + matrix-vector product.  For a stream of a [rows][cols] matrix (tiles of TL values
// along cols), tile (r, j) decodes to D H yhat / TL, so its dot product with the activation's tile
// x_j is <yhat, H D x_j> / TL (H is symmetric, D diagonal): rotate each activation tile once, then
// every matrix tile needs only its lattice values, no inverse transform.

// x~_j = H D x_j for every column tile, binary32 in the encoder's butterfly order, stored with the
// lanes' butterfly signs removed (an exact negation).  Every workgroup checks the stream header
// itself (the seed of D and the tile length come from it), and workgroup 0 also publishes the
// check for the decode that follows, so no separate check launch is needed.  A workgroup covers
// 2048 columns at every tile length.
template <int DT, int TL>
__device__ __forceinline__ void gemv_rotate_tiles(const void* __restrict__ x, uint64_t cols, uint64_t seed,
                                                  float* __restrict__ xt) {
  using TI = Tiling<TL>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, o = lane % TI::LPT, tw = lane / TI::LPT;
  const uint64_t t = (uint64_t)blockIdx.x * TI::TPR + TI::TPW * wave + tw;
  const bool valid = t < cols / TL;
  const uint32_t sgn = octet_sign_bits(seed, o);
  uint32_t smask[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) smask[i] = ((sgn >> i) & 1u) << 31;
  float y[8];
  if (valid) {
    load_octet_signed<DT, TL>(x, t, o, smask, y);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.0f;
  }
  fwht_lane(y);
  fwht_cross<TI::LPT>(y, o);
  if (!valid) return;
  const uint32_t neg = lane_sign_bit<TI::LPT>(o) << 31;
  float4* dst = reinterpret_cast<float4*>(xt + t * TL + 8 * o);
  dst[0] = make_float4(__uint_as_float(__float_as_uint(y[0]) ^ neg), __uint_as_float(__float_as_uint(y[1]) ^ neg),
                       __uint_as_float(__float_as_uint(y[2]) ^ neg), __uint_as_float(__float_as_uint(y[3]) ^ neg));
  dst[1] = make_float4(__uint_as_float(__float_as_uint(y[4]) ^ neg), __uint_as_float(__float_as_uint(y[5]) ^ neg),
                       __uint_as_float(__float_as_uint(y[6]) ^ neg), __uint_as_float(__float_as_uint(y[7]) ^ neg));
}

template <int DT>
__global__ __launch_bounds__(kBlock) void gemv_rotate_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes,
                                                             uint64_t n, const void* __restrict__ x, uint64_t cols,
                                                             Workspace* ws, float* __restrict__ xt, uint64_t call) {
  DecInfo d;
  if (!check_header(in, in_bytes, n, cols, ws, blockIdx.x == 0, call, &d)) return;
  if (d.tile == 64u)
    gemv_rotate_tiles<DT, 64>(x, cols, d.seed, xt);
  else if (d.tile == 256u)
    gemv_rotate_tiles<DT, 256>(x, cols, d.seed, xt);
  else
    gemv_rotate_tiles<DT, 128>(x, cols, d.seed, xt);
}

// y_r = sum over the row's column tiles of the tile partials, in column order (one lane per row).
__global__ __launch_bounds__(kBlock) void gemv_rows_kernel(const float* __restrict__ tp, uint64_t rows,
                                                           uint64_t cols, const Workspace* ws, float* __restrict__ y) {
  if (!ws->dec_valid) return;
  const uint64_t r = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (r >= rows) return;
  const uint32_t ctiles = (uint32_t)(cols / ws->dec_tile);
  const float* p = tp + r * ctiles;
  float acc = 0.0f;
  for (uint32_t j = 0; j < ctiles; ++j) acc += p[j];
  y[r] = acc;
}

// ---------------------------------------------------------------------------------------------
// Launchers.

// Compile-time variants: lattice x dither x input type x tile length.
#define HQ_DISPATCH_TL(L, D, T, TLV, CALL) \
  do {                                     \
    if ((TLV) == 64) CALL(L, D, T, 64);    \
    else if ((TLV) == 256) CALL(L, D, T, 256); \
    else CALL(L, D, T, 128);               \
  } while (0)
#define HQ_DISPATCH_DT(L, D, DTV, TLV, CALL)                       \
  do {                                                             \
    if ((DTV) == 1) HQ_DISPATCH_TL(L, D, 1, TLV, CALL);            \
    else HQ_DISPATCH_TL(L, D, 0, TLV, CALL);                       \
  } while (0)
#define HQ_DISPATCH_D(L, DITHV, DTV, TLV, CALL)                    \
  do {                                                             \
    if (DITHV) HQ_DISPATCH_DT(L, true, DTV, TLV, CALL);            \
    else HQ_DISPATCH_DT(L, false, DTV, TLV, CALL);                 \
  } while (0)
#define HQ_DISPATCH(LATV, DITHV, DTV, TLV, CALL)                                      \
  do {                                                                                \
    if ((LATV) == kLatE8) HQ_DISPATCH_D(kLatE8, DITHV, DTV, TLV, CALL);               \
    else if ((LATV) == kLatA2) HQ_DISPATCH_D(kLatA2, DITHV, DTV, TLV, CALL);          \
    else if ((LATV) == kLatD4) HQ_DISPATCH_D(kLatD4, DITHV, DTV, TLV, CALL);          \
    else HQ_DISPATCH_D(kLatZ, DITHV, DTV, TLV, CALL);                                 \
  } while (0)

hipError_t launch_init(const EncodeArgs& a, int64_t centre, int mode) {
  const uint64_t nflags = (uint64_t)a.chunks + 1;
  const uint32_t nacc = (uint32_t)(kWsRate / sizeof(uint32_t));
  const uint64_t work = nflags > nacc ? nflags : nacc;
  uint64_t blocks = (work + kBlock - 1) / kBlock;
  if (blocks > 1024) blocks = 1024;
  uint32_t step_bits = 0;
  int32_t k = 0;
  if (mode == kInitKeep) {
    // the kernel takes the workspace's point
  } else if (a.fixed_step_bits) {
    step_bits = a.fixed_step_bits;
    k = a.rice_k >= 0 ? a.rice_k : kwin_base(a.fixed_step_bits) + 1;
  } else {
    const int64_t c = centre < kStepBitsMin ? kStepBitsMin : (centre > kStepBitsMax ? kStepBitsMax : centre);
    step_bits = (uint32_t)c;
    k = a.rice_k >= 0 ? a.rice_k : kwin_base(centre) + 1;
  }
  hipLaunchKernelGGL(init_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, a.stream, a.ws, lookback_flags(a.ws),
                     nflags, reinterpret_cast<uint32_t*>(rate_acc(a.ws, 0)), nacc, centre, step_bits, k, mode, a.call);
  return hipGetLastError();
}

static PassDesc pass_desc(const EncodeArgs& a, int pass, int nc, int half_log2, uint32_t N, uint32_t nblk) {
  PassDesc d;
  d.racc = rate_acc(a.ws, pass);
  d.nc = nc;
  d.half_log2 = half_log2;
  d.fixed_k = a.rice_k;
  d.target = a.target;
  d.N = N;
  d.nblk = nblk;
  return d;
}

static RateArgs rate_args(const EncodeArgs& a, const RatePlan& rp) {
  RateArgs r;
  r.x = a.x;
  r.T = a.tiles;
  r.seed = a.seed;
  r.df = (uint32_t)a.dither;
  r.ws = a.ws;
  r.pub = rate_pub(a.ws);
  r.two_pass = rp.two_pass;
  r.pa = pass_desc(a, 0, kRcCand, 21, rp.two_pass ? rp.NA : 0u, rp.two_pass ? rp.blkA : 0u);
  r.pb = rp.two_pass ? pass_desc(a, 1, kRcCandB, 18, rp.NB, rp.blkB) : pass_desc(a, 1, 1, 0, rp.NB, rp.blkB);
  r.centre0 = rp.centre0;
  r.nblk = r.pa.nblk + r.pb.nblk;
  r.spin_budget = a.spin_budget;
  r.call = a.call;
  return r;
}

hipError_t launch_rate(const EncodeArgs& a, const RatePlan& rp) {
  if (!rp.needed) return hipSuccess;
  const RateArgs r = rate_args(a, rp);
#define HQ_RATE(L, D, T, TL) \
  hipLaunchKernelGGL((rate_kernel<L, D, T, TL>), dim3(r.nblk), dim3(kBlock), 0, a.stream, r)
  HQ_DISPATCH(a.lattice, a.dither, a.dtype, a.tile, HQ_RATE);
#undef HQ_RATE
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a) {
  EncParams P;
  P.x = a.x;
  P.n = a.n;
  P.T = a.tiles;
  P.chunks = a.chunks;
  P.seed = a.seed;
  P.dflags = (uint32_t)a.dither;
  P.out = a.out;
  P.cap = a.cap;
  P.ws = a.ws;
  P.flags = lookback_flags(a.ws);
  P.spin_budget = a.spin_budget;
  P.call = a.call;
  const uint32_t blocks = a.chunks ? a.chunks : 1u;
#define HQ_ENC(L, D, T, TL) \
  hipLaunchKernelGGL((encode_kernel<L, D, T, TL>), dim3(blocks), dim3(kBlock), 0, a.stream, P)
  HQ_DISPATCH(a.lattice, a.dither, a.dtype, a.tile, HQ_ENC);
#undef HQ_ENC
  return hipGetLastError();
}

hipError_t launch_codes(const EncodeArgs& a, int32_t* codes, uint16_t* scales) {
  const uint64_t tpr = 4u * (64u / ((uint32_t)a.tile / 8u));  // tiles per workgroup
  const uint64_t blocks = (a.tiles + tpr - 1) / tpr;
  if (blocks == 0) return hipSuccess;
#define HQ_CODES(L, D, T, TL)                                                                          \
  hipLaunchKernelGGL((codes_kernel<L, D, T, TL>), dim3((uint32_t)blocks), dim3(kBlock), 0, a.stream, a.x, a.tiles, \
                     a.seed, (uint32_t)a.dither, a.fixed_step_bits, codes, scales, a.ws, a.call)
  HQ_DISPATCH(a.lattice, a.dither, a.dtype, a.tile, HQ_CODES);
#undef HQ_CODES
  return hipGetLastError();
}

hipError_t launch_decode(const uint8_t* in, uint64_t in_bytes, void* out, int out_dtype, uint64_t n,
                         Workspace* ws, uint64_t call, hipStream_t stream) {
  // a chunk holds kChunkValues values at every tile length (the header check rejects an n that
  // is not a whole number of the stream's tiles); an empty tensor still gets the header check
  const uint64_t chunks = (n + kChunkValues - 1) / kChunkValues;
  const uint32_t blocks = chunks ? (uint32_t)chunks : 1u;
  const GemvArgs none{nullptr, 128u, nullptr};
  if (out_dtype == 1)
    hipLaunchKernelGGL((decode_kernel<1, false>), dim3(blocks), dim3(kBlock), 0, stream, in, in_bytes, n, out, ws,
                       none, call);
  else
    hipLaunchKernelGGL((decode_kernel<0, false>), dim3(blocks), dim3(kBlock), 0, stream, in, in_bytes, n, out, ws,
                       none, call);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* in, uint64_t in_bytes, uint64_t rows, uint64_t cols, const void* x, int x_dtype,
                       float* y, Workspace* ws, float* xt, float* tp, uint64_t call, hipStream_t stream) {
  const uint64_t n = rows * cols;
  if (n == 0) {  // nothing to multiply (x may then be null): check the stream only
    hipLaunchKernelGGL(decode_check_kernel, dim3(1), dim3(64), 0, stream, in, in_bytes, n, ws, call);
    return hipGetLastError();
  }
  // the rotation kernel also checks the header (its workgroup 0 publishes the check)
  const uint32_t rblocks = (uint32_t)((cols + 2047) / 2048);
  if (x_dtype == 1)
    hipLaunchKernelGGL(gemv_rotate_kernel<1>, dim3(rblocks), dim3(kBlock), 0, stream, in, in_bytes, n, x, cols, ws, xt,
                       call);
  else
    hipLaunchKernelGGL(gemv_rotate_kernel<0>, dim3(rblocks), dim3(kBlock), 0, stream, in, in_bytes, n, x, cols, ws, xt,
                       call);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t chunks = (n + kChunkValues - 1) / kChunkValues;
  if (chunks == 0) return hipSuccess;
  const GemvArgs g{xt, cols, tp};
  hipLaunchKernelGGL((decode_kernel<1, true>), dim3((uint32_t)chunks), dim3(kBlock), 0, stream, in, in_bytes, n,
                     nullptr, ws, g, call);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemv_rows_kernel, dim3((uint32_t)((rows + kBlock - 1) / kBlock)), dim3(kBlock), 0, stream, tp,
                     rows, cols, ws, y);
  return hipGetLastError();
}

}  // namespace hq
