// hq_internal.h -- workspace layout and kernel launchers shared by hq_kernels.hip and hq_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

// Device-side error flags recorded in Workspace::err.  kErrNoPoint: an encode at the operating
// point left in the workspace (step == -1) found none there.
enum { kErrNonfinite = 1u, kErrCapacity = 2u, kErrCorrupt = 4u, kErrTimeout = 8u, kErrRange = 16u,
       kErrNoPoint = 32u };

// Workspace::point_tag holds this value while step_bits and rice_k are a complete operating point
// (the end of rate control, or a fixed step and Rice parameter); any other value means there is
// none.
constexpr uint32_t kPointTag = 0x54505148u;  // 'H' 'Q' 'P' 'T'

// Rate control (the pages ask for a realised rate within ~0.01 bits per value and give no
// algorithm; see hq_kernels.hip for the search).
constexpr uint32_t kRcSampleTiles = 8192;   // pass B (and a fixed step's Rice choice)
constexpr uint32_t kRcSampleTilesA = 2048;  // pass A
constexpr int kRcCand = 8;                  // pass A; the most a pass evaluates
constexpr int kRcCandB = 4;
constexpr int kRcKwin = 4;

// Device workspace.  The fixed part is 4 KiB; the encoder's look-back flags (one 64-bit word per
// chunk, plus one) follow it.  Every field is (re)initialised by the first kernel of a call.
struct alignas(256) Workspace {
  uint32_t pad2[3];
  uint32_t step_bits;    // operating point chosen so far (binary32 bits of the step)
  int32_t rice_k;
  uint32_t pad0;
  int64_t rc_centre;     // centre of the next rate pass (step bits)
  // encoder results, written by the chunk that finishes the look-back chain
  uint64_t res_total_bytes;
  uint64_t res_payload_bits;
  uint64_t res_unary_bits;
  uint64_t res_words;
  uint32_t res_step_bits;
  int32_t res_k;
  // decoder parameters, written by the header check
  uint32_t dec_valid;
  uint32_t dec_lattice;
  uint32_t dec_dither;
  int32_t dec_k;
  uint32_t dec_step_bits;
  uint32_t dec_F;
  uint32_t dec_chunks;
  uint32_t dec_tile;
  uint64_t dec_seed;
  uint64_t dec_tiles;
  uint64_t dec_fixed_off;
  uint64_t dec_unary_off;
  uint64_t dec_words;
  // kPointTag while step_bits / rice_k hold a complete operating point
  uint32_t point_tag;
  // Errors: err[b] holds the number of the last call that recorded error flag 1 << b, and `call`
  // the number of the call that last used the workspace (its kernels write it).  The flags of
  // that call are the bits b with err[b] == call, so no kernel has to clear anything first.  The
  // library numbers calls from a random 64-bit start.
  uint64_t call;
  uint64_t err[8];
  // Fallbacks, numbered the same way: slow[i] holds the number of the last call in which a bounded
  // wait of kind i ran out of its spin budget and its wavefront computed the awaited value itself
  // (the same result, later): kSlowLookback a look-back predecessor's aggregate, kSlowCentre pass
  // A's solve in a pass-B workgroup, kSlowPrivate a pass's sums evaluated by its solver alone.
  uint64_t slow[4];
};
static_assert(sizeof(Workspace) <= 4096, "workspace header");
enum { kSlowLookback = 0, kSlowCentre = 1, kSlowPrivate = 2 };
// The fallbacks the workspace's last call took (bit i: slow[i] holds that call's number).
inline uint32_t fallback_flags(const Workspace& h) {
  uint32_t f = 0;
  for (int i = 0; i < 3; ++i)
    if (h.slow[i] == h.call) f |= 1u << i;
  return f;
}
constexpr size_t kWsHeader = 4096;
// Counters of the two rate passes.  A workgroup of a pass adds its sums into one of kRcAccSlots
// counter sets (workgroup index mod kRcAccSlots, so that few workgroups share an address).  Each
// 64-bit word holds the sum of the contributions in bits 0-39 and their number in bits 40-63, so
// that the solver can tell from the word alone that every workgroup of the pass has added into it
// (relaxed agent-scope atomics suffice: no ordering between words is needed).  The init kernel of
// every call zeroes both passes' counters and the published words below.
constexpr int kRcAccSlots = 16;
constexpr int kRcCounters = kRcCand * kRcKwin;
constexpr int kCntShift = 40;
struct RateAcc {
  uint64_t cnt[kRcAccSlots][kRcCounters];
};
// Word in which rate workgroup 0 publishes pass A's solve, the centre of pass B, to pass B's
// workgroups (bit 63 set = published, the centre in the low 32 bits): kPubCopies copies,
// kPubStride words (256 bytes) apart, so that the waiting workgroups spread their polls over
// several addresses; and the count of pass B's workgroups that have added their sums, whose last
// solves pass B.
constexpr int kPubCopies = 16;
constexpr int kPubStride = 32;
struct RatePub {
  uint64_t centre[kPubCopies * kPubStride];
  uint64_t done_b[kPubStride];  // pass B's workgroups that have added their sums (word 0)
};
constexpr size_t kWsRate = 2 * sizeof(RateAcc) + sizeof(RatePub);  // pass A, pass B, published centre
static_assert(kWsRate % 256 == 0, "rate counters keep the flags 256-byte aligned");

inline RateAcc* rate_acc(void* ws, int pass) {
  return reinterpret_cast<RateAcc*>(reinterpret_cast<char*>(ws) + kWsHeader) + pass;
}
inline RatePub* rate_pub(void* ws) {
  return reinterpret_cast<RatePub*>(reinterpret_cast<char*>(ws) + kWsHeader + 2 * sizeof(RateAcc));
}
// the encoder's look-back flags follow the rate counters
inline uint64_t* lookback_flags(void* ws) {
  return reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + kWsHeader + kWsRate);
}

// Spin rounds a cross-workgroup wait makes before the waiting wavefront computes the awaited value
// itself (a look-back predecessor's aggregate from its input; pass A's solve from its counters).
// Far above any wait in normal operation; the environment variable HQ_SPIN_BUDGET overrides it (0
// makes every wait that finds its value missing compute it at once: the tests use that to run the
// fallback paths).
constexpr uint32_t kSpinBudget = 256;

struct EncodeArgs {
  const void* x;
  int dtype;
  uint64_t n, tiles;
  uint32_t chunks;
  int tile;            // values per tile: 64, 128 or 256
  int lattice;
  int dither;
  uint64_t seed;
  float target;
  int rice_k;          // -1 = automatic
  uint32_t fixed_step_bits;  // 0 = rate control
  uint8_t* out;
  uint64_t cap;
  Workspace* ws;
  hipStream_t stream;
  uint32_t spin_budget;
  uint64_t call;       // number of this call (see Workspace::err)
};

// Modes of the call's first kernel (see init_kernel): the operating point is provisional (rate
// workgroups follow), final, or kept from the workspace (an encode with step == -1).
enum { kInitProvisional = 0, kInitFinal = 1, kInitKeep = 2 };
hipError_t launch_init(const EncodeArgs& a, int64_t centre, int mode);

// Rate control of one call (see rate_workgroup in hq_kernels.hip): two passes (pass A: 8
// candidates around centre0 on NA sample tiles; pass B: 4 candidates around pass A's solve on NB
// tiles), or, for a fixed step with automatic k, one pass of the single candidate centre0 on NB
// tiles.  blkA workgroups run pass A and the next blkB pass B (blkA + blkB workgroups in all).
struct RatePlan {
  int needed;
  int two_pass;
  int64_t centre0;
  uint32_t NA, NB, blkA, blkB;
};
// Rate control: one launch of the rate workgroups, whose pass-B solver leaves the operating point
// in the workspace (nothing when rp.needed is 0).
hipError_t launch_rate(const EncodeArgs& a, const RatePlan& rp);
// The encoder, at the operating point the workspace holds.
hipError_t launch_encode(const EncodeArgs& a);
hipError_t launch_decode(const uint8_t* in, uint64_t in_bytes, void* out, int out_dtype, uint64_t n,
                         Workspace* ws, uint64_t call, hipStream_t stream);
hipError_t launch_codes(const EncodeArgs& a, int32_t* codes, uint16_t* scales);
hipError_t launch_gemv(const uint8_t* in, uint64_t in_bytes, uint64_t rows, uint64_t cols, const void* x, int x_dtype,
                       float* y, Workspace* ws, float* xt, float* tp, uint64_t call, hipStream_t stream);

// The error flags that the workspace's last call recorded (host copy of the workspace header).
inline uint32_t error_flags(const Workspace& h) {
  uint32_t f = 0;
  for (int b = 0; b < 8; ++b)
    if (h.err[b] == h.call) f |= 1u << b;
  return f;
}

}  // namespace hq
