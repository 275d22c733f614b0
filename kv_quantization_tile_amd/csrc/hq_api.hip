// hq_api.hip -- C ABI of the codec (declarations and contracts in include/hq.h).
//
// Host side only: argument validation, the order of kernel launches on the caller's stream and
// the read-back of results.  Every step of the method runs in the kernels of hq_kernels.hip.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <random>

#include "../../include/hq.h"
#include "hq_internal.h"

using namespace hq;

namespace {

constexpr uint32_t kFormatVersion = 1;
constexpr uint32_t kStepMin = (127u - 12u) << 23, kStepMax = (127u + 12u) << 23;

uint32_t f32_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

uint64_t align256h(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

int octet_rem_bits_h(int lattice, int k) {
  const int kh = k > 0 ? k - 1 : 0;
  return lattice == HQ_E8 ? 7 * k + kh : lattice == HQ_D4 ? 6 * k + 2 * kh : lattice == HQ_A2 ? 4 * k + 4 * kh : 8 * k;
}
// Fixed bits of a tile record: 16 scale bits, the coset bits (E8: one per octet; A2: one per pair)
// and the remainders of tile / 8 octets.
uint32_t tile_fixed_bits_h(int lattice, int k, uint32_t tile) {
  const uint32_t oct = tile / 8u;
  return 16u + (lattice == HQ_E8 ? oct : lattice == HQ_A2 ? 4u * oct : 0u) + oct * (uint32_t)octet_rem_bits_h(lattice, k);
}
bool valid_tile(uint32_t tile) { return tile == 64u || tile == 128u || tile == 256u; }

// Lowest payload rate a lattice reaches: one unary bit per value plus its raw coset bits.
float min_bps(int lattice) { return lattice == HQ_E8 ? 1.125f : lattice == HQ_A2 ? 1.5f : 1.0f; }

// A chunk holds 8192 values at every tile length (8192 / tile tiles).
uint64_t chunks_of(uint64_t n) { return (n + 8191) / 8192; }

int check_params(const hq_params* p, uint64_t n) {
  if (!p) return HQ_ERR_INVALID_ARG;
  if (!valid_tile(p->tile)) return HQ_ERR_UNSUPPORTED;
  if (p->lattice < HQ_Z || p->lattice > HQ_A2) return HQ_ERR_INVALID_ARG;
  if (n % p->tile) return HQ_ERR_INVALID_ARG;
  if (n > (1ull << 35)) return HQ_ERR_INVALID_ARG;  // the encoder's look-back packs 28-bit padding sums
  if (p->dither > 7 || (p->dither > 1 && !(p->dither & 1))) return HQ_ERR_INVALID_ARG;  // dither flags
  if (p->rice_k < -1 || p->rice_k > 15) return HQ_ERR_INVALID_ARG;
  if (p->step == -1.0f) return HQ_OK;  // operating point left in the workspace by hq_rate
  if (!(p->step >= 0.0f)) return HQ_ERR_INVALID_ARG;  // also rejects NaN
  if (p->step > 0.0f) {
    const uint32_t b = f32_bits(p->step);
    if (b < kStepMin || b > kStepMax) return HQ_ERR_INVALID_ARG;
  } else {
    if (!(p->target_bps >= min_bps(p->lattice)) || !(p->target_bps <= 12.0f)) return HQ_ERR_RATE;
  }
  return HQ_OK;
}

int status_from_flags(uint32_t f) {
  if (f & kErrNoPoint) return HQ_ERR_INVALID_ARG;  // the root cause of whatever else that call saw
  if (f & kErrCorrupt) return HQ_ERR_CORRUPT;
  if (f & kErrNonfinite) return HQ_ERR_NONFINITE;
  if (f & kErrCapacity) return HQ_ERR_CAPACITY;
  if (f & kErrRange) return HQ_ERR_UNSUPPORTED;
  if (f & kErrTimeout) return HQ_ERR_TIMEOUT;
  return HQ_OK;
}

size_t workspace_bytes_for(uint64_t n) { return kWsHeader + kWsRate + align256h(8ull * (chunks_of(n) + 1)); }

// Numbers of calls (see Workspace::err): consecutive from a random 64-bit start, so that a
// workspace's earlier contents never carry the number of a new call.
std::atomic<uint64_t> g_next_call{0};
std::once_flag g_call_once;
uint64_t next_call() {
  std::call_once(g_call_once, [] {
    std::random_device rd;
    const uint64_t r = ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^
                       (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    g_next_call.store(r | 1u);
  });
  return g_next_call.fetch_add(1);
}

uint32_t spin_budget() {
  const char* e = getenv("HQ_SPIN_BUDGET");
  if (!e || !*e) return kSpinBudget;
  const unsigned long v = strtoul(e, nullptr, 10);
  return v > 0xFFFFFFFFul ? 0xFFFFFFFFu : (uint32_t)v;
}

EncodeArgs make_args(const void* x, int dtype, uint64_t n, const hq_params* p, void* out, uint64_t cap,
                     void* ws, hq_stream_t s) {
  EncodeArgs a;
  a.x = x;
  a.dtype = dtype;
  a.n = n;
  a.tile = (int)p->tile;
  a.tiles = n / p->tile;
  a.chunks = (uint32_t)chunks_of(n);
  a.lattice = p->lattice;
  a.dither = (int)p->dither;
  a.seed = p->seed;
  a.target = p->target_bps;
  a.rice_k = p->rice_k;
  a.fixed_step_bits = p->step > 0.0f ? f32_bits(p->step) : 0u;  // 0 also for step == -1
  a.out = static_cast<uint8_t*>(out);
  a.cap = cap;
  a.ws = static_cast<Workspace*>(ws);
  a.stream = static_cast<hipStream_t>(s);
  a.spin_budget = spin_budget();
  a.call = next_call();
  return a;
}

// Initial centre of the rate search: the Gaussian high-rate guess log2(step) = 2.05 - target,
// as a binary32 bit pattern.
int64_t initial_centre(float target) {
  return (int64_t)(127u << 23) + (int64_t)floor((2.05 - (double)target) * 8388608.0 + 0.5);
}

// The rate control of a call (see RatePlan): for rate control proper (step == 0) two passes around
// the Gaussian guess; for a fixed step with automatic k one pass at that step; none otherwise (or
// for an empty tensor).  Pass A samples min(T, 2048) tiles, pass B min(T, 8192).
RatePlan plan_rate(const EncodeArgs& a) {
  RatePlan rp{};
  const uint64_t T = a.tiles;
  const uint32_t N = (uint32_t)(T < kRcSampleTiles ? T : kRcSampleTiles);
  const uint32_t NA = (uint32_t)(T < kRcSampleTilesA ? T : kRcSampleTilesA);
  const uint32_t tpw = 64u / ((uint32_t)a.tile / 8u);  // sample tiles per wavefront
  if (a.fixed_step_bits) {
    rp.needed = a.rice_k < 0 && N > 0;
    rp.two_pass = 0;
    rp.centre0 = (int64_t)a.fixed_step_bits;
  } else {
    rp.needed = N > 0;
    rp.two_pass = 1;
    rp.centre0 = initial_centre(a.target);
  }
  if (!rp.needed) return rp;
  rp.NB = N;
  rp.blkB = (N + 4u * tpw - 1u) / (4u * tpw);
  if (rp.two_pass) {
    rp.NA = NA;
    rp.blkA = (NA + tpw - 1u) / tpw;
  }
  return rp;
}

// The call's first kernel: it resets the workspace, with the operating point final (no rate
// control follows) or provisional (the rate workgroups of rp will set it).
int start_call(const EncodeArgs& a, const RatePlan& rp) {
  const int64_t centre = a.fixed_step_bits ? (int64_t)a.fixed_step_bits : initial_centre(a.target);
  return launch_init(a, centre, rp.needed ? kInitProvisional : kInitFinal) == hipSuccess ? HQ_OK : HQ_ERR_HIP;
}

struct Results {
  uint32_t status, step_bits;
  int32_t k;
  uint64_t total_bytes, payload_bits;
};

int read_results(void* ws, hipStream_t s, Results* r) {
  Workspace h;
  if (hipMemcpyAsync(&h, ws, sizeof(Workspace), hipMemcpyDeviceToHost, s) != hipSuccess) return HQ_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return HQ_ERR_HIP;
  r->status = error_flags(h);
  r->step_bits = h.res_step_bits;
  r->k = h.res_k;
  r->total_bytes = h.res_total_bytes;
  r->payload_bits = h.res_payload_bits;
  return HQ_OK;
}

void fill_info(hq_info* info, uint64_t n, uint32_t step_bits, int k, uint64_t bytes, uint64_t payload_bits) {
  if (!info) return;
  float st;
  memcpy(&st, &step_bits, 4);
  info->step = st;
  info->rice_k = k;
  info->bytes = bytes;
  info->payload_bits = payload_bits;
  const double nd = n ? (double)n : 1.0;
  info->payload_bps = (double)payload_bits / nd;
  info->total_bps = 8.0 * (double)bytes / nd;
  info->side_bps = info->total_bps - info->payload_bps;
}

// Worst-case stream bytes for n values at step `step` and Rice parameter k (see hq_encode_bound in
// hq.h for the derivation).  Per tile of TL values the encoder's lattice inputs w satisfy
// sum |w_i| <= TL K / step (Cauchy-Schwarz on the energy the tile scale normalises, K = 1 + 2^-7
// covering the bf16 rounding of the scale and the binary32 roundings), and each slot's unary part
// is at most (a_i |w_i| + b_i) / 2^k.  Summed with Cauchy-Schwarz over the tile:
//   sum of unary parts <= (A TL K / step + (TL / 8) B) / 2^k
// with A = 2 (E8, D4, Z) or sqrt(14 / 3) (A2: slopes 2 and 4 / sqrt 3 on its even and stretched
// odd slots), and B per octet = the lattice's covering-radius term (doubled with dither, U lies in
// the same cell) plus the zigzag and halved-slot constants.
double unary_per_tile_bound(int lattice, uint32_t tile, double step, int k, bool dither) {
  const double K = 1.0 + 1.0 / 128.0;
  const double d = dither ? 2.0 : 1.0;
  double A = 2.0, B = 0.0;
  switch (lattice) {
    case HQ_E8: B = 2.0 * sqrt(8.0) * 1.0 * d + 12.0; break;          // covering radius 1 per octet
    case HQ_D4: B = 2.0 * sqrt(8.0) * sqrt(2.0) * d + 8.0; break;     // radius 1 per 4-block
    case HQ_Z: B = 2.0 * sqrt(8.0) * (sqrt(8.0) / 2.0) * d; break;    // 1/2 per coordinate
    default:                                                          // A2: 1/sqrt 3 per pair
      A = sqrt(14.0 / 3.0);
      B = 4.0 * (sqrt(28.0) / 3.0) * d + 12.0;
      break;
  }
  const double q = (A * (double)tile * K / step + ((double)tile / 8.0) * B) / ldexp(1.0, k);
  return floor(q * (1.0 + 1e-12)) + (double)tile;  // plus one terminator bit per value
}

uint64_t encode_bound_at(uint64_t n, int lattice, uint32_t tile, double step, int k, bool dither) {
  const uint64_t chunks = chunks_of(n);
  const uint64_t ct = 8192ull / tile;
  const uint64_t fixed_off = align256h(128 + 4 * (chunks + 1));
  const uint64_t unary_off = align256h(fixed_off + chunks * ct * tile_fixed_bits_h(lattice, k, tile) / 8ull);
  if (chunks == 0) return unary_off;
  const double per_tile = unary_per_tile_bound(lattice, tile, step, k, dither);
  const uint64_t T = n / tile;
  const uint64_t last_tiles = T - (chunks - 1) * ct;
  const double full_words = ceil((double)ct * per_tile / 64.0);
  const double last_words = ceil((double)last_tiles * per_tile / 64.0);
  const double bytes = (double)unary_off + 8.0 * ((double)(chunks - 1) * full_words + last_words);
  return bytes >= 1.8e19 ? UINT64_MAX : (uint64_t)bytes;
}

// ---- the allocation-free encode: its workspace is a static device array ------------------------
// Largest n of hq_encode_noalloc, and the array sized for it: the workspace of an encode of that
// many values (4 KiB of state, 12.25 KiB of rate counters and published words, one 8-byte offset flag
// per 8192-value chunk plus one): 1,065,472 bytes per GPU, held until the process ends.
constexpr uint64_t kNoAllocMaxValues = 1ull << 30;
constexpr size_t kScratchBytes =
    kWsHeader + kWsRate + ((8ull * ((kNoAllocMaxValues + 8191) / 8192 + 1) + 255) & ~(uint64_t)255);

// In host code `scratch` names a host-side stand-in, not device memory: kernels and copies take the
// device address that hipGetSymbolAddress returns for the current device (scratch_address below).
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_address[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
int scratch_address(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_address[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return HQ_ERR_HIP;
    g_scratch_address[dev] = a;
  }
  *p = g_scratch_address[dev];
  return HQ_OK;
}

}  // namespace

extern "C" {

uint32_t hq_version(void) { return (1u << 16) | kFormatVersion; }

const char* hq_strerror(int code) {
  switch (code) {
    case HQ_OK: return "ok";
    case HQ_ERR_INVALID_ARG: return "invalid argument";
    case HQ_ERR_UNSUPPORTED: return "unsupported (tile size or lattice)";
    case HQ_ERR_NONFINITE: return "non-finite input tile";
    case HQ_ERR_CAPACITY: return "output buffer too small";
    case HQ_ERR_CORRUPT: return "corrupt stream";
    case HQ_ERR_RATE: return "target rate out of range";
    case HQ_ERR_HIP: return "HIP runtime error";
    case HQ_ERR_TIMEOUT: return "cross-workgroup wait exceeded its bound";
    case HQ_ERR_SCRATCH: return "n exceeds the allocation-free encode's maximum (2^30 values)";
  }
  return "unknown status";
}

int hq_workspace_size(uint64_t n, const hq_params* params, size_t* bytes) {
  (void)params;
  if (!bytes || n % 64) return HQ_ERR_INVALID_ARG;
  *bytes = workspace_bytes_for(n);
  return HQ_OK;
}

int hq_stream_fixed_bytes(uint64_t n, int32_t lattice, int32_t rice_k, uint32_t tile, uint64_t* bytes) {
  if (!bytes || lattice < HQ_Z || lattice > HQ_A2 || rice_k < 0 || rice_k > 15) return HQ_ERR_INVALID_ARG;
  if (!valid_tile(tile)) return HQ_ERR_UNSUPPORTED;
  if (n % tile) return HQ_ERR_INVALID_ARG;
  const uint64_t chunks = chunks_of(n);
  const uint64_t fixed_off = align256h(128 + 4 * (chunks + 1));
  *bytes = align256h(fixed_off + chunks * (8192ull / tile) * tile_fixed_bits_h(lattice, rice_k, tile) / 8ull);
  return HQ_OK;
}

int hq_encode_bound(uint64_t n, const hq_params* params, uint64_t* max_bytes) {
  if (!max_bytes || !params) return HQ_ERR_INVALID_ARG;
  if (!valid_tile(params->tile)) return HQ_ERR_UNSUPPORTED;
  if (params->lattice < HQ_Z || params->lattice > HQ_A2 || n % params->tile || n > (1ull << 35))
    return HQ_ERR_INVALID_ARG;
  if (params->dither > 7 || (params->dither > 1 && !(params->dither & 1))) return HQ_ERR_INVALID_ARG;
  if (params->rice_k < -1 || params->rice_k > 15) return HQ_ERR_INVALID_ARG;
  double step;
  if (params->step > 0.0f) {
    const uint32_t b = f32_bits(params->step);
    if (b < kStepMin || b > kStepMax) return HQ_ERR_INVALID_ARG;
    step = (double)params->step;
  } else if (params->step == 0.0f || params->step == -1.0f) {
    step = ldexp(1.0, -12);  // rate control may pick any step of the range: the smallest is the worst
  } else {
    return HQ_ERR_INVALID_ARG;
  }
  uint64_t worst = 0;
  for (int k = 0; k <= 15; ++k) {
    if (params->rice_k >= 0 && k != params->rice_k) continue;
    const uint64_t b = encode_bound_at(n, params->lattice, params->tile, step, k, params->dither != 0);
    if (b > worst) worst = b;
  }
  *max_bytes = worst;
  return HQ_OK;
}

int hq_rate(const void* x, int32_t dtype, uint64_t n, const hq_params* params, hq_info* info, void* workspace,
            size_t workspace_bytes, hq_stream_t stream) {
  int rc = check_params(params, n);
  if (rc) return rc;
  if (dtype != HQ_F32 && dtype != HQ_BF16) return HQ_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < workspace_bytes_for(n) || (n && !x)) return HQ_ERR_INVALID_ARG;
  if (((uintptr_t)x & 15u) || ((uintptr_t)workspace & 255u)) return HQ_ERR_INVALID_ARG;
  if (params->step == -1.0f) return HQ_ERR_INVALID_ARG;
  EncodeArgs a = make_args(x, dtype, n, params, nullptr, 0, workspace, stream);
  const RatePlan rp = plan_rate(a);
  rc = start_call(a, rp);
  if (rc) return rc;
  if (launch_rate(a, rp) != hipSuccess) return HQ_ERR_HIP;
  if (!info) return HQ_OK;  // asynchronous: the operating point stays in the workspace
  Workspace h;
  if (hipMemcpyAsync(&h, workspace, sizeof(Workspace), hipMemcpyDeviceToHost, a.stream) != hipSuccess ||
      hipStreamSynchronize(a.stream) != hipSuccess)
    return HQ_ERR_HIP;
  if (error_flags(h)) return status_from_flags(error_flags(h));
  if (info) {
    memset(info, 0, sizeof(*info));
    float st;
    memcpy(&st, &h.step_bits, 4);
    info->step = st;
    info->rice_k = h.rice_k;
    info->payload_bps = params->step > 0.0f ? 0.0 : (double)params->target_bps;
  }
  return HQ_OK;
}

int hq_encode(const void* x, int32_t dtype, uint64_t n, const hq_params* params, void* out, uint64_t out_capacity,
              uint64_t* out_bytes, hq_info* info, void* workspace, size_t workspace_bytes, hq_stream_t stream) {
  int rc = check_params(params, n);
  if (rc) return rc;
  if (dtype != HQ_F32 && dtype != HQ_BF16) return HQ_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < workspace_bytes_for(n) || (n && !x) || !out) return HQ_ERR_INVALID_ARG;
  if (((uintptr_t)out & 15u) || ((uintptr_t)x & 15u) || ((uintptr_t)workspace & 255u)) return HQ_ERR_INVALID_ARG;
  EncodeArgs a = make_args(x, dtype, n, params, out, out_capacity, workspace, stream);
  if (params->step != -1.0f) {
    const RatePlan rp = plan_rate(a);
    rc = start_call(a, rp);
    if (rc) return rc;
    if (launch_rate(a, rp) != hipSuccess) return HQ_ERR_HIP;
  } else if (launch_init(a, 0, kInitKeep) != hipSuccess) {
    // the workspace's operating point is kept; status, results and look-back flags reset
    return HQ_ERR_HIP;
  }
  if (launch_encode(a) != hipSuccess) return HQ_ERR_HIP;
  if (!out_bytes) return HQ_OK;
  Results r;
  rc = read_results(workspace, a.stream, &r);
  if (rc) return rc;
  *out_bytes = r.total_bytes;
  fill_info(info, n, r.step_bits, r.k, r.total_bytes, r.payload_bits);
  return status_from_flags(r.status);
}

int hq_encode_noalloc(const void* x, int32_t dtype, uint64_t n, const hq_params* params, void* out,
                      uint64_t out_capacity, uint64_t* out_bytes, hq_info* info, hq_stream_t stream) {
  const int rc = check_params(params, n);
  if (rc) return rc;
  if (n > kNoAllocMaxValues) return HQ_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(&ws) != HQ_OK) return HQ_ERR_HIP;
  return hq_encode(x, dtype, n, params, out, out_capacity, out_bytes, info, ws, kScratchBytes, stream);
}

int hq_decode(const void* stream_data, uint64_t stream_bytes, void* out, int32_t out_dtype, uint64_t n,
              void* workspace, size_t workspace_bytes, hq_stream_t stream) {
  if (n % 64 || chunks_of(n) >= 0xFFFFFFFFull) return HQ_ERR_INVALID_ARG;
  if (out_dtype != HQ_F32 && out_dtype != HQ_BF16) return HQ_ERR_INVALID_ARG;
  if (!stream_data || !workspace || workspace_bytes < kWsHeader || (n && !out)) return HQ_ERR_INVALID_ARG;
  if (((uintptr_t)stream_data & 15u) || ((uintptr_t)out & 15u) || ((uintptr_t)workspace & 255u))
    return HQ_ERR_INVALID_ARG;
  if (launch_decode(static_cast<const uint8_t*>(stream_data), stream_bytes, out, out_dtype, n,
                    static_cast<Workspace*>(workspace), next_call(), static_cast<hipStream_t>(stream)) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

static size_t gemv_xt_bytes(uint64_t cols) { return align256h(4ull * cols); }

int hq_gemv_workspace_size(uint64_t rows, uint64_t cols, size_t* bytes) {
  if (!bytes || cols % 64 || (rows && cols && rows > (1ull << 35) / cols)) return HQ_ERR_INVALID_ARG;
  // per-tile partial products for the shortest tile (64 values), whatever the stream's tile length
  *bytes = kWsHeader + gemv_xt_bytes(cols) + align256h(4ull * (rows * cols / 64));
  return HQ_OK;
}

int hq_gemv(const void* stream_data, uint64_t stream_bytes, uint64_t rows, uint64_t cols, const void* x,
            int32_t x_dtype, float* y, void* workspace, size_t workspace_bytes, hq_stream_t stream) {
  size_t need = 0;
  int rc = hq_gemv_workspace_size(rows, cols, &need);
  if (rc) return rc;
  if (x_dtype != HQ_F32 && x_dtype != HQ_BF16) return HQ_ERR_INVALID_ARG;
  if (!stream_data || !workspace || workspace_bytes < need || (rows && cols && (!x || !y))) return HQ_ERR_INVALID_ARG;
  if (((uintptr_t)stream_data & 15u) || ((uintptr_t)x & 15u) || ((uintptr_t)y & 3u) || ((uintptr_t)workspace & 255u))
    return HQ_ERR_INVALID_ARG;
  char* w = static_cast<char*>(workspace);
  float* xt = reinterpret_cast<float*>(w + kWsHeader);
  float* tp = reinterpret_cast<float*>(w + kWsHeader + gemv_xt_bytes(cols));
  if (launch_gemv(static_cast<const uint8_t*>(stream_data), stream_bytes, rows, cols, x, x_dtype, y,
                  static_cast<Workspace*>(workspace), xt, tp, next_call(), static_cast<hipStream_t>(stream)) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_status(void* workspace, hq_stream_t stream) {
  if (!workspace) return HQ_ERR_INVALID_ARG;
  Workspace h;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&h, workspace, sizeof(Workspace), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return HQ_ERR_HIP;
  return status_from_flags(error_flags(h));
}

int hq_fallbacks(const void* workspace, hq_stream_t stream, uint32_t* flags) {
  if (!workspace || !flags) return HQ_ERR_INVALID_ARG;
  Workspace h;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&h, workspace, sizeof(Workspace), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return HQ_ERR_HIP;
  *flags = fallback_flags(h);
  return HQ_OK;
}

int hq_codes(const void* x, int32_t dtype, uint64_t n, const hq_params* params, int32_t* codes, uint16_t* scales,
             void* workspace, size_t workspace_bytes, hq_stream_t stream) {
  if (!params || !(params->step > 0.0f)) return HQ_ERR_INVALID_ARG;
  int rc = check_params(params, n);
  if (rc) return rc;
  if (dtype != HQ_F32 && dtype != HQ_BF16) return HQ_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < workspace_bytes_for(0) || (n && (!x || !codes || !scales)))
    return HQ_ERR_INVALID_ARG;
  // the kernel reads x and writes codes with 16-byte vector accesses
  if (((uintptr_t)x & 15u) || ((uintptr_t)codes & 15u) || ((uintptr_t)scales & 1u) || ((uintptr_t)workspace & 255u))
    return HQ_ERR_INVALID_ARG;
  EncodeArgs a = make_args(x, dtype, n, params, nullptr, 0, workspace, stream);
  a.chunks = 0;  // no look-back flags are needed
  if (launch_init(a, (int64_t)a.fixed_step_bits, kInitFinal) != hipSuccess) return HQ_ERR_HIP;
  if (launch_codes(a, codes, scales) != hipSuccess) return HQ_ERR_HIP;
  return HQ_OK;
}

}  // extern "C"
