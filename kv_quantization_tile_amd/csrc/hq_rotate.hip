// hq_rotate.hip -- per-layer Haar-uniform rotation of 128-value vectors (KV path), on MFMA.
//
// HyperQuant technical summary (gist.science/ko/paper/2606.23406), "Methodology: the HyperQuant
// pipeline", component 4: against the KV cache's bias, each layer is rotated either by a full
// Haar-uniform matrix or by the cheap +-1 sign diagonal.  The sign diagonal folds into the codec's
// own D through the per-layer seed; this file provides the full matrix:
//   hq_haar_matrix  the matrix Q of a seed (host, binary64 inside): G with independent N(0,1)
//                   entries from Philox4x32-10 (key = seed, counter (e / 4, 0, 0, 2) for entry
//                   e = 128 i + j, two Box-Muller pairs per call), G = Q R by Householder
//                   reflections, columns of Q signed so that diag(R) > 0 (then Q is Haar on O(128));
//   hq_rotate       y_v = Q x_v (or Q^T x_v) for every 128-value bf16 vector v, bf16 out.  This is
//                   the one dense contraction of the path: [vectors x 128] x [128 x 128], on
//                   v_mfma_f32_32x32x16_bf16 with Q split as Q_hi + Q_lo (bf16 each), so the
//                   products of the exact bf16 inputs with Q carry about 16 bits of Q and
//                   accumulate in binary32.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/hq.h"

namespace hq_rot {

// ---------------------------------------------------------------------------------------------
// Host: the matrix of a seed.

static void philox4x32_10_host(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

static void gaussian_matrix(uint64_t seed, double* g) {
  const double two_pi = 6.283185307179586476925286766559;
  for (uint32_t c = 0; c < 128u * 128u / 4u; ++c) {
    uint32_t w[4] = {c, 0u, 0u, 2u};
    philox4x32_10_host(w, (uint32_t)seed, (uint32_t)(seed >> 32));
    for (int pair = 0; pair < 2; ++pair) {
      const double u1 = ((double)w[2 * pair] + 0.5) * 0x1p-32, u2 = ((double)w[2 * pair + 1] + 0.5) * 0x1p-32;
      const double r = std::sqrt(-2.0 * std::log(u1));
      g[4 * c + 2 * pair] = r * std::cos(two_pi * u2);
      g[4 * c + 2 * pair + 1] = r * std::sin(two_pi * u2);
    }
  }
}

// Householder QR of a (row-major 128 x 128); returns Q with diag(R) > 0.
static void haar_from_gaussian(std::vector<double>& a, std::vector<double>& q) {
  const int n = 128;
  q.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) q[(size_t)i * n + i] = 1.0;
  std::vector<double> v(n), rdiag(n);
  for (int k = 0; k < n; ++k) {
    double norm = 0.0;
    for (int i = k; i < n; ++i) norm += a[(size_t)i * n + k] * a[(size_t)i * n + k];
    norm = std::sqrt(norm);
    const double akk = a[(size_t)k * n + k];
    const double alpha = akk >= 0.0 ? -norm : norm;
    double vn = 0.0;
    for (int i = k; i < n; ++i) {
      v[i] = a[(size_t)i * n + k] - (i == k ? alpha : 0.0);
      vn += v[i] * v[i];
    }
    rdiag[k] = alpha;
    if (vn == 0.0) {
      rdiag[k] = akk;
      continue;
    }
    const double beta = 2.0 / vn;
    for (int j = k; j < n; ++j) {  // A[k:, k:] -= beta v (v^T A[k:, k:])
      double s = 0.0;
      for (int i = k; i < n; ++i) s += v[i] * a[(size_t)i * n + j];
      s *= beta;
      for (int i = k; i < n; ++i) a[(size_t)i * n + j] -= s * v[i];
    }
    for (int i = 0; i < n; ++i) {  // Q[:, k:] -= beta (Q[:, k:] v) v^T
      double s = 0.0;
      for (int j = k; j < n; ++j) s += q[(size_t)i * n + j] * v[j];
      s *= beta;
      for (int j = k; j < n; ++j) q[(size_t)i * n + j] -= s * v[j];
    }
  }
  for (int k = 0; k < n; ++k)
    if (rdiag[k] < 0.0)
      for (int i = 0; i < n; ++i) q[(size_t)i * n + k] = -q[(size_t)i * n + k];
}

// ---------------------------------------------------------------------------------------------
// Device: y_v = M x_v with M = Q or Q^T.  A workgroup of four wavefronts; wavefront w keeps rows
// 32 w .. 32 w + 31 of M in registers (bf16 hi and lo parts, all 128 columns) for its whole life,
// and the grid is one resident wave of workgroups looping over groups of 32 x kColTiles vectors.
// Per group: the vectors (coalesced 16-byte loads, issued kStages groups ahead) are staged in LDS;
// each wavefront computes D (its 32 features x 32 vectors) += A (32 features x 16 k) * B (16 k x 32
// vectors) over 8 k-steps and the two halves of M; the results go back through LDS so that the
// stores are whole 16-byte chunks of consecutive vectors.  Every vector is read from HBM once and
// written once; M is read once per workgroup.
// MFMA 32x32x16 bf16 lane layout (checked on the device): A lane l: row l % 32, k = 8 (l / 32) + e;
// B lane l: column l % 32, same k; D register r: column l % 32, row 8 (r / 4) + 4 (l / 32) + r % 4.

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kRotBlock = 256;  // four wavefronts: one per 32 rows of M

constexpr int kColTiles = 2;  // 32-vector column tiles per group
constexpr int kStages = 2;    // groups in flight per workgroup (register ring)
constexpr int kGroupVec = 32 * kColTiles;        // vectors per group
constexpr int kGroupChunks = kGroupVec * 16;     // 16-byte chunks per group
constexpr int kLoadsPerThread = kGroupChunks / kRotBlock;
static_assert(kGroupChunks % kRotBlock == 0, "whole chunks per thread");

__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);  // finite inputs
}

// In LDS vector v of a group is a row of 16 chunks of 8 bf16; chunk c sits at slot c ^ (v & 15), so
// the 32 vectors a wavefront reads at one k-step, and the 16 chunks of a vector written together,
// spread over all banks.
__device__ __forceinline__ int lds_slot(int v, int c) { return v * 16 + (c ^ (v & 15)); }

// Buffer resource over bytes [base, base + bytes) of global memory (raw, no stride); loads past the
// end return zeros and stores past it are dropped, so the ragged last group needs no branches.  The
// range check covers the per-lane and immediate offsets only, so every offset goes there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(kRotBlock) void rotate_kernel(const uint16_t* __restrict__ x, uint64_t nvec,
                                                           const float* __restrict__ q, int transpose,
                                                           uint16_t* __restrict__ y) {
  __shared__ uint4 s_lds[2 * kGroupChunks];
  uint4* const s_x = s_lds;                 // a group's vectors
  uint4* const s_y = s_lds + kGroupChunks;  // its results
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const uint64_t ngroups = (nvec + kGroupVec - 1) / kGroupVec;
  constexpr uint32_t kGroupBytes = kGroupVec * 256u;
  uint64_t grp = blockIdx.x;
  if (grp >= ngroups) return;  // uniform over the workgroup
  // bytes of group gi that lie inside the tensor (0 past the end)
  auto group_bytes = [&](uint64_t gi) -> uint32_t {
    if (gi >= ngroups) return 0u;
    const uint64_t rest = (nvec - gi * kGroupVec) * 256u;
    return rest < kGroupBytes ? (uint32_t)rest : kGroupBytes;
  };

  // a group's chunks: thread t takes chunks t, t + 256, ... (16 per vector)
  auto load = [&](uint64_t gi, uint4* xr) {
    const __amdgpu_buffer_rsrc_t r = byte_range(x + gi * kGroupVec * 128, group_bytes(gi));
#pragma unroll
    for (int j = 0; j < kLoadsPerThread; ++j) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, (tid + j * kRotBlock) * 16, 0, 0);
      xr[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  // register ring: stage st holds the group kStages - 1 ahead of the one being multiplied
  uint4 xr[kStages][kLoadsPerThread];
#pragma unroll
  for (int st = 0; st < kStages; ++st) load(grp + (uint64_t)st * gridDim.x, xr[st]);

  // this wavefront's rows of M as A fragments: k-step s holds M[32 wave + col][16 s + 8 half + e],
  // split into bf16 hi and lo parts.  M = Q: each lane reads 32 contiguous bytes of its row per
  // k-step; M = Q^T: the 32 lanes of a half read 32 consecutive floats of one row of Q.
  bf16x8 ah[8], al[8];
  auto put = [&](int s, const float* m) __attribute__((always_inline)) {
    uint16_t hb[8], lb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hb[e] = bf16_rne_bits(m[e]);
      lb[e] = bf16_rne_bits(m[e] - __uint_as_float((uint32_t)hb[e] << 16));
    }
    ah[s] = __builtin_bit_cast(bf16x8, make_uint4(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16),
                                                  hb[4] | ((uint32_t)hb[5] << 16), hb[6] | ((uint32_t)hb[7] << 16)));
    al[s] = __builtin_bit_cast(bf16x8, make_uint4(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16),
                                                  lb[4] | ((uint32_t)lb[5] << 16), lb[6] | ((uint32_t)lb[7] << 16)));
  };
  {
    const int row = 32 * wave + col;
    if (!transpose) {
      // rows of Q pass through LDS (coalesced reads), kRowsPerPass rows of each wavefront at a time;
      // row r's 16-byte chunk c sits at slot c ^ (r & 15) of the row
      constexpr int kRowsPerPass = 2 * kGroupChunks / (4 * 32);
      static_assert(kRowsPerPass >= 2 && 32 % kRowsPerPass == 0, "LDS holds whole rows of Q per pass");
      uint4* const s_m = s_lds + wave * kRowsPerPass * 32;
#pragma unroll
      for (int p = 0; p < 32 / kRowsPerPass; ++p) {
        const uint4* src = reinterpret_cast<const uint4*>(q + (32 * wave + p * kRowsPerPass) * 128);
#pragma unroll
        for (int i = 0; i < kRowsPerPass / 2; ++i) {
          const int f = i * 64 + lane, r = f >> 5, c = f & 31;
          s_m[r * 32 + (c ^ (r & 15))] = src[f];
        }
        __syncthreads();
        const int r = col - p * kRowsPerPass;
        if (r >= 0 && r < kRowsPerPass) {
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int c = 4 * s + 2 * half;
            const float4 u = __builtin_bit_cast(float4, s_m[r * 32 + (c ^ (r & 15))]);
            const float4 v = __builtin_bit_cast(float4, s_m[r * 32 + ((c + 1) ^ (r & 15))]);
            const float m[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
            put(s, m);
          }
        }
        __syncthreads();
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float m[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = q[(16 * s + 8 * half + e) * 128 + row];
        put(s, m);
      }
    }
  }

  // one group: stage it into LDS, refill its registers with the group kStages ahead, multiply,
  // stage the result in LDS and store it row by row; false once the workgroup's groups are done
  // (uniform over the workgroup).  Two barriers per group: s_x is rewritten only after every
  // wavefront passed the previous group's second barrier (its MFMAs were done), s_y only after
  // every wavefront passed this group's first (its stores of the previous group were read out).
  auto step = [&](uint4* xs) __attribute__((always_inline)) -> bool {
    if (grp >= ngroups) return false;
#pragma unroll
    for (int j = 0; j < kLoadsPerThread; ++j) {
      const int f = j * kRotBlock + tid;
      s_x[lds_slot(f >> 4, f & 15)] = xs[j];
    }
    __syncthreads();
    load(grp + (uint64_t)kStages * gridDim.x, xs);
    f32x16 acc[kColTiles];
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) acc[ct] = (f32x16){};
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, s_x[lds_slot(32 * ct + col, 2 * s + half)]);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[s], b, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[s], b, acc[ct], 0, 0, 0);
      }
    // register r of tile ct holds feature 32 wave + 8 (r / 4) + 4 half + r % 4 of vector 32 ct + col
    // of the group: four consecutive features per four registers, 8 bytes into the vector's LDS row
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const bf16x2 p0 = __builtin_convertvector((f32x2){acc[ct][4 * g4], acc[ct][4 * g4 + 1]}, bf16x2);
        const bf16x2 p1 = __builtin_convertvector((f32x2){acc[ct][4 * g4 + 2], acc[ct][4 * g4 + 3]}, bf16x2);
        const int v = 32 * ct + col;
        reinterpret_cast<uint2*>(s_y)[2 * lds_slot(v, 4 * wave + g4) + half] =
            make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
      }
    __syncthreads();
    {
      const __amdgpu_buffer_rsrc_t r = byte_range(y + grp * kGroupVec * 128, group_bytes(grp));
#pragma unroll
      for (int j = 0; j < kLoadsPerThread; ++j) {
        const int f = j * kRotBlock + tid;
        const uint4 w = s_y[lds_slot(f >> 4, f & 15)];
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){w.x, w.y, w.z, w.w}, r, f * 16, 0, 0);
      }
    }
    grp += gridDim.x;
    return true;
  };
  static_assert(kStages >= 1 && kStages <= 4, "register ring of one to four groups");
  for (;;) {
    if (!step(xr[0])) return;
    if constexpr (kStages > 1)
      if (!step(xr[1])) return;
    if constexpr (kStages > 2)
      if (!step(xr[2])) return;
    if constexpr (kStages > 3)
      if (!step(xr[3])) return;
  }
}

// Workgroups of rotate_kernel resident at once on the current device (0 on a runtime error); asked
// once per device.
static uint64_t resident_blocks() {
  static std::atomic<uint64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const uint64_t c = cached[dev].load(std::memory_order_relaxed);
    if (c) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rotate_kernel, kRotBlock, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const uint64_t n = (uint64_t)(per_cu > 0 ? per_cu : 1) * (uint64_t)(cus > 0 ? cus : 1);
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace hq_rot

extern "C" {

int hq_haar_matrix(uint64_t seed, float* q) {
  if (!q) return HQ_ERR_INVALID_ARG;
  std::vector<double> a(128 * 128), qd;
  hq_rot::gaussian_matrix(seed, a.data());
  hq_rot::haar_from_gaussian(a, qd);
  for (int i = 0; i < 128 * 128; ++i) q[i] = (float)qd[i];
  return HQ_OK;
}

int hq_rotate(const void* x, uint64_t n, const float* q, int32_t transpose, void* y, hq_stream_t stream) {
  if (n % 128 || (n && (!x || !y || !q)) || (transpose != 0 && transpose != 1)) return HQ_ERR_INVALID_ARG;
  if (((uintptr_t)x & 15u) || ((uintptr_t)y & 15u) || ((uintptr_t)q & 3u)) return HQ_ERR_INVALID_ARG;
  const uint64_t nvec = n / 128;
  if (nvec == 0) return HQ_OK;
  const uint64_t groups = (nvec + hq_rot::kGroupVec - 1) / hq_rot::kGroupVec;
  // one resident wave of workgroups (each loads M once, then loops over groups)
  const uint64_t resident = hq_rot::resident_blocks();
  if (resident == 0) return HQ_ERR_HIP;
  const uint64_t blocks = groups < resident ? groups : resident;
  hipLaunchKernelGGL(hq_rot::rotate_kernel, dim3((uint32_t)blocks), dim3(hq_rot::kRotBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x), nvec, q, (int)transpose,
                     static_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_ERR_HIP;
}

}  // extern "C"
