// Internal definitions shared by the liboal HIP sources (not part of the ABI).
//
// Feature layout of the prefix state.  With u = [v; 1] (W = d_v + 1 = 65 columns)
// the state of [OAL] Eq. 5 is  H = sum_j phi_k(k_j) u_j^T  where the key-side
// feature vector phi_k has, in canonical packed order ([OAL] App. D, packed-
// symmetric states):
//   f = 0                 1                      (H0)
//   f = 1 .. 64           k_r                    (H1_r)
//   f = 65 + p            k_r k_t, p-th pair r <= t in row-major order (H2_rt)
// and the readout of Eq. 6 is  u~ = phi_q(q)^T H  with
//   phi_q = [a, b'_r q_r, c'_rt q_r q_t]   (b' = b / sqrt d_h, c' = m_rt C_rt / d_h,
//   m_rt = 1 on the diagonal and 2 off it).
// The persistent state stores H column-major: [unit][w = 0..64][f = 0..DS-1]
// (fp32, DS = 2176 >= 2145, padding rows are zero), unit = b * n_kv_heads + kv.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "../../include/oal.h"

namespace oal {

constexpr int DH = 64;                  // query/key head dimension
constexpr int DV = 64;                  // value head dimension
constexpr int W = DV + 1;               // value channels + the all-ones channel
constexpr int NPAIR = DH * (DH + 1) / 2;  // 2080 packed pairs r <= t
constexpr int DCAN = 1 + DH + NPAIR;    // 2145 canonical feature rows
constexpr int DS = 2176;                // padded row count of a state column
constexpr int GMAX = 6;                 // largest supported group count
constexpr int LDIM = GMAX + 1;          // leading dimension of L and M in coeffs
constexpr size_t STATE_FLOATS = (size_t)W * DS;  // per (batch, kv head) unit

// Index of pair (r, t), r <= t, in the packed order.
__host__ __device__ constexpr inline int pair_index(int r, int t) {
  return r * DH - r * (r - 1) / 2 + (t - r);
}

// The pair (r, t), r <= t, of packed index p = pair_index(r, t), by arithmetic: row r
// starts at S(r) = r (2 DH + 1 - r) / 2, so r is the floor of the smaller root of
// S(r) = p, corrected by one either way for the rounding of the square root (exact
// for all NPAIR pairs).  No table read: a lane-indexed table load inside a branch
// would be awaited on the spot.
__device__ __forceinline__ void pair_decode(int p, int& r, int& t) {
  int rr = (int)((129.f - __builtin_sqrtf(16641.f - 8.f * (float)p)) * 0.5f);
  if (rr * (129 - rr) / 2 > p)
    --rr;
  else if ((rr + 1) * (128 - rr) / 2 <= p)
    ++rr;
  r = rr;
  t = p - rr * (129 - rr) / 2 + rr;
}
static_assert(DH == 64, "pair_decode's constants are for d_h = 64");

// LDS staging of a contiguous span by a block of NT threads: element i < N (the
// tile's capacity) gets load(i) for i < n and zero beyond (1 <= n <= N).  The loads
// are unconditional (index clamped to n - 1) and all issued before the first is
// awaited: a loop striding by blockDim.x is not unrolled, so each element would
// wait for its own load, and a load in a divergent block is awaited at its end.
template <int N, int NT = 256, typename Load, typename Store>
__device__ __forceinline__ void stage_span(int tid, int n, Load load, Store store) {
  constexpr int E = (N + NT - 1) / NT;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = load(min(tid + NT * e, n - 1));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + NT * e;
    if (i < N) store(i, i < n ? x[e] : 0.f);
  }
}

// record index of c_f for a feature f < DCAN (no branch: for loads that must not
// wait in a divergent block)
__device__ __forceinline__ int coef_index(int f) {
  return f == 0 ? OAL_COEF_A : (f <= DH ? OAL_COEF_BP + f - 1 : OAL_COEF_CP + f - 1 - DH);
}

// The same for a thread count nt known only at run time (0 <= n <= N): K loads of
// each thread in flight per round.
template <int K, typename Load, typename Store>
__device__ __forceinline__ void stage_span_rt(int tid, int nt, int N, int n, Load load, Store store) {
  for (int i0 = 0; i0 < N; i0 += K * nt) {
    float x[K];
#pragma unroll
    for (int e = 0; e < K; ++e) x[e] = load(max(min(i0 + tid + e * nt, n - 1), 0));
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const int i = i0 + tid + e * nt;
      if (i < N) store(i, i < n ? x[e] : 0.f);
    }
  }
}


// ---- element access ------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
  // four consecutive elements, i a multiple of 4
  static __device__ __forceinline__ void store4(float* p, size_t i, const float* x) {
    *reinterpret_cast<float4*>(p + i) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <> struct Elem<uint16_t> {  // bf16 stored as raw bits
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf16_bits_to_float(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float x) {
    p[i] = float_to_bf16_bits(x);
  }
  static __device__ __forceinline__ void store4(uint16_t* p, size_t i, const float* x) {
    uint2 w;
    w.x = (uint32_t)float_to_bf16_bits(x[0]) | ((uint32_t)float_to_bf16_bits(x[1]) << 16);
    w.y = (uint32_t)float_to_bf16_bits(x[2]) | ((uint32_t)float_to_bf16_bits(x[3]) << 16);
    *reinterpret_cast<uint2*>(p + i) = w;
  }
};

// ---- coefficient record accessors ---------------------------------------

__device__ __forceinline__ const float* coef_rec(const void* coeffs, int h) {
  return reinterpret_cast<const float*>(coeffs) + (size_t)h * OAL_COEF_WORDS;
}

// ---- host-side launch helpers (defined in oal_api.hip) ----------------------

oal_status set_error(oal_status st, const char* fmt, ...);
oal_status check_launch(const char* what);

// Optional per-kernel timing with HIP events recorded on the launch stream
// (enabled through oal_profile_enable).  prof_begin returns -1 when disabled.
int prof_begin(const char* kernel, hipStream_t stream);
void prof_end(int slot, hipStream_t stream);
struct ProfScope {
  int slot;
  hipStream_t stream;
  ProfScope(const char* kernel, hipStream_t s) : slot(prof_begin(kernel, s)), stream(s) {}
  ~ProfScope() {
    if (slot >= 0) prof_end(slot, stream);
  }
};

}  // namespace oal

// Opaque state handle (definition shared by the host shim and kernels' launchers).
struct oal_state {
  int batch;
  int n_kv_heads;
  int device;
  float* data;        // [batch * n_kv_heads][W][DS] fp32
  size_t bytes;
  int64_t tokens;     // tokens absorbed so far (host-side bookkeeping)
};
