// Tiled per-chunk prefix-state layout read by the matrix-core readout, and the
// MFMA helpers shared by the matrix-core kernels (gfx950, wave64).
//
// The readout of [OAL] Eq. 6 is a contraction over feature rows f of the state:
//   u~^T[w][i] = sum_f H[f][w] phi_q(q_i)[f]
// evaluated on v_mfma_f32_32x32x16_f16 with the state as the A operand (rows w)
// and the query features as the B operand (columns = tokens).  The K dimension
// (features) is cut into K-steps of 16 rows:
//   K-steps 0..3      linear rows H1_r, r = 16 ks + j                  (j = 0..15)
//   then, per t-block c = 0..3 (t = 16 c + j), 16 c + 12 K-steps from quad_base(c):
//     r = 0 .. 16 c + 7     one K-step per r (quad_base(c) + r), element j = H2_rt
//     r = 16 c + 8 + 2 s + e (s = 0..3, e = 0, 1): K-step quad_base(c) + 16 c + 8 + s,
//                           element 8 e + jj = H2_rt at t = 16 c + 8 + jj
// Symmetric pairs follow [OAL] App. D (packed states: multiplicity one on the
// diagonal, two off it).  Off the diagonal 16-block (r < 16 c) only t > r is
// stored, read with multiplicity 2.  In the diagonal block, rows r = 16 c + i
// with i < 8 keep all 16 t's: for t < 16 c + 8 both orders of a pair are present
// (multiplicity 1 each), for t >= 16 c + 8 only this one (multiplicity 2); rows
// with i >= 8 keep only t >= 16 c + 8, where again both orders are present, and
// two such rows share a K-step.  Every half K-step (8 elements) has a single r,
// so the query feature c_rt q_r q_t / d_h of it is (m q_r) * qhat_{g(r)}[t] with
// qhat_gamma[t] = q_t M_{gamma, g(t)} / d_h per 8-wide t-range.
// Layout of one K-step: [w = 0..63][j = 0..15] fp16 (2 KB).  The fp16 values are
// H * 2^-e_S with one exponent e_S per (unit, call), chosen from a bound on |H|
// (see oal_state_mfma.hip) so that every entry stays below 2^15; the readout
// scales its query features and everything else it adds into the same
// accumulators by powers of two, so the common factor cancels in y = u~/u~_65.
//
// The all-ones channel (denominator) is kept separately in fp32 "side" data:
// H0 value channels, z1_r = sum k_r, z0 = token count, Z_rt = sum k_r k_t (full
// 64 x 64); the denominator is a z0 + sum_r b'_r q_r z1_r + q^T (C/d_h o Z) q.
// These side values are not scaled; side[SIDE_SEXP] holds e_S as a float.
#pragma once

#include "oal_common.h"

namespace oal {
namespace tile {

constexpr int NKS_LIN = 4;
constexpr int NKS = 148;
constexpr int KS_BYTES = 64 * 16 * 2;                  // one K-step, fp16
constexpr size_t TILE_BYTES = (size_t)NKS * KS_BYTES;  // 303104
constexpr int SIDE_H0 = 0;       // [64] sum v (value channels of H0)
constexpr int SIDE_Z1 = 64;      // [64] sum k_r
constexpr int SIDE_Z0 = 128;     // token count
constexpr int SIDE_SEXP = 129;   // e_S: the fp16 entries are H * 2^-e_S (then padding to 192)
constexpr int SIDE_Z = 192;      // [64][64] sum k_r k_t
constexpr int SIDE_FLOATS = SIDE_Z + DH * DH;           // 4288
constexpr size_t BYTES = TILE_BYTES + (size_t)SIDE_FLOATS * 4;   // 320256 = 1251 * 256

// First K-step of t-block c (c = 4: the end of the tile).
__host__ __device__ constexpr int quad_base(int c) { return NKS_LIN + 8 * c * c + 4 * c; }
static_assert(quad_base(4) == NKS, "K-step count");

// K-step that holds row r of t-block c (r < 16 c + 16); element of t in it: t % 16,
// or for the merged rows (r - 16 c >= 8, t % 16 >= 8 only) 8 (r % 2) + t % 8.
__host__ __device__ constexpr int quad_ks(int r, int c) {
  return quad_base(c) + (r - 16 * c < 8 ? r : 16 * c + 8 + ((r - 16 * c - 8) >> 1));
}
__host__ __device__ constexpr bool quad_merged(int r, int c) { return r - 16 * c >= 8; }

// Inverse: the pair (r, t) that element pos of quadratic K-step ks holds.
__host__ __device__ inline void quad_rt(int ks, int pos, int& r, int& t) {
  const int c = ks >= quad_base(3) ? 3 : ks >= quad_base(2) ? 2 : ks >= quad_base(1) ? 1 : 0;
  const int i = ks - quad_base(c);
  if (i < 16 * c + 8) {
    r = i;
    t = 16 * c + pos;
  } else {
    r = 16 * c + 8 + 2 * (i - 16 * c - 8) + (pos >> 3);
    t = 16 * c + 8 + (pos & 7);
  }
}

}  // namespace tile

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// D = A B + C on a 32x32x16 tile.  Lane layout (wave64):
//   A[i][k]: lane = i + 32 (k / 8), element k % 8
//   B[k][j]: lane = j + 32 (k / 8), element k % 8
//   D[i][j]: lane = j + 32 ((i / 4) % 2), register (i % 4) + 4 (i / 8)
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same tile shape with fp16 operands.
__device__ __forceinline__ f32x16 mfma32h(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of D held in register i by lane-half h.
__device__ __forceinline__ int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = x;
  return r;
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

__device__ __forceinline__ float bf(const __bf16 x) { return (float)x; }

// Swizzle key of a 128-byte LDS row: 16-byte chunk c of row r sits at slot
// c ^ row_key(r).  Consecutive rows read by consecutive lanes then fall on
// distinct banks whether the LDS serves 8, 16 or 32 lanes of a 16-byte read per
// cycle (any 8 aligned consecutive rows, the 8 rows of one parity among 16, and
// the 8 rows of one residue mod 4 among 32 have distinct keys).
__device__ __forceinline__ int row_key(int r) { return (r ^ (r >> 3)) & 7; }

// A row of 64 bf16 in a swizzled 128-byte LDS row.
struct SwRow {
  const uint8_t* p;
  int key;
  __device__ __forceinline__ SwRow(const uint8_t* base, int row) : p(base + row * 128), key(row_key(row)) {}
  // 16-byte chunk c (elements 8 c .. 8 c + 7)
  __device__ __forceinline__ const uint8_t* chunk(int c) const { return p + ((c ^ key) << 4); }
  // element d
  __device__ __forceinline__ const __bf16* elem(int d) const {
    return reinterpret_cast<const __bf16*>(p + (((d >> 3) ^ key) << 4) + ((d & 7) << 1));
  }
};

// ---- direct-to-LDS loads ---------------------------------------------------
// The loads are issued from inline assembly so that the compiler neither waits
// for them before LDS reads it cannot prove disjoint from their destination,
// nor before rewriting their operand registers; their completion is awaited
// explicitly with wait_vmcnt before the barrier that hands a buffer to the
// waves.  Other memory operations of a wave complete in issue order with them,
// so the compiler's own counts stay safe (only stricter).

// Wait until at most N vector-memory operations of this wave are outstanding
// (the direct-to-LDS loads count there); LDS: also until this wave's LDS reads
// have returned, so that no buffer is refilled while one of them is in flight.
// The immediate holds vmcnt in bits 3:0 and 15:14, lgkmcnt in 11:8, expcnt in 6:4.
template <int N, bool LDS = false>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((LDS ? 0x0070 : 0x0F70) | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which would wait
// for the prefetches still in flight); the clobber keeps LDS accesses in place.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes) (reads beyond it return zero).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;                                                  // 32-bit data format
  return r;
}

// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from rsrc + soff + voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void load_lds16(const i32x4& rsrc, uint32_t lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}

// Largest magnitude among 8 bf16 values, as bf16 magnitude bits (for
// non-negative bf16 numbers the integer order is the numeric order).
__device__ __forceinline__ uint32_t absmax8_bits(const uint4& x) {
  const uint32_t a = x.x & 0x7fff7fffu, b = x.y & 0x7fff7fffu;
  const uint32_t c = x.z & 0x7fff7fffu, d = x.w & 0x7fff7fffu;
  const uint32_t m0 = max(max(a & 0xffffu, a >> 16), max(b & 0xffffu, b >> 16));
  const uint32_t m1 = max(max(c & 0xffffu, c >> 16), max(d & 0xffffu, d >> 16));
  return max(m0, m1);
}

}  // namespace oal
