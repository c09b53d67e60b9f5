// Prefix states of the chunked prefill on the gfx950 matrix cores.
//
// [OAL] Eq. 5: H = sum_j phi_k(k_j) u_j^T with u_j = [v_j; 1] and
// phi_k = [1, k_r, k_r k_t].  The readout of chunk c needs the exclusive prefix
// H_{<c}; this kernel keeps the running prefix of a slice of feature rows in MFMA
// accumulators (fp32) while it walks the chunks of a sequence segment, writes the
// fp16 prefix tile of each chunk (layout in oal_tile.h) before adding the chunk,
// and adds each 16-token step as  D[(r,t)][w] += sum_tok (k_r k_t)[tok] v[tok][w]
// (A = key products in fp16, two per packed multiply; B = V in fp16; both scaled
// by powers of two taken from the segment's largest |k| and |v|).
//
// Work decomposition per (batch, KV head) unit and segment: 7 workgroups of 4 waves.
//   waves 0..23 (workgroups 0..5): the quadratic rows, as the 144 quadratic
//                 K-steps of the tile layout (oal_tile.h) taken two at a time as
//                 72 accumulator tiles of 32 rows, three per wave; row i of tile j
//                 is element i % 16 of K-step 2 j + i / 16, so every accumulator
//                 row is a stored tile row (the diagonal-block mirrors included)
//                 and lane i forms the key products k_r k_t of its own pair.
//   workgroup 6:  wave 0 the linear rows H1_r (A = K^T) and H0 = sum v, z1 = sum k,
//                 z0 = count; wave 1 the all-ones channel Z_rt = sum k_r k_t
//                 (A = K^T, B = K); waves 2, 3 only help copy the blocks.
// Each computing wave holds 3 (quadratic) or 2 (side) accumulator tiles of 32
// rows x 2 channel halves.
//
// The running prefix is summed into, and seeded from, per-(unit, segment) buffers
// in the raw accumulator layout (sums in fp32; the starting prefixes of the
// quadratic rows as fp16 in the tiles' scale, the precision they are stored in
// anyway, those of the side workgroup in fp32: the all-ones channel and H0 are
// not covered by the tiles' bound); the segment-scan kernel
// converts between that layout and the canonical state (initial state in, final
// state out).
// A batch-1 long sequence has too few units to fill 256 CUs, so the sequence is
// cut into S segments:  pass 1 (sum mode) adds up every segment,  the scan forms
// each segment's starting prefix (plus the caller's initial state) and the final
// state,  pass 2 (prefix mode) replays each segment writing the per-chunk tiles
// (up to the segment's last chunk, whose sum no tile needs).  With enough units
// for at most two segments and a sequence that starts empty, one pass (mode 2)
// walks each whole sequence, writing the tiles and, at its end, the final state
// straight in the canonical layout.
//
// fp16 tiles need a scale: every entry of every prefix of a unit is bounded by
//   B = max |H_init| + sum_j beta_j,   beta_j = max(|k_j|, |k_j|^2) |v_j|
// (|.| the largest magnitude of a vector), since each entry of H1 and H2 is a sum
// of k_r v_w or k_r k_t v_w over the tokens.  The staging pass adds up beta per
// block, the first pass takes max |H_init|, and pass 2 stores H * 2^-e_S with
// 2^(e_S + 15) > B, so that no entry exceeds 2^15 (the fp16 limit is 65504).
#include "oal_tile.h"

namespace oal {

namespace st {
constexpr int WAVES_PER_WG = 4;
constexpr int NWG = 7;                  // workgroups per (unit, segment): 6 quadratic, 1 side
constexpr int QTILES = 3;               // accumulator tiles per quadratic wave
static_assert(24 * QTILES * 2 == tile::NKS - tile::NKS_LIN, "two K-steps per tile");
// Slots of the per-(unit, segment) buffers, in the raw accumulator layout
// [register][lane]: quadratic wave omega at omega * QSLOT_FLOATS, then the side
// slot (H1 registers 0..63 from wave 0, Z 64..127 from wave 1, then H0, z1, z0).
constexpr int QSLOT_REGS = QTILES * 2 * 16;   // 96
constexpr int QSLOT_FLOATS = QSLOT_REGS * 64;
constexpr int SIDE_REGS = 132;
constexpr int SIDE_FLOATS = SIDE_REGS * 64;
constexpr int QUAD_SEG_FLOATS = 24 * QSLOT_FLOATS;             // the quadratic waves
constexpr int UNIT_SEG_FLOATS = QUAD_SEG_FLOATS + SIDE_FLOATS;  // one (unit, segment)
constexpr int TB = 64;                  // tokens staged per block
constexpr int STG_BYTES = (DH + DV) * TB * 2;   // one staged block: k^T, v^T in fp16
constexpr int REG_H0 = 128, REG_Z1 = 129, REG_Z0 = 130;
}  // namespace st

// Canonical location (row f, channel w) of accumulator register `reg` of `lane`
// in quadratic wave `omega` (24: the side slot).  valid: the element is a real
// state entry; primary: it is the stored copy of its pair (the tile rows also
// hold mirrors).
__host__ __device__ inline void state_elem(int omega, int reg, int lane, int& f, int& w,
                                           bool& valid, bool& primary) {
  const int h = lane >> 5, col = lane & 31;
  f = 0;
  w = 0;
  valid = true;
  primary = true;
  if (omega < 24) {
    const int m = reg >> 5, nt = (reg >> 4) & 1, i = reg & 15;
    const int row = 8 * (i >> 2) + 4 * h + (i & 3);
    int r, t;
    tile::quad_rt(tile::NKS_LIN + 2 * (st::QTILES * omega + m) + (row >> 4), row & 15, r, t);
    w = 32 * nt + col;
    primary = r <= t;
    f = 1 + DH + pair_index(r < t ? r : t, r < t ? t : r);
    return;
  }
  if (reg >= 128) {   // H0, z1, z0
    valid = (reg != st::REG_Z0 || lane == 0) && reg <= st::REG_Z0;
    if (reg == st::REG_H0) { f = 0; w = lane; }
    else if (reg == st::REG_Z1) { f = 1 + lane; w = DV; }
    else { f = 0; w = DV; }
    return;
  }
  const int m = reg >> 5, nt = (reg >> 4) & 1, i = reg & 15;
  const int row = 8 * (i >> 2) + 4 * h + (i & 3);
  if (m < 2) {               // linear rows
    f = 1 + 32 * m + row;
    w = 32 * nt + col;
    return;
  }
  const int r = 32 * (m - 2) + row, t = 32 * nt + col;   // Z_rt
  f = 1 + DH + pair_index(r < t ? r : t, r < t ? t : r);
  w = DV;
  primary = r <= t;
}

namespace {

// Byte offset of element `tok` (0..63) of transposed row d in a staged block:
// each row holds the block's 64 tokens (128 bytes), its 16-byte chunks swizzled
// by row_key(d) so that the lanes of every read and write hit distinct banks.
__device__ __forceinline__ int st_off(int d, int tok) {
  return d * 128 + (((tok >> 3) ^ row_key(d)) << 4) + ((tok & 7) << 1);
}

// Stage one block of TB tokens: global (token-major) -> registers -> LDS
// (dimension-major).  Thread t holds dims 8 (t & 7) .. + 7 of the tokens
// 2 (t >> 3) and 2 (t >> 3) + 1, so that each LDS write stores both tokens of a
// dim as one 32-bit word; the 8 threads of a token are consecutive lanes.  The
// quadratic workgroups stage fp16 values times a power of two; the side
// workgroup stages the raw bf16 bits.
struct Stager {
  const uint16_t* k;
  const uint16_t* v;
  size_t row0;
  int tok_end;
  uint4 pk[2], pv[2];
  __device__ void fetch(int t0, int tid) {
    const int i = tid >> 3, part = tid & 7;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int gt = t0 + 2 * i + e;
      if (gt < tok_end) {
        pk[e] = reinterpret_cast<const uint4*>(k + (row0 + gt) * DH)[part];
        pv[e] = reinterpret_cast<const uint4*>(v + (row0 + gt) * DV)[part];
      } else {
        pk[e] = make_uint4(0, 0, 0, 0);
        pv[e] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  // word of dim 2 j + hi of both tokens
  static __device__ __forceinline__ uint32_t bf16_pair(uint32_t w0, uint32_t w1, int hi) {
    return hi ? (w0 >> 16) | (w1 & 0xffff0000u) : (w0 & 0xffffu) | (w1 << 16);
  }
  static __device__ __forceinline__ uint32_t f16_pair(uint32_t w0, uint32_t w1, int hi, float s) {
    const float a = __uint_as_float(hi ? (w0 & 0xffff0000u) : (w0 << 16));
    const float b = __uint_as_float(hi ? (w1 & 0xffff0000u) : (w1 << 16));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a * s, b * s}, f16x2));
  }
  template <bool F16>
  __device__ void deposit(uint8_t* skt, uint8_t* svt, int tid, float ks, float vs) {
    const int i = tid >> 3, part = tid & 7;
    const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&pk[0]);
    const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&pk[1]);
    const uint32_t* b0 = reinterpret_cast<const uint32_t*>(&pv[0]);
    const uint32_t* b1 = reinterpret_cast<const uint32_t*>(&pv[1]);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int d = part * 8 + x;
      const int off = st_off(d, 2 * i);
      const uint32_t wk = F16 ? f16_pair(a0[x >> 1], a1[x >> 1], x & 1, ks) : bf16_pair(a0[x >> 1], a1[x >> 1], x & 1);
      const uint32_t wv = F16 ? f16_pair(b0[x >> 1], b1[x >> 1], x & 1, vs) : bf16_pair(b0[x >> 1], b1[x >> 1], x & 1);
      *reinterpret_cast<uint32_t*>(skt + off) = wk;
      *reinterpret_cast<uint32_t*>(svt + off) = wv;
    }
  }
};

// Four fp32 accumulators times the tile scale s, as fp16 (round to nearest even).
__device__ __forceinline__ uint2 pack4_f16(float a, float b, float c, float d, float s) {
  const f16x2 lo = __builtin_convertvector((f32x2){a * s, b * s}, f16x2);
  const f16x2 hi = __builtin_convertvector((f32x2){c * s, d * s}, f16x2);
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Tile exponent e_S of a unit from the bound pieces (identical in every wave that
// evaluates it: the summation order is fixed).  bound: [units][n_blk] per-block
// sums of beta, then [units][nip] partial maxima of |H_init|.
__device__ __forceinline__ int tile_scale_exp(const float* bound, int units, int n_blk, int nip,
                                              int unit, int lane) {
  // 8 loads in flight per lane and round (a rolled loop of single loads waits out
  // the memory latency once per 64 entries); the sum keeps the entry order
  constexpr int R = 8;
  float sum = 0.f, mx = 0.f;
  for (int i0 = lane; i0 < n_blk; i0 += 64 * R) {
    float x[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int i = i0 + 64 * j;
      x[j] = i < n_blk ? bound[(size_t)unit * n_blk + i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) sum += x[j];
  }
  for (int i0 = lane; i0 < nip; i0 += 64 * R) {
    float x[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int i = i0 + 64 * j;
      x[j] = i < nip ? bound[(size_t)units * n_blk + (size_t)unit * nip + i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) mx = fmaxf(mx, x[j]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sum += __shfl_xor(sum, o, 64);
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  }
  sum = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sum)));
  mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));
  const float B = mx + sum;
  int e = 0;
  if (B > 0.f) {
    int ex;
    frexpf(B, &ex);   // B < 2^ex
    e = ex - 15;
  }
  return min(max(e, -40), 100);
}

// e with x < 2^e for x > 0; 0 otherwise.
__device__ __forceinline__ int st_exp_above(float x) {
  int e = 0;
  if (x > 0.f) frexpf(x, &e);
  return e;
}

// Wait until at most x (>= 0, any value) vector-memory operations of this wave
// are outstanding, and for its LDS reads: the largest immediate not above x.
__device__ __forceinline__ void wait_vm_upto(int x) {
  if (x >= 63) wait_vmcnt<63, true>();
  else if (x >= 50) wait_vmcnt<50, true>();
  else if (x >= 36) wait_vmcnt<36, true>();
  else if (x >= 32) wait_vmcnt<32, true>();
  else if (x >= 20) wait_vmcnt<20, true>();
  else if (x >= 16) wait_vmcnt<16, true>();
  else if (x >= 4) wait_vmcnt<4, true>();
  else wait_vmcnt<0, true>();
}

}  // namespace

// Largest |k| and |v| of each (unit, segment), as KVP partial maxima over
// interleaved token ranges: the fp16 staging scales of the quadratic workgroups.
// One workgroup per (segment, part, unit).  The nip = gridDim.x workgroups of a
// unit also copy its initial state (when there is one) to init, in nip pieces,
// so that the segment scan can overwrite the state with the final one, and
// record the largest |H_init| of each piece in bmax (when not null).
constexpr int KVP = 8;
__global__ void __launch_bounds__(256)
k_state_kvmax(int seq_len, int chunk, int n_chunks, int cps, const uint16_t* __restrict__ k,
              const uint16_t* __restrict__ v, float* __restrict__ kvmax,
              const float* __restrict__ state, float* __restrict__ init, float* __restrict__ bmax) {
  __shared__ uint32_t s_m[3][4];
  const int seg = blockIdx.x / KVP, part = blockIdx.x % KVP, unit = blockIdx.y;
  const int nip = gridDim.x;
  const int n_seg = gridDim.x / KVP;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int s_begin = seg * cps * chunk;
  const int s_end = min(seq_len, min(n_chunks, (seg + 1) * cps) * chunk);
  const int per = (s_end - s_begin + KVP - 1) / KVP;
  const int t_begin = s_begin + part * per;
  const int t_end = min(s_end, t_begin + per);
  const size_t row0 = (size_t)unit * seq_len;
  uint32_t mk = 0, mv = 0, mi = 0;   // mi: largest |H_init| as bits (non-negative floats order alike)
  if (state != nullptr) {
    // eight 16-byte loads of each thread in flight per round (with a few workgroups
    // per unit a thread copies dozens: one at a time, each would wait out the
    // memory latency); a clamped duplicate leaves the maximum alone
    constexpr int CB = 8;
    const int per = (int)((STATE_FLOATS / 4 + nip - 1) / nip);
    const int i0 = blockIdx.x * per, i1 = min((int)(STATE_FLOATS / 4), i0 + per);
    const float4* src = reinterpret_cast<const float4*>(state + (size_t)unit * STATE_FLOATS);
    float4* dst = reinterpret_cast<float4*>(init + (size_t)unit * STATE_FLOATS);
    for (int ib = i0 + tid; ib < i1; ib += 256 * CB) {
      float4 x[CB];
#pragma unroll
      for (int e = 0; e < CB; ++e) x[e] = src[min(ib + 256 * e, i1 - 1)];
#pragma unroll
      for (int e = 0; e < CB; ++e) {
        if (ib + 256 * e < i1) dst[ib + 256 * e] = x[e];
        mi = max(mi, __float_as_uint(fmaxf(fmaxf(fabsf(x[e].x), fabsf(x[e].y)),
                                           fmaxf(fabsf(x[e].z), fabsf(x[e].w)))));
      }
    }
  }
  // four rounds of 16-byte loads in flight at a time (a clamped duplicate leaves the
  // maximum alone); one at a time, each would wait out the memory latency
  const int np = (t_end - t_begin) * 8;
  constexpr int KB = 4;
  for (int p0 = 0; p0 < np; p0 += 256 * KB) {
    uint4 xk[KB], xv[KB];
#pragma unroll
    for (int e = 0; e < KB; ++e) {
      const int p = min(p0 + tid + 256 * e, np - 1);
      const size_t row = row0 + t_begin + (p >> 3);
      xk[e] = reinterpret_cast<const uint4*>(k + row * DH)[p & 7];
      xv[e] = reinterpret_cast<const uint4*>(v + row * DV)[p & 7];
    }
#pragma unroll
    for (int e = 0; e < KB; ++e) {
      mk = max(mk, absmax8_bits(xk[e]));
      mv = max(mv, absmax8_bits(xv[e]));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mk = max(mk, (uint32_t)__shfl_xor((int)mk, o, 64));
    mv = max(mv, (uint32_t)__shfl_xor((int)mv, o, 64));
    mi = max(mi, (uint32_t)__shfl_xor((int)mi, o, 64));
  }
  if (lane == 0) {
    s_m[0][wv] = mk;
    s_m[1][wv] = mv;
    s_m[2][wv] = mi;
  }
  __syncthreads();
  if (tid < 3) {
    const uint32_t m = max(max(s_m[tid][0], s_m[tid][1]), max(s_m[tid][2], s_m[tid][3]));
    if (tid < 2) kvmax[(((size_t)unit * n_seg + seg) * KVP + part) * 2 + tid] = __uint_as_float(m << 16);
    else if (bmax != nullptr) bmax[(size_t)unit * nip + blockIdx.x] = __uint_as_float(m);
  }
}

// Largest |k| (which = 0) or |v| (which = 1) of a (unit, segment).
__device__ __forceinline__ float seg_max(const float* kvmax, int unit, int n_seg, int seg, int which) {
  const float* p = kvmax + ((size_t)unit * n_seg + seg) * KVP * 2 + which;
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < KVP; ++i) m = fmaxf(m, p[2 * i]);
  return m;
}

// One 64-token block of one unit, staged once for both builder passes: k^T then
// v^T (64 rows of 128 bytes each), fp16 times the segment's scales 2^-e_k and
// 2^-e_v, in the st_off layout, so that the passes fill LDS with straight
// direct-to-LDS copies.  Also adds up beta over the block for the tile-scale
// bound: bound[unit * n_blk + blk].  One workgroup per (block, unit).
__global__ void __launch_bounds__(256)
k_state_stage(int seq_len, int chunk, int n_seg, int cps, const uint16_t* __restrict__ k,
              const uint16_t* __restrict__ v, const float* __restrict__ kvmax,
              uint8_t* __restrict__ stg, float* __restrict__ bound) {
  __shared__ __attribute__((aligned(16))) uint8_t s_img[st::STG_BYTES];
  __shared__ float s_bred[4];
  const int blk = blockIdx.x, unit = blockIdx.y, n_blk = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int t0 = blk * st::TB;
  const int seg = t0 / (cps * chunk);
  const int e_k = st_exp_above(seg_max(kvmax, unit, n_seg, seg, 0)) - 7;
  const int e_v = st_exp_above(seg_max(kvmax, unit, n_seg, seg, 1)) - 7;
  Stager sg{k, v, (size_t)unit * seq_len, seq_len, {}, {}};
  sg.fetch(t0, tid);
  if (bound != nullptr) {
    // beta_j = max(|k_j|, |k_j|^2) |v_j| of the thread's two tokens (8 lanes each)
    float beta = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float km = __uint_as_float(absmax8_bits(sg.pk[e]) << 16);
      float vm = __uint_as_float(absmax8_bits(sg.pv[e]) << 16);
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        km = fmaxf(km, __shfl_xor(km, o, 64));
        vm = fmaxf(vm, __shfl_xor(vm, o, 64));
      }
      if ((tid & 7) == 0) beta += fmaxf(km, km * km) * vm;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) beta += __shfl_xor(beta, o, 64);
    if (lane == 0) s_bred[wv] = beta;
  }
  sg.deposit<true>(s_img, s_img + DH * 128, tid, ldexpf(1.0f, -e_k), ldexpf(1.0f, -e_v));
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(stg + ((size_t)unit * n_blk + blk) * st::STG_BYTES);
#pragma unroll
  for (int i = 0; i < st::STG_BYTES / 16 / 256; ++i)
    dst[i * 256 + tid] = reinterpret_cast<const uint4*>(s_img)[i * 256 + tid];
  if (bound != nullptr && tid == 0)
    bound[(size_t)unit * n_blk + blk] = (s_bred[0] + s_bred[1]) + (s_bred[2] + s_bred[3]);
}

// MODE 0: segment sums; 1: per-chunk prefix tiles from the segments' starting
// prefixes; 2: one segment from zero, the tiles and the sum in one pass.
template <int MODE>
__global__ void __launch_bounds__(256, 2)
k_state_mfma(int seq_len, int chunk, int n_chunks, int n_seg, int cps, int n_blk,
             const uint8_t* __restrict__ stg,     // staged blocks (k_state_stage)
             float* __restrict__ segsum,          // MODE 0, 2: out sums
             const uint16_t* __restrict__ segpre, // MODE 1: starting prefixes of waves 0..23, fp16 times 2^-e_S
             const float* __restrict__ sidepre,   // MODE 1: starting prefixes of wave 24
             uint8_t* __restrict__ ts,            // MODE 1, 2: per-chunk prefix tiles
             const float* __restrict__ bound,     // MODE 1, 2: tile-scale bound
             const float* __restrict__ kvmax,     // per (unit, segment): max |k|, max |v|
             int units, int nip,
             float* __restrict__ state_out) {     // MODE 2: the final state (canonical), or null
  // three staged blocks in flight: block i is read while i + 1 and i + 2 load
  __shared__ __attribute__((aligned(16))) uint8_t s_b0[st::STG_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_b1[st::STG_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_b2[st::STG_BYTES];

  // Workgroups are dealt to the 8 XCDs round robin (XCD = blockIdx mod 8); the 7
  // workgroups of a (unit, segment) sit on one XCD, so that its L2 serves their
  // shared reads of the staged blocks.  The grid is padded to whole rounds.
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int g = j % st::NWG;
  const int us = (j / st::NWG) * 8 + xcd;   // unit * n_seg + seg
  if (us >= units * n_seg) return;
  const int seg = us % n_seg;
  const int unit = us / n_seg;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int c0 = seg * cps;
  const int c1 = min(n_chunks, c0 + cps);
  const int tok_begin = c0 * chunk;
  const int tok_end = min(seq_len, c1 * chunk);
  const int n_blocks = (tok_end - tok_begin + st::TB - 1) / st::TB;
  // Blocks copied and added.  Prefix mode stores each chunk's tile before adding
  // the chunk; the sum over the segment's last chunk is no tile's prefix (the
  // scan forms the final state from the segment sums), so that mode adds the
  // blocks before the last chunk only and stores the last tile after them.
  const int n_add = MODE == 1 ? (c1 - 1 - c0) * chunk / st::TB : n_blocks;
  constexpr bool TILES = MODE != 0;   // per-chunk prefix tiles stored
  constexpr bool SUMS = MODE != 1;    // the segment's sum stored
  const uint8_t* sblk = stg + ((size_t)unit * n_blk + tok_begin / st::TB) * st::STG_BYTES;
  float* segslot = segsum + ((size_t)unit * n_seg + seg) * st::UNIT_SEG_FLOATS;
  const uint16_t* preslot = segpre + ((size_t)unit * n_seg + seg) * st::QUAD_SEG_FLOATS;
  // Where a sum goes: its raw slot (MODE 0), or the canonical final state (MODE 2,
  // each entry from its stored copy; with no state, nowhere).
  float* ustate = state_out ? state_out + (size_t)unit * STATE_FLOATS : nullptr;
  const bool put_sums = MODE == 0 || (MODE == 2 && ustate != nullptr);
  auto put = [&](float* slot_, int omega_, int reg, float x) __attribute__((always_inline)) {
    if (MODE == 0) {
      slot_[(size_t)reg * 64 + lane] = x;
      return;
    }
    int f, w;
    bool valid, primary;
    state_elem(omega_, reg, lane, f, w, valid, primary);
    if (valid && primary) ustate[(size_t)w * DS + f] = x;
  };
  // staged values are k 2^-e_k and v 2^-e_v
  const int e_k = st_exp_above(seg_max(kvmax, unit, n_seg, seg, 0)) - 7;
  const int e_v = st_exp_above(seg_max(kvmax, unit, n_seg, seg, 1)) - 7;
  // with tiles: the tile scale 2^-e_S of this unit
  const int e_s = TILES ? tile_scale_exp(bound, units, n_blk, nip, unit, lane) : 0;
  const float tscale = ldexpf(1.0f, -e_s);

  // Copies block bi of the segment into buf: PIECES 1 KB pieces per wave.
  auto issue = [&](int bi, uint8_t* buf, auto pieces) {
    constexpr int P = decltype(pieces)::value;
    const i32x4 rs = buffer_rsrc(sblk + (size_t)bi * st::STG_BYTES, (uint32_t)st::STG_BYTES);
    const uint32_t dst = lds_addr(buf) + wv * P * 1024;
#pragma unroll
    for (int j = 0; j < P; ++j) load_lds16(rs, dst + j * 1024, lane * 16, (wv * P + j) * 1024);
  };

  using P4 = std::integral_constant<int, 4>;
  if (n_add > 0) issue(0, s_b0, P4{});
  if (n_add > 1) issue(1, s_b1, P4{});

  if (g < st::NWG - 1) {
    // ===================== quadratic rows (waves 0..23) =====================
    // The accumulators hold the sums times 2^-(2 e_k + e_v).
    const float unscale = ldexpf(1.0f, 2 * e_k + e_v);
    const float rescale = ldexpf(1.0f, e_s - (2 * e_k + e_v));   // seed -> accumulator
    const int omega = g * st::WAVES_PER_WG + wv;
    float* slot = segslot + (size_t)omega * st::QSLOT_FLOATS;
    const uint16_t* pslot = preslot + (size_t)omega * st::QSLOT_FLOATS;
    // K-step of tile m's first row; this lane's pair (r, t) = A row `col` of tile m
    int ks0[st::QTILES], ra[st::QTILES], ta[st::QTILES];
#pragma unroll
    for (int m = 0; m < st::QTILES; ++m) {
      ks0[m] = tile::NKS_LIN + 2 * (st::QTILES * omega + m);
      tile::quad_rt(ks0[m] + (col >> 4), col & 15, ra[m], ta[m]);
    }
    f32x16 acc[st::QTILES][2];
#pragma unroll
    for (int m = 0; m < st::QTILES; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[m][nt][i] = MODE == 1 ? (float)__builtin_bit_cast(_Float16, pslot[(size_t)((m * 2 + nt) * 16 + i) * 64 + lane]) * rescale
                                    : 0.f;
    const float wscale = unscale * tscale;   // accumulator -> tile entry
    // tile stores per chunk start: every tile, one 16-byte store per (tile, column half, K-step)
    constexpr int NST = st::QTILES * 2 * 2;   // store instructions per tile store (per lane)
    auto stores_at = [&](int b) { return (TILES && b >= 0 && (b * st::TB) % chunk == 0) ? NST : 0; };

    // The running prefix is chunk (t0 / chunk)'s exclusive prefix: store it;
    // rows 8 gq + 4 half .. + 3 of tile m are elements of one K-step.
    auto store_tile = [&](int t0) {
      uint16_t* tl = reinterpret_cast<uint16_t*>(ts + ((size_t)unit * n_chunks + t0 / chunk) * tile::BYTES);
#pragma unroll
      for (int m = 0; m < st::QTILES; ++m) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int w = 32 * nt + col;
          // K-step ks0 + kk holds rows 8 kk .. 8 kk + 7 of the lane pair (lane,
          // lane ^ 32): elements 4 half .. + 3 and 8 + 4 half .. + 3 of the 16 of
          // column w.  One exchange gives each lane 8 contiguous elements, so that
          // every store writes 16 contiguous bytes (the pass is about 9 % faster
          // than with two 8-byte stores per lane, measured)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int ks_ = ks0[m] + kk;
            const uint2 A = pack4_f16(acc[m][nt][8 * kk], acc[m][nt][8 * kk + 1], acc[m][nt][8 * kk + 2],
                                      acc[m][nt][8 * kk + 3], wscale);
            const uint2 B = pack4_f16(acc[m][nt][8 * kk + 4], acc[m][nt][8 * kk + 5],
                                      acc[m][nt][8 * kk + 6], acc[m][nt][8 * kk + 7], wscale);
            const uint2 X = half ? A : B;   // the half the partner lane stores
            const uint2 Y = make_uint2(__shfl_xor((int)X.x, 32, 64), __shfl_xor((int)X.y, 32, 64));
            const uint4 out = half ? make_uint4(Y.x, Y.y, B.x, B.y) : make_uint4(A.x, A.y, Y.x, Y.y);
            *reinterpret_cast<uint4*>(tl + (size_t)ks_ * 1024 + w * 16 + 8 * half) = out;
          }
          asm volatile("" ::: "memory");   // keep the conversions next to their stores
        }
      }
    };

    auto body = [&](int bi, const uint8_t* cur, uint8_t* nxt) {
      if (bi >= n_add) return;
      // Block bi has landed, for every wave.  Memory operations complete in issue
      // order, and the ones issued after block bi's copy may stay in flight: the
      // tile stores of the two previous blocks and the copy of block bi + 1.
      wait_vm_upto(stores_at(bi - 2) + (bi + 1 < n_add ? 4 : 0) + stores_at(bi - 1));
      barrier_nofence();
      if (bi + 2 < n_add) issue(bi + 2, nxt, P4{});
      const int t0 = tok_begin + bi * st::TB;
      if (TILES && (t0 % chunk) == 0) store_tile(t0);
      const uint8_t* kt_ = cur;
      const uint8_t* vt_ = cur + DH * 128;
#pragma unroll
      for (int kk = 0; kk < st::TB / 16; ++kk) {
        const int tk = 16 * kk + 8 * half;     // this lane's 8 tokens inside the block
        f16x8 bv[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bv[nt] = *reinterpret_cast<const f16x8*>(vt_ + st_off(32 * nt + col, tk));
#pragma unroll
        for (int m = 0; m < st::QTILES; ++m) {
          const f16x8 kr = *reinterpret_cast<const f16x8*>(kt_ + st_off(ra[m], tk));
          const f16x8 kt = *reinterpret_cast<const f16x8*>(kt_ + st_off(ta[m], tk));
          const f16x8 af = kr * kt;                                                   // k_r k_t
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[m][nt] = mfma32h(af, bv[nt], acc[m][nt]);
        }
      }
    };
    for (int bi = 0; bi < n_add; bi += 3) {
      body(bi, s_b0, s_b2);
      body(bi + 1, s_b1, s_b0);
      body(bi + 2, s_b2, s_b1);
    }
    if (MODE == 1) store_tile(tok_begin + n_add * st::TB);   // the last chunk's tile
    if (SUMS && put_sums) {
#pragma unroll
      for (int m = 0; m < st::QTILES; ++m)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) put(slot, omega, (m * 2 + nt) * 16 + i, acc[m][nt][i] * unscale);
    }
    return;
  }

  // ===================== linear rows and the all-ones channel ================
  // All four waves copy the blocks; wave 0 adds up H1 = K^T V and H0, z1, z0,
  // wave 1 Z = K^T K.  Sums held scaled: H1 by 2^-(e_k + e_v), Z by 2^-2 e_k,
  // H0 by 2^-e_v, z1 by 2^-e_k.
  const bool lin = wv == 0, ones = wv == 1;
  float* slot = segslot + st::QUAD_SEG_FLOATS;
  const float* pslot = sidepre + ((size_t)unit * n_seg + seg) * st::SIDE_FLOATS;
  const int mo = ones ? 2 : 0;   // first register tile of this wave in the side slot
  const float sc_acc = ldexpf(1.0f, ones ? 2 * e_k : e_k + e_v);
  const float sc_h0 = ldexpf(1.0f, e_v), sc_z1 = ldexpf(1.0f, e_k);
  const float inv_acc = ldexpf(1.0f, ones ? -2 * e_k : -(e_k + e_v));
  f32x16 acc[2][2];   // H1 (wave 0) or Z (wave 1): rows 32 m.., columns 32 nt..
  float side_h0 = 0.f, side_z1 = 0.f, side_z0 = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[m][nt] = splat16(0.f);
  if (MODE == 1 && (lin || ones)) {   // one branch: all loads in flight together
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[m][nt][i] = pslot[(size_t)(((mo + m) * 2 + nt) * 16 + i) * 64 + lane] * inv_acc;
  }
  if (MODE == 1 && lin) {
    side_h0 = pslot[(size_t)st::REG_H0 * 64 + lane] * ldexpf(1.0f, -e_v);
    side_z1 = pslot[(size_t)st::REG_Z1 * 64 + lane] * ldexpf(1.0f, -e_k);
    side_z0 = pslot[(size_t)st::REG_Z0 * 64];
  }
  const float h1scale = sc_acc * tscale;
  // side stores per chunk start: wave 0 16 for H1, 2 for H0 and z1, 1 or 2 by lane 0
  // (adjacent words; the lower count, so that the wait below is never short);
  // wave 1 16 for Z
  const int side_stores = lin ? 19 : ones ? 16 : 0;
  auto stores_at = [&](int b) { return (TILES && b >= 0 && (b * st::TB) % chunk == 0) ? side_stores : 0; };
  auto store_tile = [&](int t0) {
    uint8_t* slotp = ts + ((size_t)unit * n_chunks + t0 / chunk) * tile::BYTES;
    uint16_t* tl = reinterpret_cast<uint16_t*>(slotp);
    float* side = reinterpret_cast<float*>(slotp + tile::TILE_BYTES);
    if (lin) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int w = 32 * nt + col;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int r = 32 * m + 8 * gq + 4 * half;
            *reinterpret_cast<uint2*>(tl + (size_t)(r >> 4) * 1024 + w * 16 + (r & 15)) =
                pack4_f16(acc[m][nt][4 * gq], acc[m][nt][4 * gq + 1], acc[m][nt][4 * gq + 2],
                          acc[m][nt][4 * gq + 3], h1scale);
          }
          asm volatile("" ::: "memory");
        }
      side[tile::SIDE_H0 + lane] = side_h0 * sc_h0;
      side[tile::SIDE_Z1 + lane] = side_z1 * sc_z1;
      if (lane == 0) {
        side[tile::SIDE_Z0] = side_z0;
        side[tile::SIDE_SEXP] = (float)e_s;
      }
    } else if (ones) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          // Z is symmetric: block (rows r, columns t) goes to (t, r), so that each
          // lane's four consecutive rows r form one float4 of row t = 32 nt + col
          float* zb = side + tile::SIDE_Z + (32 * nt + col) * DH + 32 * m + 4 * half;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            *reinterpret_cast<float4*>(zb + 8 * gq) =
                make_float4(acc[m][nt][4 * gq] * sc_acc, acc[m][nt][4 * gq + 1] * sc_acc,
                            acc[m][nt][4 * gq + 2] * sc_acc, acc[m][nt][4 * gq + 3] * sc_acc);
          asm volatile("" ::: "memory");
        }
    }
  };
  auto body = [&](int bi, const uint8_t* cur, uint8_t* nxt) {
    if (bi >= n_add) return;
    wait_vm_upto(stores_at(bi - 2) + (bi + 1 < n_add ? 4 : 0) + stores_at(bi - 1));
    barrier_nofence();
    if (bi + 2 < n_add) issue(bi + 2, nxt, P4{});
    const int t0 = tok_begin + bi * st::TB;
    if (TILES && (t0 % chunk) == 0) store_tile(t0);
    const uint8_t* kt_ = cur;
    const uint8_t* vt_ = cur + DH * 128;
    if (lin) {
      // H0 = sum v, z1 = sum k, z0 = count over this block (row `lane`)
      const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
      float sh = 0.f, sz = 0.f;
#pragma unroll
      for (int c = 0; c < st::TB / 8; ++c) {
        const f16x8 xv = *reinterpret_cast<const f16x8*>(vt_ + st_off(lane, 8 * c));
        const f16x8 xk = *reinterpret_cast<const f16x8*>(kt_ + st_off(lane, 8 * c));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sh = __builtin_amdgcn_fdot2((f16x2){xv[2 * j], xv[2 * j + 1]}, one2, sh, false);
          sz = __builtin_amdgcn_fdot2((f16x2){xk[2 * j], xk[2 * j + 1]}, one2, sz, false);
        }
      }
      side_h0 += sh;
      side_z1 += sz;
      side_z0 += (float)min(st::TB, tok_end - t0);
    }
    if (lin || ones) {
#pragma unroll
      for (int kk = 0; kk < st::TB / 16; ++kk) {
        const int tk = 16 * kk + 8 * half;
        f16x8 ak[2], bn[2];   // A = K^T rows; B = V^T (wave 0) or K^T (wave 1) rows
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          ak[x] = *reinterpret_cast<const f16x8*>(kt_ + st_off(32 * x + col, tk));
          bn[x] = *reinterpret_cast<const f16x8*>((ones ? kt_ : vt_) + st_off(32 * x + col, tk));
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[m][nt] = mfma32h(ak[m], bn[nt], acc[m][nt]);
      }
    }
  };
  for (int bi = 0; bi < n_add; bi += 3) {
    body(bi, s_b0, s_b2);
    body(bi + 1, s_b1, s_b0);
    body(bi + 2, s_b2, s_b1);
  }
  if (MODE == 1) store_tile(tok_begin + n_add * st::TB);   // the last chunk's tile
  if (SUMS && put_sums && (lin || ones)) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) put(slot, 24, ((mo + m) * 2 + nt) * 16 + i, acc[m][nt][i] * sc_acc);
    if (lin) {
      put(slot, 24, st::REG_H0, side_h0 * sc_h0);
      put(slot, 24, st::REG_Z1, side_z1 * sc_z1);
      put(slot, 24, st::REG_Z0, lane == 0 ? side_z0 : 0.f);
    }
  }
}

// Exclusive prefix over segments (plus the initial state), in the accumulator
// layout, four consecutive elements (same wave slot and register, lanes
// 4 j .. 4 j + 3) per thread.  segpre (when not null): the starting prefixes of
// waves 0..23 as fp16 times 2^-e_S, of wave 24 in fp32 (sidepre).  state (when
// not null): receives init + the total in the canonical layout; init is the
// initial state's copy (null: zero), so no thread reads what another writes.
// A workgroup's 1024 elements are one 32 x 32 accumulator tile (16 registers of
// one wave slot).  The tiles of the quadratic slots and of H1 (the first 148
// workgroups) hold 32 channels w in their columns and, in their rows, runs of
// consecutive features of one channel; their initial and final states go through
// LDS so that the canonical reads and writes run along the features (eight
// threads per channel, four rows each) instead of striding over channels.
constexpr int SCAN_TILED_BLOCKS = (st::QUAD_SEG_FLOATS + 64 * 64) / 1024;   // 144 + 4
template <int SB>   // segments whose loads are in flight together
__global__ void __launch_bounds__(256)
k_state_segscan(int n_seg, const float* __restrict__ segsum, uint16_t* __restrict__ segpre,
                float* __restrict__ sidepre, const float* __restrict__ init, float* __restrict__ state,
                const float* __restrict__ bound, int n_blk, int nip) {
  __shared__ float s_t[32][33];
  const int unit = blockIdx.y, units = gridDim.y;
  const int tid = threadIdx.x;
  const int e0 = 4 * (blockIdx.x * blockDim.x + tid);
  const bool in = e0 < st::UNIT_SEG_FLOATS;
  const bool quad = e0 < st::QUAD_SEG_FLOATS;
  const int omega = quad ? e0 / st::QSLOT_FLOATS : 24;
  const bool tiled = blockIdx.x < SCAN_TILED_BLOCKS;   // uniform over the workgroup
  // every wave evaluates the tile scale (the same value everywhere)
  const float tscale = segpre ? ldexpf(1.0f, -tile_scale_exp(bound, units, n_blk, nip, unit, tid & 63)) : 1.f;
  float* ustate = state ? state + (size_t)unit * STATE_FLOATS : nullptr;
  const float* uinit = init ? init + (size_t)unit * STATE_FLOATS : nullptr;
  // tiled workgroups: canonical (f, w) of tile row rho, column c (rho = the
  // accumulator row, c = the lane's column), for this thread's channel c = tid / 8
  // and rows 4 (tid % 8) .. + 3
  const int reg0 = (quad ? (e0 / 64) % st::QSLOT_REGS : (e0 - st::QUAD_SEG_FLOATS) / 64) & ~15;
  const int cc = tid >> 3, rr0 = 4 * (tid & 7);
  int cf[4];
  bool cvalid[4], ckeep[4];
  if (tiled) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rho = rr0 + j;
      const int i = 4 * (rho >> 3) + (rho & 3), h = (rho >> 2) & 1;   // mrow(i, h) = rho
      int f = 0, w = 0;
      bool valid = false, primary = false;
      state_elem(omega, reg0 + i, cc + 32 * h, f, w, valid, primary);
      cf[j] = w * DS + f;
      cvalid[j] = valid;
      ckeep[j] = valid && primary;
    }
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (uinit && cvalid[j]) ? uinit[cf[j]] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s_t[rr0 + j][cc] = x[j];
    __syncthreads();
  }
  if (!in) return;   // (never in a tiled workgroup)
  float run[4];
  int fw[4];
  bool keep[4];
  const int lane0 = e0 & 63;
  const int reg = quad ? (e0 / 64) % st::QSLOT_REGS : (e0 - st::QUAD_SEG_FLOATS) / 64;
  const int trow = acc_row(reg & 15, lane0 >> 5), tcol = lane0 & 31;   // tiled: this thread's tile row
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (tiled) {
      run[j] = s_t[trow][tcol + j];
      fw[j] = 0;
      keep[j] = false;
      continue;
    }
    int f = 0, w = 0;
    bool valid = false, primary = false;
    state_elem(omega, reg, lane0 + j, f, w, valid, primary);
    fw[j] = w * DS + f;
    keep[j] = valid && primary;
    run[j] = (uinit && valid) ? uinit[fw[j]] : 0.f;
  }
  float4 r = make_float4(run[0], run[1], run[2], run[3]);
  const size_t base = (size_t)unit * n_seg * st::UNIT_SEG_FLOATS + e0;
  // the loads of SB segments are issued together (one at a time, each thread
  // would wait out the full memory latency n_seg times), unconditionally with the
  // segment index clamped, so that each use waits for its own load only (a load
  // behind a branch ends its block with a wait for every load in flight); SB
  // follows n_seg, so that few segments issue few duplicate loads
  for (int s0 = 0; s0 < n_seg; s0 += SB) {
    float4 a[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j)
      a[j] = *reinterpret_cast<const float4*>(segsum + base + (size_t)min(s0 + j, n_seg - 1) * st::UNIT_SEG_FLOATS);
#pragma unroll
    for (int j = 0; j < SB; ++j)
      if (s0 + j < n_seg) {
        if (segpre) {
          const size_t us = (size_t)unit * n_seg + s0 + j;
          if (quad) {
            const f16x2 lo = __builtin_convertvector((f32x2){r.x * tscale, r.y * tscale}, f16x2);
            const f16x2 hi = __builtin_convertvector((f32x2){r.z * tscale, r.w * tscale}, f16x2);
            *reinterpret_cast<uint2*>(segpre + us * st::QUAD_SEG_FLOATS + e0) =
                make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
          } else {
            *reinterpret_cast<float4*>(sidepre + us * st::SIDE_FLOATS + (e0 - st::QUAD_SEG_FLOATS)) = r;
          }
        }
        r.x += a[j].x;
        r.y += a[j].y;
        r.z += a[j].z;
        r.w += a[j].w;
      }
  }
  if (!ustate) return;   // (uniform)
  const float fin[4] = {r.x, r.y, r.z, r.w};
  if (tiled) {
    __syncthreads();   // every thread has taken its initial values out of s_t
#pragma unroll
    for (int j = 0; j < 4; ++j) s_t[trow][tcol + j] = fin[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (ckeep[j]) ustate[cf[j]] = s_t[rr0 + j][cc];
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (keep[j]) ustate[fw[j]] = fin[j];
}

// ---------------------------------------------------------------------------

static int choose_segments(int units, int n_chunks) {
  // as many segments as fit in one round of 2 workgroups per CU on 256 CUs: a
  // few workgroups more than the slots would add a second round of equal length
  int s = 512 / (units * st::NWG);
  if (s < 1) s = 1;
  if (s > n_chunks) s = n_chunks;
  return s;
}

static size_t stage_bytes(int units, int seq_len) {
  return (size_t)units * ((seq_len + st::TB - 1) / st::TB) * st::STG_BYTES;
}

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Scratch of the builder, in this order: segment sums, the segments' max |k| and
// |v|, the staged blocks, the initial state's copy, then (with tiles) the
// quadratic and side starting prefixes and the tile-scale bound.
struct StateWs {
  float* segsum;
  float* kvmax;
  uint8_t* stg;
  float* init;
  uint16_t* segpre;
  float* sidepre;
  float* bound;
  size_t bytes;
};

static StateWs state_ws(void* ws, int units, int seq_len, int n_seg, bool with_tiles) {
  const int n_blk = (seq_len + st::TB - 1) / st::TB;
  const int nip = n_seg * KVP;
  StateWs w{};
  size_t off = 0;
  auto take = [&](size_t b) {
    uint8_t* p = ws ? reinterpret_cast<uint8_t*>(ws) + off : nullptr;
    off += round256(b);
    return p;
  };
  w.segsum = reinterpret_cast<float*>(take((size_t)units * n_seg * st::UNIT_SEG_FLOATS * sizeof(float)));
  w.kvmax = reinterpret_cast<float*>(take((size_t)units * n_seg * KVP * 2 * sizeof(float)));
  w.stg = take(stage_bytes(units, seq_len));
  w.init = reinterpret_cast<float*>(take((size_t)units * STATE_FLOATS * sizeof(float)));
  if (with_tiles) {
    w.segpre = reinterpret_cast<uint16_t*>(take((size_t)units * n_seg * st::QUAD_SEG_FLOATS * sizeof(uint16_t)));
    w.sidepre = reinterpret_cast<float*>(take((size_t)units * n_seg * st::SIDE_FLOATS * sizeof(float)));
    w.bound = reinterpret_cast<float*>(take((size_t)units * (n_blk + nip) * sizeof(float)));
  }
  w.bytes = off;
  return w;
}

size_t state_mfma_workspace(int batch, int n_kv_heads, int seq_len, int chunk, bool with_tiles) {
  const int units = batch * n_kv_heads;
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  const int n_seg = choose_segments(units, n_chunks);
  const int cps = (n_chunks + n_seg - 1) / n_seg;
  const int n_seg_eff = (n_chunks + cps - 1) / cps;
  size_t bytes = state_ws(nullptr, units, seq_len, n_seg_eff, with_tiles).bytes;
  if (with_tiles) bytes += (size_t)units * n_chunks * tile::BYTES;
  return bytes;
}

// Builds the per-chunk prefix tiles (when ts != null) and the final state (when
// state != null; its content on entry is the initial state, or, with init_zero,
// ignored: the sequence starts empty and the state is only written).  ws: the
// scratch part of state_mfma_workspace (see state_ws).
oal_status launch_state_mfma(int batch, int n_kv_heads, int seq_len, int chunk, const void* k,
                             const void* v, float* state, bool init_zero, uint8_t* ts, void* ws,
                             hipStream_t stream) {
  const float* init_src = init_zero ? nullptr : state;   // the initial state, when one is read
  const int units = batch * n_kv_heads;
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  // With enough units for at most two segments and a sequence that starts empty,
  // one pass walks whole sequences storing both the tiles and the sums (the final
  // state's), instead of a sum pass over two segments before the tile pass.
  const bool one_pass = ts != nullptr && init_src == nullptr && choose_segments(units, n_chunks) <= 2;
  const int n_seg = one_pass ? 1 : choose_segments(units, n_chunks);
  const int cps = (n_chunks + n_seg - 1) / n_seg;
  const int n_seg_eff = (n_chunks + cps - 1) / cps;
  const int n_blk = (seq_len + st::TB - 1) / st::TB;
  const int nip = n_seg_eff * KVP;
  const uint16_t* kk = reinterpret_cast<const uint16_t*>(k);
  const uint16_t* vv = reinterpret_cast<const uint16_t*>(v);
  const dim3 grid((units * n_seg_eff + 7) / 8 * 8 * st::NWG);
  const StateWs w = state_ws(ws, units, seq_len, n_seg_eff, ts != nullptr);
  {
    ProfScope ps("k_state_kvmax", stream);
    hipLaunchKernelGGL(k_state_kvmax, dim3(nip, units), dim3(256), 0, stream, seq_len, chunk,
                       n_chunks, cps, kk, vv, w.kvmax, init_src, w.init,
                       ts ? w.bound + (size_t)units * n_blk : (float*)nullptr);
    oal_status s = check_launch("k_state_kvmax");
    if (s != OAL_OK) return s;
  }
  {
    ProfScope ps("k_state_stage", stream);
    hipLaunchKernelGGL(k_state_stage, dim3(n_blk, units), dim3(256), 0, stream, seq_len, chunk, n_seg_eff,
                       cps, kk, vv, (const float*)w.kvmax, w.stg, w.bound);
    oal_status s = check_launch("k_state_stage");
    if (s != OAL_OK) return s;
  }
  if (one_pass) {   // the sums go straight into the canonical state: no scan
    ProfScope ps("k_state_mfma", stream);
    hipLaunchKernelGGL(k_state_mfma<2>, grid, dim3(256), 0, stream, seq_len, chunk, n_chunks,
                       n_seg_eff, cps, n_blk, (const uint8_t*)w.stg, w.segsum, (const uint16_t*)nullptr,
                       (const float*)nullptr, ts, (const float*)w.bound, (const float*)w.kvmax, units,
                       nip, state);
    return check_launch("k_state_mfma");
  }
  {
    ProfScope ps("k_state_seg", stream);
    hipLaunchKernelGGL(k_state_mfma<0>, grid, dim3(256), 0, stream, seq_len, chunk, n_chunks,
                       n_seg_eff, cps, n_blk, (const uint8_t*)w.stg, w.segsum, (const uint16_t*)nullptr,
                       (const float*)nullptr, (uint8_t*)nullptr, (const float*)nullptr,
                       (const float*)w.kvmax, units, nip, (float*)nullptr);
    oal_status s = check_launch("k_state_seg");
    if (s != OAL_OK) return s;
  }
  {
    ProfScope ps("k_state_segscan", stream);
    auto* fn = n_seg_eff >= 16 ? k_state_segscan<16> : n_seg_eff >= 4 ? k_state_segscan<4>
                                                                       : k_state_segscan<2>;
    hipLaunchKernelGGL(fn, dim3((st::UNIT_SEG_FLOATS / 4 + 255) / 256, units), dim3(256),
                       0, stream, n_seg_eff, (const float*)w.segsum, w.segpre, w.sidepre,
                       init_src ? (const float*)w.init : (const float*)nullptr, state,
                       (const float*)w.bound, n_blk, nip);
    oal_status s = check_launch("k_state_segscan");
    if (s != OAL_OK) return s;
  }
  if (ts == nullptr) return OAL_OK;
  ProfScope ps("k_state_mfma", stream);
  hipLaunchKernelGGL(k_state_mfma<1>, grid, dim3(256), 0, stream, seq_len, chunk, n_chunks,
                     n_seg_eff, cps, n_blk, (const uint8_t*)w.stg, w.segsum, (const uint16_t*)w.segpre,
                     (const float*)w.sidepre, ts, (const float*)w.bound, (const float*)w.kvmax, units,
                     nip, (float*)nullptr);
  return check_launch("k_state_mfma");
}

}  // namespace oal
