// Chunked causal prefill for bf16 inputs on the gfx950 matrix cores.
//
// [OAL] Algorithm 1 evaluated by chunks of C tokens (the paper's backend uses
// 128-token blocks with bf16 tensor-core contractions and fp32 coefficients,
// [OAL] App. E):
//   u~_i = phi_q(q_i)^T H_{<c}  +  sum_{j in chunk, j <= i} kappa(q_i, k_j) u_j
//   y_i  = u~_{i,1:64} / u~_{i,65}
// The inter-chunk term reads the exclusive prefix state H_{<c} of the chunk (a
// scaled fp16 copy in the tiled layout of oal_tile.h, plus fp32 side data for
// the denominator); the intra-chunk term evaluates kappa = eps + sum_p t_p^2,
// t_p = L_0p + sum_r ell_p[r] q_r k_r (the expansion of ||L^T s_bar||^2, Eq. 7)
// on the matrix cores and applies it to [V; 1].
#include <type_traits>

#include "oal_tile.h"

namespace oal {

// ---------------------------------------------------------------------------
// Readout.  Workgroup = 4 waves = (256 / C) query heads of one KV group x C
// tokens of one chunk; wave = one head x 64 tokens (token tiles sub and
// 2 WPH - 1 - sub of 32 tokens, sub = the wave's index within its head, so that
// each wave meets an equal share of the causal triangle).  In the u~^T orientation
// (rows = value channel w, columns = tokens) each wave owns a 64 x 64 tile of
// fp32 accumulators (2 x 2 MFMA tiles).
//
// Scaling.  The inter-chunk contraction runs in fp16 (A = state tile, stored as
// H 2^-e_S; B = query features built with packed fp16 multiplies).  Per head the
// query features are scaled by F_f = 2^(12 - 2 e_q - e_M - x) so that every
// fp16 operand and intermediate stays below 2^14 (|q| < 2^e_q, |M/d_h| < 2^e_M,
// x keeps the linear features in range as well).  Every other term added into
// the same accumulators or the denominator (the intra-chunk kappa, a H0, the
// inter-chunk denominator) is multiplied by the same F = 2^E, E = F_f's
// exponent - e_S: the factor cancels in y = u~_{1:64} / u~_65 and all scalings
// are exact powers of two.
//
// LDS.  Every region is a __shared__ object of its own (the q tile, four 8 KB
// buffers that hold the chunk's k rows and v^T rows for the intra-chunk part,
// the per-head tables).  Rows of 64 bf16 are 128 bytes with the 16-byte chunks
// XOR-swizzled by row_key(row) instead of padded.  The state tile is not staged:
// each wave reads its fragments from the tile in global memory (an L2 shared by
// the head groups of the chunk) one half-slab ahead.
// ---------------------------------------------------------------------------
template <int CH>
struct ReadoutCfg {
  static constexpr int WPH = CH / 64;               // waves per head
  static constexpr int HPW = 4 / WPH;               // heads per workgroup
  static constexpr int HS_BYTES = 4 * tile::KS_BYTES;   // one half-slab = 4 K-steps = 8 KB
  static constexpr int NHS = tile::NKS / 4;         // 37 half-slabs per tile
  static constexpr int Q_BYTES = HPW * CH * 128;    // = 32 KB
  // The chunk's keys are staged for the intra-chunk part in the four 8 KB
  // buffers, 128 at a time (k rows in buffers 0, 1, v^T rows in 2, 3): one pass
  // up to C = 128, two at C = 256 (which keeps the workgroup's LDS below 80 KB, so
  // that two workgroups fit a CU).  With two passes, pass p holds the 32-key tiles
  // p, p + 2, p + 4, p + 6: every wave's token tiles (t, 7 - t) then meet five key
  // tiles in the first pass and four in the second (contiguous halves gave 5 to 8
  // and 4 to 1, and the barrier between the passes waits for the slowest).
  static constexpr int KPASS = CH < 128 ? CH : 128;  // keys per staging pass
  static constexpr int NPASS = CH / KPASS;
  static constexpr int KIT = KPASS / 64;             // token pairs per thread and pass
};

// Per-head table (floats), written from the coefficient record with the head's
// scales folded in.
namespace htab {
constexpr int ELL = 0;                  // [LDIM][DH] ell_p[r] 2^(E/2)
constexpr int L0 = LDIM * DH;           // [8]  L_{0,p} 2^(E/2)
constexpr int ELLC = L0 + 8;            // [LDIM][16] (ell_p - c_p) at the compact dims, 2^(E/2)
constexpr int CIDX = ELLC + LDIM * 16;  // [16] int: the dims with g(r) >= 2 (compact path)
constexpr int CP = CIDX + 16;           // [8] c_p = L_{1,p} / sqrt(d_h) (ell_p on group 1), 2^(E/2)
constexpr int BPF = CP + 8;             // [DH] b'_r F_f
constexpr int BZ = BPF + DH;            // [DH] b'_r z1_r 2^-e_M (z1 of the chunk's prefix)
constexpr int FLOATS = BZ + DH;
}  // namespace htab


__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, 64));
  return x;
}

// e with x < 2^e for x > 0; 0 for x == 0.
__device__ __forceinline__ int exp_above(float x) {
  int e = 0;
  if (x > 0.f) frexpf(x, &e);
  return e;
}

template <bool B>
using bool_t = std::integral_constant<bool, B>;

// HALF: each wave takes one token tile (as N-tile 1) instead of two, so that a
// workgroup covers half of its head's chunk (chunk 256 only).  A half workgroup
// takes about 80 % of a whole one's time, so an item that has a round to itself
// finishes sooner as two of them (short sequences).
template <int CH, typename O, bool HALF>
__global__ void __launch_bounds__(256, 2)
k_readout_mfma(int n_q_heads, int n_kv_heads, int seq_len, int n_chunks, int n_hg, int n_uc,
               const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const float* __restrict__ coeffs,
               const uint8_t* __restrict__ ws_tile, O* __restrict__ y) {
  using Cfg = ReadoutCfg<CH>;
  static_assert(!HALF || CH == 256, "half workgroups are laid out for chunk 256");
  constexpr int NT0 = HALF ? 1 : 0;   // first N-tile of the wave
  __shared__ __attribute__((aligned(16))) uint8_t s_q[Cfg::Q_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_b0[Cfg::HS_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_b1[Cfg::HS_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_b2[Cfg::HS_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_b3[Cfg::HS_BYTES];
  __shared__ __attribute__((aligned(16))) _Float16 s_mg[Cfg::HPW * LDIM * DH];
  __shared__ __attribute__((aligned(16))) float s_ht[Cfg::HPW * htab::FLOATS];
  __shared__ float s_red[16];
  __shared__ __attribute__((aligned(16))) float s_h0[DV];   // H0 of the chunk's prefix
  // inter-chunk denominators handed to the mirror waves, per (head, wave pair)
  __shared__ float s_dx[Cfg::HPW * (Cfg::WPH > 1 ? Cfg::WPH / 2 : 1) * 64];
  // k rows (64 per array) and v^T rows (64 keys per array) of the keys staged
  // by one pass (i: 64-key block inside the pass)
  auto k_arr = [&](int i) -> uint8_t* { return i == 0 ? s_b0 : s_b1; };
  auto v_arr = [&](int i) -> uint8_t* { return i == 0 ? s_b2 : s_b3; };

  // ---- which (unit, chunk, head group): the head groups of one (unit, chunk)
  //      share an XCD (blockIdx % 8) so they hit the same L2 for the state.
  //      slot: the item's index among those of its XCD; in half mode two
  //      consecutive workgroups of an XCD share an item.
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int slot = HALF ? (L >> 4) : (L >> 3);
  const int part = HALF ? (L >> 3) & 1 : 0;
  const int uc = (slot / n_hg) * 8 + xcd;
  const int hg = slot % n_hg;
  if (uc >= n_uc) return;
  const int unit = uc / n_chunks, chunk = uc % n_chunks;
  const int b = unit / n_kv_heads, kv = unit % n_kv_heads;
  const int rep = n_q_heads / n_kv_heads;
  const int t0 = chunk * CH;
  const int clen = min(CH, seq_len - t0);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int hslot = wave / Cfg::WPH, sub = wave % Cfg::WPH;
  // Wave sub >= WPH / 2 meets one key tile fewer inside the chunk than its
  // mirror WPH - 1 - sub (token tiles below): it computes the inter-chunk
  // denominators of both (one Z operand) and hands the mirror's over through LDS.
  constexpr bool PAIRED = Cfg::WPH > 1 && !HALF;
  const bool den_giver = !PAIRED || sub >= Cfg::WPH / 2;
  const int msub = Cfg::WPH - 1 - sub;
  const int hl = hg * Cfg::HPW + hslot;
  const bool head_ok = hl < rep;
  const int hq = kv * rep + (head_ok ? hl : 0);
  const float* rec = coef_rec(coeffs, hq);
  const uint8_t* tsrc = ws_tile + ((size_t)unit * n_chunks + chunk) * tile::BYTES;
  const float* ts_side = reinterpret_cast<const float*>(tsrc + tile::TILE_BYTES);

  // ---- prologue loads, all issued before any of them is used (bounds by
  //      clamping the address and zeroing the value afterwards): q of all heads
  //      of the group, k and v of the chunk, and this wave's coefficients
  constexpr int QIT = Cfg::HPW * CH * 8 / 256;   // 16-byte q pieces per thread
  constexpr int KIT = Cfg::KIT;                  // token pairs per thread and pass
  uint4 qv[QIT];
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int hs = it * 256 / (CH * 8);          // compile-time after unrolling
    const int rem = tid + 256 * it - hs * CH * 8, tok = rem >> 3, part = rem & 7;
    const int hh = min(hg * Cfg::HPW + hs, rep - 1);
    const size_t row = ((size_t)b * n_q_heads + kv * rep + hh) * seq_len + t0 + min(tok, clen - 1);
    qv[it] = reinterpret_cast<const uint4*>(q + row * DH)[part];
  }
  // Chunk key of key s (0 .. KPASS - 1) of staging pass `pass`: staged 32-key tile
  // j is the chunk's key tile 2 j + pass with two passes, j with one.
  auto pass_key = [](int s, int pass) {
    return Cfg::NPASS == 1 ? s : 32 * (2 * (s >> 5) + pass) + (s & 31);
  };
  // k and v of a staging pass: thread t holds dims 8 (t & 7) .. + 7 of the keys
  // 64 it + 2 (t >> 3) + e of the pass
  const size_t kvrow0 = (size_t)unit * seq_len + t0;
  const int kpart = tid & 7, kpair = tid >> 3;
  uint4 kq[KIT][2], vq[KIT][2];
  auto load_kv = [&](int pass) {
#pragma unroll
    for (int it = 0; it < KIT; ++it)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const size_t row = kvrow0 + min(pass_key(64 * it + 2 * kpair + e, pass), clen - 1);
        kq[it][e] = reinterpret_cast<const uint4*>(k + row * DH)[kpart];
        vq[it][e] = reinterpret_cast<const uint4*>(v + row * DV)[kpart];
      }
  };
  load_kv(0);
  const float mval = rec[OAL_COEF_M + min(lane, LDIM * LDIM - 1)];
  const float bval = rec[OAL_COEF_BP + lane];
  const int gl = reinterpret_cast<const int32_t*>(rec)[OAL_COEF_GMAP + lane];   // g(r), lane r
  float mgv[LDIM], ellv[LDIM];
#pragma unroll
  for (int p = 0; p < LDIM; ++p) {
    mgv[p] = rec[OAL_COEF_MG + p * DH + lane];
    ellv[p] = rec[OAL_COEF_ELL + p * DH + lane];
  }
  const float l0v = rec[OAL_COEF_L + min(lane, LDIM - 1)];           // L_{0,lane}
  const float l1v = rec[OAL_COEF_L + LDIM + min(lane, LDIM - 1)];    // L_{1,lane}
  const float z1v = ts_side[tile::SIDE_Z1 + lane];
  const float h0v = ts_side[tile::SIDE_H0 + lane];   // read in the epilogue, from LDS
  const float esv = ts_side[tile::SIDE_SEXP];
  // Z rows 32 mt + col, columns 16 ks + 8 half .. + 7: the inter-chunk
  // denominator's operand.  With several waves per head (C >= 128) it is loaded
  // once the staging's loads are consumed, so that its latency overlaps the
  // reductions, barrier and tables, and the denominator is computed before the
  // intra-chunk part; with one (C = 64, four
  // heads staged, where holding it would spill) it is loaded in place, after the
  // intra-chunk part, while the first half-slab's fragments load.
  constexpr bool ZPRE = Cfg::WPH > 1;
  float4 zv[2][4][2];
  auto load_z = [&]() {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          zv[mt][ks][e] = *reinterpret_cast<const float4*>(ts_side + tile::SIDE_Z + (32 * mt + col) * DH +
                                                           16 * ks + 8 * half + 4 * e);
  };

  // ---- q tile, with each thread's max |q| per head
  uint32_t qmax[Cfg::HPW];
#pragma unroll
  for (int hs = 0; hs < Cfg::HPW; ++hs) qmax[hs] = 0;
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int hs = it * 256 / (CH * 8);
    const int rem = tid + 256 * it - hs * CH * 8, tok = rem >> 3, part = rem & 7;
    const bool ok = hg * Cfg::HPW + hs < rep && tok < clen;
    const uint4 val = ok ? qv[it] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(s_q + (hs * CH + tok) * 128 + ((part ^ row_key(tok)) << 4)) = val;
    qmax[hs] = max(qmax[hs], absmax8_bits(val));
  }
  // ---- k rows, and v^T rows with the keys of each 16-block permuted: position
  //      8h + 4a + e holds key 8a + 4h + e (the key order of the kappa accumulator
  //      rows); the two tokens of a thread are adjacent there (one 32-bit write).
  //      tok: the key inside the pass, pass_key(tok, pass) inside the chunk.
  auto stage_kv = [&](int pass) {
  // the thread's indices taken afresh: the compiler would otherwise keep the first
  // pass's LDS addresses live (spilled) across the intra-chunk part for the second
  int kpair_ = kpair, kpart_ = kpart;
  asm volatile("" : "+v"(kpair_), "+v"(kpart_));
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int tok = 64 * it + 2 * kpair_;      // even; tok + 1 is the pair's second token
    const int ctok = pass_key(tok, pass);     // tok even: ctok + 1 is the pair's second key
    const bool ok0 = ctok < clen, ok1 = ctok + 1 < clen;
    const uint4 k0 = ok0 ? kq[it][0] : make_uint4(0, 0, 0, 0);
    const uint4 k1 = ok1 ? kq[it][1] : make_uint4(0, 0, 0, 0);
    const uint4 v0 = ok0 ? vq[it][0] : make_uint4(0, 0, 0, 0);
    const uint4 v1 = ok1 ? vq[it][1] : make_uint4(0, 0, 0, 0);
    uint8_t* ka = k_arr(tok >> 6);
    *reinterpret_cast<uint4*>(ka + (tok & 63) * 128 + ((kpart_ ^ row_key(tok & 63)) << 4)) = k0;
    *reinterpret_cast<uint4*>(ka + ((tok + 1) & 63) * 128 + ((kpart_ ^ row_key((tok + 1) & 63)) << 4)) = k1;
    const int pos = (tok & ~15) | (((tok >> 2) & 1) << 3) | (((tok >> 3) & 1) << 2) | (tok & 3);
    uint8_t* va = v_arr(pos >> 6);
    const int pk = pos & 63;
    const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&v0);
    const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&v1);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int w = kpart_ * 8 + x;
      const uint32_t word = (x & 1) ? (a0[x >> 1] >> 16) | (a1[x >> 1] & 0xffff0000u)
                                    : (a0[x >> 1] & 0xffffu) | (a1[x >> 1] << 16);
      *reinterpret_cast<uint32_t*>(va + w * 128 + (((pk >> 3) ^ row_key(w)) << 4) + ((pk & 7) << 1)) = word;
    }
  }
  };
  stage_kv(0);

  // (after the staging's last use of its loads: memory operations complete in
  // order, so no later wait of the staging waits for these)
  __builtin_amdgcn_sched_barrier(0);
  if (ZPRE && den_giver) load_z();
  // ---- this head's coefficient magnitudes (wave-uniform)
  const int e_m = exp_above(wave_max(lane < LDIM * LDIM ? fabsf(mval) * (1.0f / DH) : 0.f));
  const int e_b = exp_above(wave_max(fabsf(bval)));
  if (head_ok && sub == 0) {   // fp16 table M_{gamma,g(t)} / d_h 2^-e_M of the head
    _Float16* mg = s_mg + hslot * LDIM * DH;
    const float sc = ldexpf(1.0f, -e_m);
#pragma unroll
    for (int p = 0; p < LDIM; ++p) mg[p * DH + lane] = (_Float16)(mgv[p] * sc);
  }
#pragma unroll
  for (int hs = 0; hs < Cfg::HPW; ++hs) {
    const uint32_t m = wave_umax(qmax[hs]);
    if (lane == 0) s_red[wave * 4 + hs] = __uint_as_float(m << 16);
  }
  if (wave == 0) s_h0[lane] = h0v;
  __syncthreads();

  // ---- the head's scales (identical in the waves of one head)
  const float qm = fmaxf(fmaxf(s_red[0 * 4 + hslot], s_red[1 * 4 + hslot]),
                         fmaxf(s_red[2 * 4 + hslot], s_red[3 * 4 + hslot]));
  const int e_q = exp_above(qm);
  const int e_s = (int)esv;
  int xs = max(0, e_b - e_q - e_m - 3);
  int E = -e_s + 12 - 2 * e_q - e_m - xs;
  if (E & 1) {   // even, so that sqrt(F) is a power of two as well
    ++xs;
    --E;
  }
  const float F = ldexpf(1.0f, E);
  const float sroot = ldexpf(1.0f, E / 2);
  const float Ff = ldexpf(1.0f, 12 - 2 * e_q - e_m - xs);
  const float qt_scale = ldexpf(1.0f, 6 - e_q - xs);
  const float qr_scale = ldexpf(1.0f, 6 - e_q);

  // ---- per-head table; both waves of a head write the same values, and each
  //      wave only reads back what it wrote itself (LDS ops of a wave are ordered)
  const int G = reinterpret_cast<const int32_t*>(rec)[OAL_COEF_NG];
  float* ht = s_ht + hslot * htab::FLOATS;
  const uint64_t cmask = __ballot(gl >= 2);   // dims of the groups 2..G
  const int n_out = __popcll(cmask);
  const bool compact = n_out <= 14;            // t_p from one 16-deep K-step (+ 2 constant slots)
  if (head_ok) {
#pragma unroll
    for (int p = 0; p < LDIM; ++p) ht[htab::ELL + p * DH + lane] = ellv[p] * sroot;
    if (lane < LDIM) ht[htab::L0 + lane] = l0v * sroot;
    if (lane < LDIM) ht[htab::CP + lane] = l1v * (0.125f * sroot);
    ht[htab::BPF + lane] = bval * Ff;
    ht[htab::BZ + lane] = bval * z1v * ldexpf(1.0f, -e_m);
    if (compact) {
      int* cidx = reinterpret_cast<int*>(ht + htab::CIDX);
      float c1[LDIM];   // L_{1,p} / sqrt(d_h), read across lanes before the branches below
      float l0s[LDIM];  // L_{0,p} 2^(E/2)
#pragma unroll
      for (int p = 0; p < LDIM; ++p) {
        c1[p] = __shfl(l1v, p, 64) * 0.125f;
        l0s[p] = __shfl(l0v, p, 64) * sroot;
      }
      if (gl >= 2) {
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(cmask >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)cmask, 0));
        cidx[rank] = lane;
#pragma unroll
        for (int p = 0; p < LDIM; ++p)
          ht[htab::ELLC + p * 16 + rank] = (ellv[p] - c1[p]) * sroot;
      }
      if (lane >= n_out && lane < 16) {
        // slots 14 and 15 carry L_{0,p} (a bf16-exact high part and the rest)
        // against key and query entries of 1: the product's constant term
        cidx[lane] = 0;
#pragma unroll
        for (int p = 0; p < LDIM; ++p) {
          const float hi = __uint_as_float(__float_as_uint(l0s[p]) & 0xffff0000u);
          ht[htab::ELLC + p * 16 + lane] = lane == 14 ? hi : lane == 15 ? l0s[p] - hi : 0.f;
        }
      }
    }
  }

  // token tiles of this wave (32 tokens each): sub and 2 WPH - 1 - sub, so that
  // the waves of a head meet equal parts of the causal triangle inside the chunk
  // (half mode: the one tile, as N-tile 1, is 7, 0, 5, 2 in part 0 and 6, 1, 4, 3
  // in part 1, so that the two workgroups of an item meet 15 and 13 key tiles)
  const int T1 = HALF ? ((sub & 1) ? sub - 1 + part : 7 - sub - part) : 2 * Cfg::WPH - 1 - sub;
  const int T0 = HALF ? T1 : sub;
  const uint8_t* qw = s_q + hslot * CH * 128;
  const SwRow qrow0(qw, 32 * T0 + col), qrow1(qw, 32 * T1 + col);   // tokens of N-tiles 0, 1
  // q fragment (B operand, columns = tokens, K = head dims): exact bf16 inputs
  auto qfrag = [&](int nt, int ks) {
    return *reinterpret_cast<const bf16x8*>((nt ? qrow1 : qrow0).chunk(2 * ks + half));
  };

  float den[2] = {0.f, 0.f};   // this lane's partial denominators of tokens (col, nt), times F
  f32x16 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = splat16(0.f);

  // ---- inter-chunk denominator: a z0 + sum_r q_r (b'_r z1_r + ((C / d_h o Z) q)_r),
  //      T = b' o z1 + (C/d_h o Z) q^T on the matrix cores (the first term as the
  //      accumulator seed); C/d_h from the head's M_{g(n),g(t)}/d_h 2^-e_M table
  float* dx = s_dx + (hslot * (PAIRED ? Cfg::WPH / 2 : 1) + min(sub, msub)) * 64;   // this pair's slots
  auto denominator = [&](auto two_t) {
    constexpr bool TWO = decltype(two_t)::value;
    constexpr int NT = TWO ? 4 : 2;
    if (!ZPRE) load_z();
    // N-tiles 0, 1 of this wave, then (TWO) those of its mirror
    const SwRow rows[4] = {qrow0, qrow1, SwRow(qw, 32 * msub + col), SwRow(qw, 32 * (2 * Cfg::WPH - 1 - msub) + col)};
    float dd[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dd[nt] = 0.f;
    constexpr int D0 = TWO ? 0 : NT0;   // first N-tile computed
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int n = 32 * mt + col;
      const int gn = __shfl(gl, n, 64);   // g(n)
      const _Float16* mrow = s_mg + (hslot * LDIM + gn) * DH + 8 * half;
      f32x16 T[NT];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 bz = *reinterpret_cast<const float4*>(ht + htab::BZ + 32 * mt + 8 * g4 + 4 * half);
#pragma unroll
        for (int nt = D0; nt < NT; ++nt) {
          T[nt][4 * g4 + 0] = bz.x;
          T[nt][4 * g4 + 1] = bz.y;
          T[nt][4 * g4 + 2] = bz.z;
          T[nt][4 * g4 + 3] = bz.w;
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float4 z0 = zv[mt][ks][0], z1 = zv[mt][ks][1];
        const f16x8 m8 = *reinterpret_cast<const f16x8*>(mrow + 16 * ks);
        const float x[8] = {z0.x * (float)m8[0], z0.y * (float)m8[1], z0.z * (float)m8[2], z0.w * (float)m8[3],
                            z1.x * (float)m8[4], z1.y * (float)m8[5], z1.z * (float)m8[6], z1.w * (float)m8[7]};
        const bf16x8 az = pack8(x);
#pragma unroll
        for (int nt = D0; nt < NT; ++nt)
          T[nt] = mfma32(az, *reinterpret_cast<const bf16x8*>(rows[nt].chunk(2 * ks + half)), T[nt]);
      }
#pragma unroll
      for (int nt = D0; nt < NT; ++nt) {
        float d = 0.f;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {   // rows 32 mt + 8 g4 + 4 half + e, e = 0..3
          const uint2 u = *reinterpret_cast<const uint2*>(rows[nt].elem(32 * mt + 8 * g4 + 4 * half));
          d = fmaf(__uint_as_float(u.x << 16), T[nt][4 * g4 + 0], d);
          d = fmaf(__uint_as_float(u.x & 0xffff0000u), T[nt][4 * g4 + 1], d);
          d = fmaf(__uint_as_float(u.y << 16), T[nt][4 * g4 + 2], d);
          d = fmaf(__uint_as_float(u.y & 0xffff0000u), T[nt][4 * g4 + 3], d);
        }
        dd[nt] += d;
      }
    }
    const float az0 = half == 0 ? rec[OAL_COEF_A] * ts_side[tile::SIDE_Z0] : 0.f;
    const float sc = ldexpf(F, e_m);
#pragma unroll
    for (int nt = D0; nt < 2; ++nt) den[nt] += dd[nt] * sc + az0 * F;
    if (TWO) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {   // whole sums (both lane halves) of the mirror's tokens
        float xm = dd[NT - 2 + nt] * sc + az0 * F;
        xm += __shfl_xor(xm, 32, 64);
        if (half == 0) dx[32 * nt + col] = xm;
      }
    }
  };
  if (ZPRE && head_ok && den_giver) denominator(bool_t<PAIRED>{});

  // ================= intra-chunk part ======================================
  // kappa^T[key][tok] F = eps F + sum_p t_p^2,  t_p = sqrt(F) (L_0p + sum_r ell_p[r] q_r k_r),
  // then the causal mask and u~^T += [V; 1]^T kappa^T (values on the matrix cores,
  // the ones channel as column sums into the denominator).  ell_p[r] = L_{g(r),p} /
  // sqrt(d_h) equals c_p = L_{1,p} / sqrt(d_h) on group 1, so with S = q . k
  //   t_p = sqrt(F) (L_0p + c_p S + sum_{g(r) >= 2} (ell_p[r] - c_p) q_r k_r);
  // when at most 14 dims lie outside group 1 (compact), S is one 64-deep product of
  // the raw inputs and each t_p one 16-deep product over the gathered outlier dims
  // plus two constant slots that add L_0p, seeded with c_p S (zero for p >= 2).
  // Otherwise each t_p is a 64-deep product with A = k o ell_p, seeded with L_0p.
  // Key tiles are addressed inside the staged pass (kt - 4 pass).
  {
    const float epsF = rec[OAL_COEF_EPS] * F;
    const int* cidx = reinterpret_cast<const int*>(ht + htab::CIDX) + 8 * half;
    bf16x8 qc[2];                              // compact q (B operand) of the wave's tokens
    if (compact) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = cidx[j];
        const bool one = half && j >= 6;           // the constant slots 14, 15
        qc[0][j] = one ? (__bf16)1.0f : *qrow0.elem(d);
        qc[1][j] = one ? (__bf16)1.0f : *qrow1.elem(d);
      }
    }
    // One unit of the intra-chunk work: two products of a 32-key tile with a
    // 32-token tile, in slots x = 0, 1, that share their operand reads and run as
    // independent chains (so that their latencies overlap).  MODE 1: key tile kt
    // against token tiles 0 and 1; MODE 0: slot 1 only, kt against token tile 1;
    // MODE 2 (compact path only): key tiles kt and kt + 1 against token tile 1.
    // MASKx: slot x's key tile is the diagonal one of its token tile (key row
    // acc_row(i, h) visible iff <= col).
    auto unit = [&](int kt, auto mode_t, auto mask0_t, auto mask1_t) __attribute__((always_inline)) {
      constexpr int MODE = decltype(mode_t)::value;
      constexpr bool MASK[2] = {decltype(mask0_t)::value, decltype(mask1_t)::value};
      constexpr bool USE[2] = {MODE != 0, true};
      constexpr int NT[2] = {MODE == 1 ? 0 : 1, 1};   // token tile of slot x
      constexpr int NK = MODE == 2 ? 2 : 1;            // distinct key tiles
      constexpr int KX[2] = {0, MODE == 2 ? 1 : 0};    // key tile (of the NK) of slot x
      f32x16 kap[2] = {splat16(epsF), splat16(epsF)};
      const SwRow krow[2] = {SwRow(k_arr(kt >> 1), (32 * kt + col) & 63),
                             SwRow(k_arr((kt + NK - 1) >> 1), (32 * (kt + NK - 1) + col) & 63)};
      bf16x8 kr[NK][4];
#pragma unroll
      for (int j = 0; j < NK; ++j)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kr[j][ks] = *reinterpret_cast<const bf16x8*>(krow[j].chunk(2 * ks + half));
      if (compact) {
        f32x16 S[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          if (!USE[x]) continue;
          S[x] = splat16(0.f);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) S[x] = mfma32(kr[KX[x]][ks], qfrag(NT[x], ks), S[x]);
        }
        float kc[NK][8];
#pragma unroll
        for (int j = 0; j < NK; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) kc[j][i] = (half && i >= 6) ? 1.0f : bf(*krow[j].elem(cidx[i]));
        // A operand of t_p for key tile j: the compact key entries times (ell_p - c_p) 2^(E/2)
        auto akc_of = [&](int j, int p) __attribute__((always_inline)) {
          const float* ec = ht + htab::ELLC + p * 16 + 8 * half;
          const float4 e0 = *reinterpret_cast<const float4*>(ec);
          const float4 e1 = *reinterpret_cast<const float4*>(ec + 4);
          const float x[8] = {kc[j][0] * e0.x, kc[j][1] * e0.y, kc[j][2] * e0.z, kc[j][3] * e0.w,
                              kc[j][4] * e1.x, kc[j][5] * e1.y, kc[j][6] * e1.z, kc[j][7] * e1.w};
          return pack8(x);
        };
        // The terms go two at a time, so that up to four independent products are
        // in flight before their squares are summed: p = 0, 1 (seeded with c_p S),
        // then pairs of p >= 2 (c_p = 0 there: L is lower triangular), then a
        // single last term when G + 1 is odd.
        {
          bf16x8 a[NK][2];
#pragma unroll
          for (int j = 0; j < NK; ++j) {
            a[j][0] = akc_of(j, 0);
            a[j][1] = akc_of(j, 1);
          }
          const float c0 = ht[htab::CP + 0], c1 = ht[htab::CP + 1];
          f32x16 t[2][2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (!USE[x]) continue;
            f32x16 s0, s1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              s0[i] = c0 * S[x][i];
              s1[i] = c1 * S[x][i];
            }
            t[x][0] = mfma32(a[KX[x]][0], qc[NT[x]], s0);
            t[x][1] = mfma32(a[KX[x]][1], qc[NT[x]], s1);
          }
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (!USE[x]) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              kap[x][i] = fmaf(t[x][0][i], t[x][0][i], fmaf(t[x][1][i], t[x][1][i], kap[x][i]));
          }
        }
        int p = 2;
        for (; p + 1 <= G; p += 2) {
          bf16x8 a[NK][2];
#pragma unroll
          for (int j = 0; j < NK; ++j) {
            a[j][0] = akc_of(j, p);
            a[j][1] = akc_of(j, p + 1);
          }
          f32x16 t[2][2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (!USE[x]) continue;
            t[x][0] = mfma32(a[KX[x]][0], qc[NT[x]], splat16(0.f));
            t[x][1] = mfma32(a[KX[x]][1], qc[NT[x]], splat16(0.f));
          }
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (!USE[x]) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              kap[x][i] = fmaf(t[x][0][i], t[x][0][i], fmaf(t[x][1][i], t[x][1][i], kap[x][i]));
          }
        }
        if (p <= G) {
          bf16x8 a[NK];
#pragma unroll
          for (int j = 0; j < NK; ++j) a[j] = akc_of(j, p);
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (!USE[x]) continue;
            const f32x16 t = mfma32(a[KX[x]], qc[NT[x]], splat16(0.f));
#pragma unroll
            for (int i = 0; i < 16; ++i) kap[x][i] = fmaf(t[i], t[i], kap[x][i]);
          }
        }
      } else if constexpr (MODE != 2) {
        float kf[4][8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j) kf[ks][j] = bf(kr[0][ks][j]);
        for (int p = 0; p <= G; ++p) {
          const float* ell = ht + htab::ELL + p * DH + 8 * half;
          bf16x8 ak[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const float4 e0 = *reinterpret_cast<const float4*>(ell + 16 * ks);
            const float4 e1 = *reinterpret_cast<const float4*>(ell + 16 * ks + 4);
            const float x[8] = {kf[ks][0] * e0.x, kf[ks][1] * e0.y, kf[ks][2] * e0.z, kf[ks][3] * e0.w,
                                kf[ks][4] * e1.x, kf[ks][5] * e1.y, kf[ks][6] * e1.z, kf[ks][7] * e1.w};
            ak[ks] = pack8(x);
          }
          const float l0 = ht[htab::L0 + p];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (!USE[x]) continue;
            f32x16 sacc = splat16(l0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sacc = mfma32(ak[ks], qfrag(NT[x], ks), sacc);
#pragma unroll
            for (int i = 0; i < 16; ++i) kap[x][i] = fmaf(sacc[i], sacc[i], kap[x][i]);
          }
        }
      }
      // causal mask, denominators, and P [V; 1]
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (!USE[x]) continue;
        const int ktx = kt + KX[x];
        const uint8_t* va = v_arr(ktx >> 1);
        if (MASK[x]) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (acc_row(i, half) > col) kap[x][i] = 0.f;
        }
        float ds = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ds += kap[x][i];
        den[NT[x]] += ds;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float xv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[j] = kap[x][8 * s2 + j];
          const bf16x8 pb = pack8(xv);
          const int kc8 = (4 * (ktx & 1) + 2 * s2 + half);   // 16-byte chunk of the v^T row
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const SwRow vr(va, 32 * mt + col);
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(vr.chunk(kc8));
            acc[mt][NT[x]] = mfma32(av, pb, acc[mt][NT[x]]);
          }
        }
      }
    };
    using M0 = std::integral_constant<int, 0>;
    using M1 = std::integral_constant<int, 1>;
    using M2 = std::integral_constant<int, 2>;
    using F_ = bool_t<false>;
    // key tiles lo .. hi - 1 (staged indices) against token tile 1 alone, the last
    // one masked when ML; two at a time on the compact path
    auto singles = [&](int lo, int hi, auto ml_t) __attribute__((always_inline)) {
      using ML = decltype(ml_t);
      if (lo >= hi) return;
      if (compact) {
        int kt = lo;
        for (; kt + 2 < hi; kt += 2) unit(kt, M2{}, F_{}, F_{});
        if (kt + 2 == hi)
          unit(kt, M2{}, F_{}, ML{});
        else
          unit(kt, M0{}, F_{}, ML{});
      } else {
        for (int kt = lo; kt + 1 < hi; ++kt) unit(kt, M0{}, F_{}, F_{});
        unit(hi - 1, M0{}, F_{}, ML{});
      }
    };
    // The key tiles of a pass against this wave's token tiles: both token tiles for
    // key tiles up to T0 (T0 the diagonal one of N-tile 0), then N-tile 1 alone up
    // to T1 (its diagonal one); in half mode N-tile 1 alone.  Units take staged
    // key tiles j (chunk key tile kt_of(j)).
    auto pass_units = [&](int pass) __attribute__((always_inline)) {
      auto kt_of = [&](int j) { return Cfg::NPASS == 1 ? j : 2 * j + pass; };
      // staged tiles with a chunk key tile <= kt, and the first one >= kt
      auto j_upto = [&](int kt) { return Cfg::NPASS == 1 ? kt + 1 : (kt >= pass ? ((kt - pass) >> 1) + 1 : 0); };
      auto j_from = [&](int kt) { return Cfg::NPASS == 1 ? kt : (kt <= pass ? 0 : (kt - pass + 1) >> 1); };
      int lo = 0;
      if constexpr (!HALF) {
        const int m = j_upto(T0);
        const bool d0 = m > 0 && kt_of(m - 1) == T0;
        for (int j = 0; j + (d0 ? 1 : 0) < m; ++j) unit(j, M1{}, F_{}, F_{});
        if (d0) unit(m - 1, M1{}, bool_t<true>{}, F_{});
        lo = j_from(T0 + 1);
      }
      const int hi = j_upto(T1);
      if (hi > 0 && kt_of(hi - 1) == T1)
        singles(lo, hi, bool_t<true>{});
      else
        singles(lo, hi, F_{});
    };
    if (head_ok) pass_units(0);
    if (Cfg::NPASS > 1) {
      load_kv(1);        // (issued here: in flight during the first pass they would spill)
      __syncthreads();   // every wave is done with the first pass's keys
      stage_kv(1);
      __syncthreads();
      if (head_ok) pass_units(1);
    }
  }

  // ================= inter-chunk part ======================================
  // The main loop uses no LDS buffer; the waves still meet here so that they
  // start it together and their fragment reads of the same tile meet in the
  // caches (without it, 3 % slower at N=32768, measured).  It also orders the
  // mirror waves' denominators (dx) before their reads in the epilogue.
  __syncthreads();
  if (!ZPRE && head_ok) denominator(bool_t<false>{});

  // ---- main K loop over the 37 half-slabs: 1 linear, then 4 c + 3 per t-block c
  //      (the last of them the merged rows of the diagonal block).  Each wave
  //      reads its state fragments straight from the tile (L2: the head groups of
  //      a (unit, chunk) share an XCD) one half-slab ahead into registers, so the
  //      loop has no barrier and the waves of a workgroup run independently.
  const uint8_t* mgh0 = reinterpret_cast<const uint8_t*>(s_mg + hslot * LDIM * DH);
  const uint8_t* mgh = mgh0 + 16 * half;
  f16x8 qt[2], qh[2];   // qh: q_t M of the current group (chunk 64)
  int cur = -1;
  // The state fragments of a half-slab in registers: K-step i, rows 32 mt + col.
  using AFrag = f16x8[4][2];
  auto load_af = [&](AFrag& af, int hs) {
    const uint8_t* g = tsrc + (size_t)min(hs, Cfg::NHS - 1) * Cfg::HS_BYTES + col * 32 + 16 * half;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[i][mt] = *reinterpret_cast<const f16x8*>(g + i * tile::KS_BYTES + mt * 32 * 32);
  };
  // One half-slab of rows r0 .. r0 + 3 of t-block c (K-steps (r0 + i, c)) from the
  // fragments af, while the fragments of half-slab nsb load into nx (when pf).
  // From chunk 128 on the feature build has no branch (every row's M row is read
  // and q_t M formed again), so that the compiler can interleave the next step's
  // multiplies with the current step's products; at chunk 64 (four heads staged,
  // where the extra registers would spill) M rows are read and q_t M formed only
  // where the group changes from the row before.
  constexpr bool BRANCH_FREE = CH >= 128;
  auto quad = [&](int c, int h, const AFrag& af, AFrag& nx, int nsb, bool pf) {
    const int r0 = 4 * h;
    uint2 u[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) u[nt] = *reinterpret_cast<const uint2*>((nt ? qrow1 : qrow0).elem(r0));
    const uint8_t* mgc = mgh + 32 * c;
    int gi[4];
    f16x8 m8[4];   // M_{g(r), g(t)} / d_h (scaled) of the four rows
    int pg = cur;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gi[i] = __builtin_amdgcn_readlane(gl, r0 + i);
      if (BRANCH_FREE || gi[i] != pg) m8[i] = *reinterpret_cast<const f16x8*>(mgc + gi[i] * (DH * 2));
      pg = gi[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (pf) load_af(nx, nsb);
    __builtin_amdgcn_sched_barrier(0);
    const float qs = (r0 < 16 * c || half == 1) ? 2.0f * qr_scale : qr_scale;
    _Float16 qr[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const f16x2 lo = __builtin_convertvector(
          (f32x2){__uint_as_float(u[nt].x << 16) * qs, __uint_as_float(u[nt].x & 0xffff0000u) * qs}, f16x2);
      const f16x2 hi = __builtin_convertvector(
          (f32x2){__uint_as_float(u[nt].y << 16) * qs, __uint_as_float(u[nt].y & 0xffff0000u) * qs}, f16x2);
      qr[nt][0] = lo[0];
      qr[nt][1] = lo[1];
      qr[nt][2] = hi[0];
      qr[nt][3] = hi[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x8 f0, f1;
      if constexpr (BRANCH_FREE) {
        f0 = (qt[0] * m8[i]) * qr[0][i];
        f1 = (qt[1] * m8[i]) * qr[1][i];
      } else {
        if (gi[i] != cur) {   // qhat = q_t M_{g(r), g(t)} / d_h (scaled), recomputed when g(r) changes
          cur = gi[i];
          qh[0] = qt[0] * m8[i];
          qh[1] = qt[1] * m8[i];
        }
        f0 = qh[0] * qr[0][i];
        f1 = qh[1] * qr[1][i];
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc[mt][0] = mfma32h(af[i][mt], f0, acc[mt][0]);
        acc[mt][1] = mfma32h(af[i][mt], f1, acc[mt][1]);
      }
    }
  };
  // the merged half-slab of t-block c: K-step i holds rows 16 c + 8 + 2 i + half
  // against t = 16 c + 8 .. 16 c + 15 in both lane halves (multiplicity 1)
  auto quad_merged = [&](int c, const AFrag& af, AFrag& nx, int nsb, bool pf) {
    bf16x8 qv[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) qv[nt] = *reinterpret_cast<const bf16x8*>((nt ? qrow1 : qrow0).chunk(2 * c + 1));
    const uint8_t* mgc = mgh0 + 32 * c + 16;   // M rows at t = 16 c + 8 .. + 7
    f16x8 m8[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g0 = __builtin_amdgcn_readlane(gl, 16 * c + 8 + 2 * i);
      const int g1 = __builtin_amdgcn_readlane(gl, 16 * c + 9 + 2 * i);
      m8[i] = *reinterpret_cast<const f16x8*>(mgc + (half ? g1 : g0) * (DH * 2));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (pf) load_af(nx, nsb);
    __builtin_amdgcn_sched_barrier(0);
    f16x8 qu[2];          // q_t, t = 16 c + 8 .. + 7, times qt_scale
    _Float16 qr[2][4];    // q_r, r = 16 c + 8 + 2 i + half, times qr_scale
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const f16x2 hv = __builtin_convertvector((f32x2){bf(qv[nt][j]) * qt_scale, bf(qv[nt][j + 1]) * qt_scale}, f16x2);
        qu[nt][j] = hv[0];
        qu[nt][j + 1] = hv[1];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) qr[nt][i] = (_Float16)(bf(half ? qv[nt][2 * i + 1] : qv[nt][2 * i]) * qr_scale);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x8 f0 = (qu[0] * m8[i]) * qr[0][i];
      const f16x8 f1 = (qu[1] * m8[i]) * qr[1][i];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc[mt][0] = mfma32h(af[i][mt], f0, acc[mt][0]);
        acc[mt][1] = mfma32h(af[i][mt], f1, acc[mt][1]);
      }
    }
  };
  auto main_loop = [&]() {
    AFrag afa, afb;
    load_af(afa, 0);
    // linear half-slab 0: phi = b'_r F_f q_r, r = 16 ks + 8 half + j
    {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float4 b0 = *reinterpret_cast<const float4*>(ht + htab::BPF + 16 * ks + 8 * half);
        const float4 b1 = *reinterpret_cast<const float4*>(ht + htab::BPF + 16 * ks + 8 * half + 4);
        const float bq[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        f16x8 fb[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const bf16x8 qv = *reinterpret_cast<const bf16x8*>((nt ? qrow1 : qrow0).chunk(2 * ks + half));
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const f16x2 hv = __builtin_convertvector((f32x2){bq[j] * bf(qv[j]), bq[j + 1] * bf(qv[j + 1])}, f16x2);
            fb[nt][j] = hv[0];
            fb[nt][j + 1] = hv[1];
          }
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          acc[mt][0] = mfma32h(afa[ks][mt], fb[0], acc[mt][0]);
          acc[mt][1] = mfma32h(afa[ks][mt], fb[1], acc[mt][1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_af(afb, 1);
    }
    // t-block c: 4 c + 2 half-slabs of 4 c rows, then the merged one; its first
    // half-slab hs0 has its fragments in X
    auto cblock = [&](int c, int hs0, AFrag& X, AFrag& Y) {
      {
        // q_t of this lane's 8 t's of block c, times qt_scale, as fp16
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const bf16x8 qv = *reinterpret_cast<const bf16x8*>((nt ? qrow1 : qrow0).chunk(2 * c + half));
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const f16x2 hv = __builtin_convertvector((f32x2){bf(qv[j]) * qt_scale, bf(qv[j + 1]) * qt_scale}, f16x2);
            qt[nt][j] = hv[0];
            qt[nt][j + 1] = hv[1];
          }
        }
        cur = -1;
      }
      for (int pr = 0; pr < 2 * c + 1; ++pr) {
        const int hs = hs0 + 2 * pr;
        quad(c, 2 * pr, X, Y, hs + 1, true);
        quad(c, 2 * pr + 1, Y, X, hs + 2, true);
      }
      const int hs = hs0 + 4 * c + 2;
      quad_merged(c, X, Y, hs + 1, hs + 1 < Cfg::NHS);
    };
    cblock(0, 1, afb, afa);
    cblock(1, 4, afa, afb);
    cblock(2, 11, afb, afa);
    cblock(3, 22, afa, afb);
  };
  if (head_ok) main_loop();

  // ================= epilogue: + a F H0, normalise, store ======================
  if (!head_ok) return;
#pragma unroll
  for (int nt = NT0; nt < 2; ++nt) {
    den[nt] += __shfl_xor(den[nt], 32, 64);
    if (!den_giver) den[nt] += dx[32 * nt + col];   // written before the barrier ahead of the main loop
  }
  const float aF = rec[OAL_COEF_A] * F;
  // the lane's column taken afresh: the compiler would otherwise compute the
  // token offsets before the main loop and keep them spilled across it
  int col_e = (int)(threadIdx.x & 31);
  asm volatile("" : "+v"(col_e));
#pragma unroll
  for (int nt = NT0; nt < 2; ++nt) {
    const int tok = 32 * (nt ? T1 : T0) + col_e;
    if (tok >= clen) continue;
    // NG = 0 marks a dimension-specific record, which this grouped readout
    // cannot evaluate: its outputs are made NaN rather than silently wrong
    const float inv = G >= 1 ? 1.0f / den[nt] : __builtin_nanf("");
    O* yr = y + (((size_t)b * n_q_heads + hq) * seq_len + t0 + tok) * DV;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int w0 = 32 * mt + 8 * g4 + 4 * half;
        const float4 hv = *reinterpret_cast<const float4*>(s_h0 + w0);
        const float o[4] = {(acc[mt][nt][4 * g4 + 0] + aF * hv.x) * inv, (acc[mt][nt][4 * g4 + 1] + aF * hv.y) * inv,
                            (acc[mt][nt][4 * g4 + 2] + aF * hv.z) * inv, (acc[mt][nt][4 * g4 + 3] + aF * hv.w) * inv};
        Elem<O>::store4(yr, w0, o);
      }
  }
}

// ---------------------------------------------------------------------------

size_t state_mfma_workspace(int batch, int n_kv_heads, int seq_len, int chunk, bool with_tiles);
oal_status launch_state_mfma(int batch, int n_kv_heads, int seq_len, int chunk, const void* k,
                             const void* v, float* state, bool init_zero, uint8_t* ts, void* ws,
                             hipStream_t stream);

// Workgroup slots of one XCD for the readout: two workgroups per CU, the CUs
// split evenly over the 8 XCDs.
static int readout_slots_per_xcd() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    return 64;
  return 2 * (cus / 8);
}

template <int CH, typename O, bool HALF>
static void readout_grid(int S, int n_q_heads, int n_kv_heads, int seq_len, int n_chunks,
                         int n_hg, int n_uc, const void* q, const void* k, const void* v,
                         const void* coeffs, const uint8_t* ts, void* y, hipStream_t stream) {
  const long long blocks = 8LL * (HALF ? 2 : 1) * S;
  hipLaunchKernelGGL((k_readout_mfma<CH, O, HALF>), dim3((unsigned)blocks), dim3(256), 0, stream, n_q_heads,
                     n_kv_heads, seq_len, n_chunks, n_hg, n_uc,
                     reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
                     reinterpret_cast<const uint16_t*>(v), reinterpret_cast<const float*>(coeffs), ts,
                     reinterpret_cast<O*>(y));
}

// The items (unit x chunk, head group) of each XCD run in rounds of its slots.
// At chunk 256, items that fill at most half of one round run as half
// workgroups (two per item in the same slots, each about 80 % as long as a whole
// one): a short sequence then finishes sooner.  A half round after whole rounds
// stays whole: as a second launch it cost more than it saved (measured).
template <int CH, typename O>
static oal_status readout_launch(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                                 int n_chunks, const void* q, const void* k, const void* v,
                                 const void* coeffs, const uint8_t* ts, void* y,
                                 hipStream_t stream) {
  using Cfg = ReadoutCfg<CH>;
  const int units = batch * n_kv_heads;
  const int rep = n_q_heads / n_kv_heads;
  const int n_hg = (rep + Cfg::HPW - 1) / Cfg::HPW;
  const int n_uc = units * n_chunks;
  const int S = n_hg * ((n_uc + 7) / 8);   // items per XCD
  ProfScope ps("k_readout_mfma", stream);
  bool half = false;
  if constexpr (CH == 256) half = 2 * S <= readout_slots_per_xcd();
  if (half) {
    if constexpr (CH == 256)
      readout_grid<CH, O, true>(S, n_q_heads, n_kv_heads, seq_len, n_chunks, n_hg, n_uc, q, k, v, coeffs,
                                ts, y, stream);
  } else {
    readout_grid<CH, O, false>(S, n_q_heads, n_kv_heads, seq_len, n_chunks, n_hg, n_uc, q, k, v, coeffs,
                               ts, y, stream);
  }
  return check_launch("k_readout_mfma");
}

template <typename O>
static oal_status readout_dispatch(int chunk, int batch, int n_q_heads, int n_kv_heads,
                                   int seq_len, int n_chunks, const void* q, const void* k,
                                   const void* v, const void* coeffs, const uint8_t* ts,
                                   void* y, hipStream_t stream) {
  if (chunk == 64)
    return readout_launch<64, O>(batch, n_q_heads, n_kv_heads, seq_len, n_chunks, q, k, v, coeffs, ts, y, stream);
  if (chunk == 128)
    return readout_launch<128, O>(batch, n_q_heads, n_kv_heads, seq_len, n_chunks, q, k, v, coeffs, ts, y, stream);
  return readout_launch<256, O>(batch, n_q_heads, n_kv_heads, seq_len, n_chunks, q, k, v, coeffs, ts, y, stream);
}

oal_status launch_prefill_mfma(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                               const void* q, const void* k, const void* v, const void* coeffs,
                               int chunk, float* state, bool init_zero, void* y, oal_dtype out_dtype,
                               void* ws, hipStream_t stream) {
  const int units = batch * n_kv_heads;
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  // workspace: the per-chunk prefix tiles (with output), then the builder's scratch
  if (y == nullptr)   // state only: no per-chunk prefixes are needed
    return launch_state_mfma(batch, n_kv_heads, seq_len, chunk, k, v, state, init_zero, nullptr, ws,
                             stream);
  uint8_t* ts = reinterpret_cast<uint8_t*>(ws);
  uint8_t* scratch = ts + (size_t)units * n_chunks * tile::BYTES;
  oal_status st = launch_state_mfma(batch, n_kv_heads, seq_len, chunk, k, v, state, init_zero, ts,
                                    scratch, stream);
  if (st != OAL_OK) return st;
  if (out_dtype == OAL_F32)
    return readout_dispatch<float>(chunk, batch, n_q_heads, n_kv_heads, seq_len, n_chunks, q, k, v,
                                   coeffs, ts, y, stream);
  return readout_dispatch<uint16_t>(chunk, batch, n_q_heads, n_kv_heads, seq_len, n_chunks, q, k, v,
                                    coeffs, ts, y, stream);
}

}  // namespace oal
