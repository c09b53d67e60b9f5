// Backward pass of the causal prefill on the vector ALUs in fp32.
//
// The forward of a sequence that starts from an empty state ([OAL] Algorithm 1,
// Eq. 5-6) is, per query head, u~_i = sum_{j<=i} kappa_ij u_j with u_j = [v_j; 1],
// kappa_ij = phi_q(q_i) . phi_k(k_j) = sum_f c_f psi_f(q_i) psi_f(k_j), the
// monomials psi = (1, x_r, x_r x_t (r <= t)) and the record's expanded
// coefficients c = (a, b'_r, c'_rt), and y_i = u~_i[:64] / u~_i[64].  For a loss
// with gradient dy_i on y_i:
//   g_i = [dy_i / den_i ; -(dy_i . y_i) / den_i]   (gradient on u~_i)
//   alpha_ij = g_i . u_j                            (gradient on kappa_ij)
//   dq_i = sum_{j<=i} alpha_ij grad_q kappa_ij,  grad_q kappa = k o (b' + 2 S p)
//   dk_j = sum_h sum_{i>=j} alpha_ij grad_k kappa_ij,  grad_k kappa = q o (b' + 2 S p)
//   dv_j = sum_h sum_{i>=j} kappa_ij g_i[:64]
//   dc_f = sum_{i, j<=i} alpha_ij psi_f(q_i) psi_f(k_j)
// with p = q o k and S the symmetric C / d_h square of the record; the sums over
// h run over the query heads that share the KV head.  Linear time, chunk by
// chunk like the forward: the part of a row's sums that lies in earlier chunks
// goes through the prefix states H_{<c} (dq_i from H_{<c} g_i), the part in later
// chunks through suffix states R_{>c} = sum_h sum_{i in later chunks}
// phi_q(q_i) g_i^T (dv_j and dk_j from R_{>c}^T psi(k_j) and R_{>c} u_j), and the
// chunk itself is summed pair by pair.
//
// Kernels, in launch order:
//   prefix build + scan (oal_prefill_vec.hip)  H_{<c}
//   k_bwd_ustate    the state part of u~_i: Phi(q) H_{<c} (to the g rows)
//   k_bwd_pair      grouped records at chunk 64, on the matrix cores: the chunk's pair
//                   matrices (group sums, kappa, alpha), g_i, alpha rows and the pair parts
//                   of dq_i, dk_j, dv_j
//   k_bwd_query     the other records: four (chunk 64) or two threads per query: the pair
//                   part of u~_i, g_i; the pair part of dq_i; alpha rows
//   k_bwd_dqstate   the state part of dq_i: H_{<c} g_i against d psi(q_i) / dq_i, by pair rows
//   k_bwd_rbuild    per chunk: sum_h c_f psi_f(q_i) g_i^T (suffix deltas) and the
//                   state part of dc: sum_i psi_f(q_i) (H_{<c} g_i)_f
//   k_bwd_rscan     exclusive suffix sums over chunks: R_{>c}
//   k_bwd_key       the other records: four (chunk 64) or two threads per key and query
//                   head: the pair parts of dv_j, dk_j
//   k_bwd_kstate    the parts through R_{>c}: R^T psi(k_j) and R u_j against d psi(k_j) / dk_j,
//                   by pair rows in four feature splits;  k_bwd_ksum adds the parts
//   k_bwd_dc_intra  pair part of dc: sum_{i, j<=i in the chunk} alpha_ij psi_f(q_i) psi_f(k_j)
//   k_bwd_dcoef     sum over chunks and batch; (da, db, dC) of [OAL] Eq. 3
#include "oal_common.h"

namespace oal {

namespace {
constexpr int WP = 68;                 // rows of H, R, u and g padded to 16 bytes
constexpr int TB = 64;                 // tokens per staged tile
constexpr int FB = 64;                 // feature rows per build block
constexpr int NFB = DS / FB;           // 34
constexpr int WPT = (W + 3) / 4;       // 17 columns per thread in the build
constexpr int WPH = W + 1;             // LDS row of a staged H block: channels 0..64, a zero

// fp32 matrix-core product v_mfma_f32_32x32x2_f32: A 32 x 2 (lane l holds
// A[l % 32][l / 32]), B 2 x 32 (lane l holds B[l / 32][l % 32]), D 32 x 32 (lane l,
// register i holds D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]).
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float fx16;
__device__ __forceinline__ fx16 mfma_f32(float a, float b, fx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int mrow(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// x of the lane whose index differs in bit 0 (bit 1): DPP quad permutations
__device__ __forceinline__ float lane_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// feature f of the canonical order: kind 0 constant, 1 linear x_r, 2 pair x_r x_t,
// 3 padding
__device__ __forceinline__ int feat_decode(int f, int& r, int& t) {
  r = 0;
  t = 0;
  if (f == 0) return 0;
  if (f <= DH) {
    r = f - 1;
    return 1;
  }
  if (f < DCAN) {
    pair_decode(f - 1 - DH, r, t);
    return 2;
  }
  return 3;
}
static_assert(TB * DH % 256 == 0 && TB * WP % 256 == 0, "staging by 256 threads");

// Row blocks of the features with a gradient, 64 feature slots each.  Block b < 32:
// the pair rows r = b (pairs (b, t), t = b .. 63) and r = 63 - b (pairs (63 - b, t),
// t = 63 - b .. 62); block 32: the linear features x_t; block 33: the column
// (t, 63), t = 32 .. 63.  Every pair and linear feature lies in exactly one block
// (the constant has no gradient).  A block's slots form up to two rows, each with a
// multiplier index m and a run of t: slot s < na is (m0, t = ta0 + s), slot
// na <= s < na + nb is (m1, t = tb0 + s - na).  Multiplier DH is the constant slot
// q~[64] = 1 of the linear features.
constexpr int NRB = 34;
struct RowBlk {
  int m0, ta0, na, m1, tb0, nb;
};
__device__ __forceinline__ RowBlk row_block(int blk) {
  if (blk < 32) return RowBlk{blk, blk, DH - blk, DH - 1 - blk, DH - 1 - blk, blk};
  if (blk == 32) return RowBlk{DH, 0, DH, DH, 0, 0};
  return RowBlk{DH - 1, 32, 32, DH, 0, 0};
}
// first pair index of row r of the upper triangle: r (2 DH + 1 - r) / 2
__device__ __forceinline__ int pair_row_start(int r) { return r * (2 * DH + 1 - r) / 2; }
// canonical feature of slot s of block blk (-1: an empty slot)
__device__ __forceinline__ int row_block_feature(int blk, const RowBlk& d, int s) {
  if (s < d.na) {
    const int t = d.ta0 + s;
    if (blk == 32) return 1 + t;
    if (blk == 33) return 1 + DH + pair_row_start(t) + (DH - 1 - t);   // pair (t, 63)
    return 1 + DH + pair_row_start(d.m0) + (t - d.m0);
  }
  if (s < d.na + d.nb) {
    const int t = d.tb0 + s - d.na;
    return 1 + DH + pair_row_start(d.m1) + (t - d.m1);
  }
  return -1;
}

__device__ __forceinline__ float coef_of(const float* rec, int f) {
  if (f == 0) return rec[OAL_COEF_A];
  if (f <= DH) return rec[OAL_COEF_BP + f - 1];
  if (f < DCAN) return rec[OAL_COEF_CP + f - 1 - DH];
  return 0.f;
}

// acc += s * row (16-byte aligned LDS row of WP floats)
__device__ __forceinline__ void axpy_row(float (&acc)[WP], float s, const float* row) {
  float4 r4[WP / 4];
#pragma unroll
  for (int i = 0; i < WP / 4; ++i) r4[i] = reinterpret_cast<const float4*>(row)[i];
#pragma unroll
  for (int i = 0; i < WP / 4; ++i) {
    acc[4 * i + 0] = fmaf(s, r4[i].x, acc[4 * i + 0]);
    acc[4 * i + 1] = fmaf(s, r4[i].y, acc[4 * i + 1]);
    acc[4 * i + 2] = fmaf(s, r4[i].z, acc[4 * i + 2]);
    acc[4 * i + 3] = fmaf(s, r4[i].w, acc[4 * i + 3]);
  }
}

// row . x over WP entries (the pads of x are zero)
__device__ __forceinline__ float dot_row(const float* row, const float (&x)[WP]) {
  float4 r4[WP / 4];
#pragma unroll
  for (int i = 0; i < WP / 4; ++i) r4[i] = reinterpret_cast<const float4*>(row)[i];
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;   // four independent chains
#pragma unroll
  for (int i = 0; i < WP / 4; ++i) {
    s0 = fmaf(r4[i].x, x[4 * i + 0], s0);
    s1 = fmaf(r4[i].y, x[4 * i + 1], s1);
    s2 = fmaf(r4[i].z, x[4 * i + 2], s2);
    s3 = fmaf(r4[i].w, x[4 * i + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// (S p)_r for the 64-float row r of S in LDS (16-byte aligned) and p in registers
__device__ __forceinline__ float srow_dot(const float* srow, const float (&p)[DH]) {
  float4 s4[DH / 4];
#pragma unroll
  for (int i = 0; i < DH / 4; ++i) s4[i] = reinterpret_cast<const float4*>(srow)[i];
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;   // four independent chains
#pragma unroll
  for (int i = 0; i < DH / 4; ++i) {
    s0 = fmaf(s4[i].x, p[4 * i + 0], s0);
    s1 = fmaf(s4[i].y, p[4 * i + 1], s1);
    s2 = fmaf(s4[i].z, p[4 * i + 2], s2);
    s3 = fmaf(s4[i].w, p[4 * i + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// kappa of one pair from a query row and a key row in LDS: a + sum_r p_r (b'_r + (S p)_r)
// (p_r of the rolled r loop is re-read from LDS: a register array indexed by it
// would live in scratch)
__device__ __forceinline__ float kappa_pair(float a, const float* qi, const float* kj,
                                            const float* s_b, const float* s_S) {
  float p[DH];
#pragma unroll
  for (int t = 0; t < DH; ++t) p[t] = qi[t] * kj[t];
  float kap = a;
#pragma unroll 1
  for (int r = 0; r < DH; ++r) kap = fmaf(s_b[r] + srow_dot(s_S + r * DH, p), qi[r] * kj[r], kap);
  return kap;
}

// Grouped records (NG >= 1): the kernel depends on a pair only through the group
// sums s_bar = [1, s_1 .. s_G], s_g = sum_{r in g} q_r k_r / sqrt(d_h) ([OAL]
// Eq. 7): kappa = eps + s_bar^T M s_bar, and the gradient of kappa with respect
// to q_r is k_r w_{g(r)} with w = (2 / sqrt(d_h)) M s_bar (and q_r w_{g(r)} with
// respect to k_r).  With few dims outside group 1 (at most 16, as the readout's
// compact path) a pair costs one masked 64-wide sum, the outlier dims and a 7 x 7
// product instead of the 64 x 64 S p of the general form.
constexpr int MAX_OUT = 16;
struct GroupTab {
  float M[LDIM][LDIM];   // M = L L^T, zero beyond G
  float bulk[DH];        // 1 on the dims of group 1, else 0
  float eps;
  int n_out;             // dims outside group 1
  int dim[MAX_OUT];
  int grp[MAX_OUT];
};

// every thread of the block calls it; a barrier must follow before use
__device__ __forceinline__ void build_group_tab(GroupTab& gt, const float* rec, int tid) {
  const int32_t* gmap = reinterpret_cast<const int32_t*>(rec) + OAL_COEF_GMAP;
  if (tid < LDIM * LDIM) gt.M[tid / LDIM][tid % LDIM] = rec[OAL_COEF_M + tid];
  if (tid < DH) gt.bulk[tid] = gmap[tid] <= 1 ? 1.f : 0.f;
  if (tid == 0) {
    gt.eps = rec[OAL_COEF_EPS];
    int n = 0;
    for (int r = 0; r < DH; ++r) {
      if (gmap[r] <= 1) continue;
      if (n < MAX_OUT) {
        gt.dim[n] = r;
        gt.grp[n] = gmap[r];
      }
      ++n;
    }
    gt.n_out = n;
  }
}

// kappa of one pair (q row and k row in LDS) and w = (2 / sqrt d_h) M s_bar
__device__ __forceinline__ float grouped_pair(const float* qi, const float* kj, const GroupTab& gt,
                                              float (&w)[LDIM]) {
  float s[LDIM];
  float s1 = 0.f;
#pragma unroll
  for (int t = 0; t < DH; ++t) s1 = fmaf(gt.bulk[t], qi[t] * kj[t], s1);
  s[0] = 1.f;
  s[1] = s1 * 0.125f;
#pragma unroll
  for (int g = 2; g < LDIM; ++g) s[g] = 0.f;
  for (int e = 0; e < gt.n_out; ++e) {
    const int d = gt.dim[e], ge = gt.grp[e];
    const float pe = qi[d] * kj[d] * 0.125f;
#pragma unroll
    for (int g = 2; g < LDIM; ++g) s[g] += ge == g ? pe : 0.f;
  }
  float kap = gt.eps;
#pragma unroll
  for (int u = 0; u < LDIM; ++u) {
    float tu = 0.f;
#pragma unroll
    for (int v = 0; v < LDIM; ++v) tu = fmaf(gt.M[u][v], s[v], tu);
    kap = fmaf(s[u], tu, kap);
    w[u] = 0.25f * tu;
  }
  return kap;
}

// x[r] += a y[r] w_{g(r)} for an LDS row x (dq or dk) and a row y (k or q) in LDS
__device__ __forceinline__ void grouped_grad(float* x, float a, const float* y, const GroupTab& gt,
                                             const float (&w)[LDIM]) {
  const float a1 = a * w[1];
#pragma unroll
  for (int r = 0; r < DH; ++r) x[r] = fmaf(a1 * gt.bulk[r], y[r], x[r]);
  for (int e = 0; e < gt.n_out; ++e) {
    const int d = gt.dim[e], ge = gt.grp[e];
    float we = 0.f;
#pragma unroll
    for (int g = 2; g < LDIM; ++g) we = ge == g ? w[g] : we;
    x[d] = fmaf(a * we, y[d], x[d]);
  }
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

// Workspace regions of the backward (each 256-byte aligned).
struct BwdWs {
  float* hc;      // [units][n_chunks][STATE_FLOATS]  H_{<c}
  float* rc;      // [units][n_chunks][STATE_FLOATS]  suffix deltas, then R_{>c}
  float* gbuf;    // [batch][Hq][n_chunks * chunk][WP] g rows (zero beyond seq_len)
  float* alpha;   // [batch][Hq][n_chunks][chunk][chunk] alpha_ij (zero for j > i)
  float* dcp;     // [DC_PARTS][batch][Hq][n_chunks][DS] per-chunk parts of dc
  float* kpart;   // [units][key_split * rep + KS_NFS][n_chunks * chunk][128] parts of [dk | dv]
  size_t bytes;
};

// Threads per key of the key-side kernel (and parts per slot in kpart): four at
// chunk 64 (256 threads, 143 KB of LDS per block), two at chunk 128.
__host__ __device__ constexpr int key_split(int chunk) { return chunk <= 64 ? 4 : 2; }

// Parts of the per-chunk dc: one per wave of k_bwd_rbuild, each its own columns'
// sums over the heads (k_bwd_dc_intra adds the pair part into part 0);
// k_bwd_dcoef adds them.
constexpr int DC_PARTS = 4;
// The suffix-state part of dk and dv walks all 2145 features while the pair part
// meets one chunk of keys; k_bwd_kstate cuts the features into this many ranges,
// one workgroup and one kpart slot each, so that it does not set the length alone.
constexpr int KS_NFS = 4;

static BwdWs bwd_ws(void* base, int batch, int n_q_heads, int n_kv_heads, int seq_len, int chunk) {
  const size_t units = (size_t)batch * n_kv_heads;
  const size_t nc = (size_t)((seq_len + chunk - 1) / chunk);
  const size_t bh = (size_t)batch * n_q_heads;
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t at = off;
    off += al256(floats * sizeof(float));
    return at;
  };
  const size_t o_h = take(units * nc * STATE_FLOATS);
  const size_t o_r = take(units * nc * STATE_FLOATS);
  const size_t o_g = take(bh * nc * chunk * WP);
  const size_t o_a = take(bh * nc * chunk * chunk);
  const size_t o_d = take(DC_PARTS * bh * nc * DS);
  const size_t o_k = take(units * ((size_t)key_split(chunk) * (n_q_heads / n_kv_heads) + KS_NFS) * nc * chunk *
                          (DH + DV));
  BwdWs w;
  uint8_t* p = reinterpret_cast<uint8_t*>(base);
  w.hc = reinterpret_cast<float*>(p + o_h);
  w.rc = reinterpret_cast<float*>(p + o_r);
  w.gbuf = reinterpret_cast<float*>(p + o_g);
  w.alpha = reinterpret_cast<float*>(p + o_a);
  w.dcp = reinterpret_cast<float*>(p + o_d);
  w.kpart = reinterpret_cast<float*>(p + o_k);
  w.bytes = off;
  return w;
}

size_t backward_workspace(int batch, int n_q_heads, int n_kv_heads, int seq_len, int chunk) {
  return bwd_ws(nullptr, batch, n_q_heads, n_kv_heads, seq_len, chunk).bytes;
}

// ---------------------------------------------------------------------------
// State part of u~ for the query kernel:  U[tok][w] = sum_f c_f psi_f(q_tok)
// H_{<c}[f][w], w <= 64, written to the token's g row of the workspace (the query
// kernel reads the row there before it writes g over it).  Block (32 tokens of a
// chunk, chunk, query head), two waves: wave = tile of 32 channels, channel 64 (the
// denominator's) on the VALU of every lane.  K = the features in 34 blocks of 64,
// product j of a block pairing feature f0 + j (lanes 0-31) with f0 + 32 + j (lanes
// 32-63), so that a lane's B operands H[f][w] over the block are 32 consecutive
// features of its channel: eight 16-byte loads, issued two blocks ahead in two
// register sets.  A = c_f psi_f(q_tok) formed per lane from the q rows and the
// feature table (psi_f = q~[ia] q~[ib], q~ = (q, 1)); features past DCAN (state
// padding, never written) are dropped.  The blocks of one (unit, chunk) share an XCD.
constexpr int US_TG = 32;   // tokens per block
template <typename T>
__global__ void __launch_bounds__(128)
k_bwd_ustate(int n_q_heads, int n_kv_heads, int seq_len, int chunk, int n_chunks, int n_units,
             const T* __restrict__ q, const void* __restrict__ coeffs,
             const float* __restrict__ hc, float* __restrict__ gbuf) {
  constexpr int TG = US_TG;
  constexpr int QS = DH + 1;             // q~ row: q, 1
  constexpr int NB = DS / 64;            // feature blocks
  static_assert(NB % 2 == 0 && DS % 64 == 0, "feature blocks taken in pairs");
  const int rep = n_q_heads / n_kv_heads;
  const int per = rep * (chunk / TG);    // blocks of one (unit, chunk)
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int uc = (slot / per) * 8 + xcd;
  if (uc >= n_units * n_chunks) return;
  const int unit = uc / n_chunks, c = uc % n_chunks;
  const int b = unit / n_kv_heads;
  const int hq = (unit % n_kv_heads) * rep + (slot % per) % rep;
  const int t0 = c * chunk + ((slot % per) / rep) * TG;
  const int ntok = min(TG, seq_len - t0);
  if (ntok <= 0) return;                 // a group past the sequence (whole block)
  const int tid = threadIdx.x, lane = tid & 63;
  const int CT = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave's channel tile
  const int tok = lane & 31, h = lane >> 5;

  __shared__ float s_q[TG * QS];
  __shared__ uint16_t s_fd[DS];          // ia | ib << 8
  __shared__ float s_fc[DS];             // c_f, zero past DCAN
  const float* rec = coef_rec(coeffs, hq);
  const float* Hc = hc + ((size_t)unit * n_chunks + c) * STATE_FLOATS;
  const size_t row0 = ((size_t)b * n_q_heads + hq) * seq_len + t0;
  stage_span<TG * DH, 128>(tid, ntok * DH, [&](int i) { return Elem<T>::load(q + row0 * DH, i); },
                           [&](int i, float x) { s_q[(i / DH) * QS + i % DH] = x; });
  if (tid < TG) s_q[tid * QS + DH] = 1.f;
  for (int f = tid; f < DS; f += 128) {
    int r, t;
    const int kind = feat_decode(f, r, t);
    s_fd[f] = (uint16_t)((kind == 0 ? DH : r) | ((kind == 2 ? t : DH) << 8));
  }
  stage_span<DS, 128>(tid, DCAN, [&](int f) { return rec[coef_index(f)]; },
                      [&](int f, float x) { s_fc[f] = x; });

  // B operands H[f0 + 32 h + j][w] of the lane's channel w, and the same features
  // of the denominator's channel (j = 4 m + e); the block offset f0 is a multiple
  // of 64 and a state row is 16-byte aligned, so the loads are aligned
  struct Ops {
    float4 hb[8], hd[8];
  };
  const float* hbp = Hc + (size_t)(32 * CT + tok) * DS + 32 * h;
  const float* hdp = Hc + (size_t)DV * DS + 32 * h;
  auto fetch = [&](int blk, Ops& o) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      o.hb[m] = *reinterpret_cast<const float4*>(hbp + 64 * blk + 4 * m);
      o.hd[m] = *reinterpret_cast<const float4*>(hdp + 64 * blk + 4 * m);
    }
  };
  fx16 D[2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < 16; ++i) D[x][i] = 0.f;
  float dacc = 0.f;
  const float* qrow = s_q + tok * QS;
  auto run = [&](int blk, Ops& o) __attribute__((always_inline)) {
    const int fb = 64 * blk + 32 * h;     // the lane's first feature of the block
    const bool tail = 64 * blk + 64 > DCAN;   // uniform: the block reaching into the padding
#pragma unroll
    for (int j0 = 0; j0 < 32; j0 += 8) {
      float av[8], bv[8], dv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int d = s_fd[fb + j];
        av[jj] = s_fc[fb + j] * qrow[d & 255] * qrow[d >> 8];
        const float4 x = o.hb[j >> 2], y = o.hd[j >> 2];
        bv[jj] = (j & 3) == 0 ? x.x : (j & 3) == 1 ? x.y : (j & 3) == 2 ? x.z : x.w;
        dv[jj] = (j & 3) == 0 ? y.x : (j & 3) == 1 ? y.y : (j & 3) == 2 ? y.z : y.w;
        if (tail && fb + j >= DCAN) {   // padding rows of the state: any bits
          bv[jj] = 0.f;
          dv[jj] = 0.f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        D[jj & 1] = mfma_f32(av[jj], bv[jj], D[jj & 1]);
        dacc = fmaf(av[jj], dv[jj], dacc);
      }
    }
    fetch(min(blk + 2, NB - 1), o);   // unconditional: the last blocks reload one
  };
  Ops oa, ob;
  fetch(0, oa);
  fetch(1, ob);
  __syncthreads();   // the q rows and the feature table are in LDS
  for (int blk = 0; blk < NB; blk += 2) {
    run(blk, oa);
    run(blk + 1, ob);
  }
  // out: D rows are tokens mrow(i, h), columns the channels; the two lane halves'
  // denominator sums added
  dacc += __shfl_xor(dacc, 32, 64);
  float* gr = gbuf + (((size_t)b * n_q_heads + hq) * ((size_t)n_chunks * chunk) + t0) * WP;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = mrow(i, h);
    if (r < ntok) gr[(size_t)r * WP + 32 * CT + tok] = D[0][i] + D[1][i];
  }
  if (CT == 0 && h == 0 && tok < ntok) gr[(size_t)tok * WP + DV] = dacc;
}

// ---------------------------------------------------------------------------
// Query side.  One block per (chunk, query head, batch); SP threads per query
// (thread SP i + h, h = 0 .. SP - 1, for query t0 + i; SP = 4 at chunk 64, 2 at
// chunk 128) split its features and its pairs round robin; the parts of u~_i are
// added through LDS, g_i is shared the same way, and each part keeps its own dq
// row, the rows added in a fixed order at the end.
template <typename T, int SP>
__global__ void __launch_bounds__(256)
k_bwd_query(int n_q_heads, int n_kv_heads, int seq_len, int chunk, int n_chunks, int n_units,
            const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
            const void* __restrict__ coeffs, const float* __restrict__ dy,
            float* __restrict__ gbuf, float* __restrict__ alpha, float* __restrict__ dq) {
  // the query heads of one (unit, chunk) in consecutive slots of one XCD
  // (workgroup id % 8), so that they read that chunk's prefix state through one L2
  const int rep = n_q_heads / n_kv_heads;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int uc = (slot / rep) * 8 + xcd;
  if (uc >= n_units * n_chunks) return;
  const int unit = uc / n_chunks, c = uc % n_chunks;
  const int b = unit / n_kv_heads;
  const int hq = (unit % n_kv_heads) * rep + slot % rep;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;                // SP * chunk
  const int qx = tid / SP;                    // query of the chunk
  const int half = tid % SP;                  // this thread's part
  const int t0 = c * chunk;
  const int clen = min(chunk, seq_len - t0);
  const bool active = qx < clen;

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* s_q = smem;                          // [chunk][DH + 1]
  float* s_dq = s_q + chunk * (DH + 1);       // [SP][chunk][DH + 1] (parts >= 1 also pass u~, g)
  float* s_k = s_dq + SP * chunk * (DH + 1);  // [TB][DH + 1]
  float* s_u = s_k + TB * (DH + 1);           // [TB][WP]
  float* s_b = s_u + TB * WP;                 // [DH]  b'
  float* s_S = s_b + DH;                      // [DH][DH]  C / d_h (symmetric)

  const float* rec = coef_rec(coeffs, hq);
  const float a = rec[OAL_COEF_A];
  __shared__ __attribute__((aligned(16))) GroupTab gt;
  const bool grouped = reinterpret_cast<const int32_t*>(rec)[OAL_COEF_NG] >= 1;
  if (SP == 4 && grouped) return;   // chunk 64: k_bwd_pair on the matrix cores
  if (grouped) build_group_tab(gt, rec, tid);
  const size_t qrow0 = ((size_t)b * n_q_heads + hq) * seq_len + t0;
  {
    const T* qs = q + qrow0 * DH;   // the chunk's q rows, one span (clen >= 1)
    stage_span<(256 / SP) * DH>(tid, clen * DH, [&](int i) { return Elem<T>::load(qs, i); },
                                [&](int i, float x) { s_q[(i / DH) * (DH + 1) + i % DH] = x; });
  }
  for (int i = tid; i < chunk; i += nthr) s_q[i * (DH + 1) + DH] = 1.f;   // psi's constant slot
  for (int i = tid; i < SP * chunk * (DH + 1); i += nthr) s_dq[i] = 0.f;
  for (int i = tid; i < DH; i += nthr) s_b[i] = rec[OAL_COEF_BP + i];
  stage_span<DH * DH>(tid, DH * DH, [&](int i) { return rec[OAL_COEF_CM + i]; },
                      [&](int i, float x) { s_S[i] = x; });
  for (int i = tid; i < TB * (WP - W); i += nthr) s_u[(i / (WP - W)) * WP + W + i % (WP - W)] = 0.f;
  __syncthreads();
  const bool fast = grouped && gt.n_out <= MAX_OUT;   // uniform over the block
  const float* qi = s_q + qx * (DH + 1);
  float* dqi = s_dq + (half * chunk + qx) * (DH + 1);
  const size_t kbase = (size_t)unit * seq_len + t0;

  auto stage_keys = [&](int j0, int nj) {
    if (nj > 0) {   // uniform; the key and value rows are one span each
      const T* ks = k + (kbase + j0) * DH;
      const T* vs = v + (kbase + j0) * DV;
      stage_span<TB * DH>(tid, nj * DH, [&](int i) { return Elem<T>::load(ks, i); },
                          [&](int i, float x) { s_k[(i / DH) * (DH + 1) + i % DH] = x; });
      stage_span<TB * DV>(tid, nj * DV, [&](int i) { return Elem<T>::load(vs, i); },
                          [&](int i, float x) { s_u[(i / DV) * WP + i % DV] = x; });
    } else {
      for (int i = tid; i < TB * DH; i += nthr) {
        s_k[(i / DH) * (DH + 1) + i % DH] = 0.f;
        s_u[(i / DV) * WP + i % DV] = 0.f;
      }
    }
    for (int jj = tid; jj < TB; jj += nthr) s_u[jj * WP + DV] = jj < nj ? 1.f : 0.f;
  };

  // ---- 1. u~_i: the state part U was written to this query's g row by
  // k_bwd_ustate; here the chunk's pairs, on the vector ALUs: this part's share
  float acc[WP];
#pragma unroll
  for (int w = 0; w < WP; ++w) acc[w] = 0.f;
  for (int j0 = 0; j0 < clen; j0 += TB) {
    const int nj = min(TB, clen - j0);
    __syncthreads();
    stage_keys(j0, nj);
    __syncthreads();
    if (active) {
      const int jmax = min(nj, qx - j0 + 1);
      for (int jj = half; jj < jmax; jj += SP) {
        float w[LDIM];
        const float kap = fast ? grouped_pair(qi, s_k + jj * (DH + 1), gt, w)
                               : kappa_pair(a, qi, s_k + jj * (DH + 1), s_b, s_S);
        axpy_row(acc, kap, s_u + jj * WP);
      }
    }
  }

  // ---- 2. u~_i = the parts' sum; g_i (zero for rows beyond the sequence), shared
  // through the dq rows of parts 1 .. SP - 1, still unused
  float* xrow = s_dq + (half * chunk + qx) * (DH + 1);   // this part's dq row
  __syncthreads();
  if (half >= 1) {
#pragma unroll
    for (int w = 0; w < W; ++w) xrow[w] = acc[w];
  }
  __syncthreads();
  float g[WP];
#pragma unroll
  for (int w = 0; w < WP; ++w) g[w] = 0.f;
  if (half == 0) {
#pragma unroll
    for (int h = 1; h < SP; ++h) {   // the parts in a fixed order
      const float* pr = s_dq + (h * chunk + qx) * (DH + 1);
#pragma unroll
      for (int w = 0; w < W; ++w) acc[w] += pr[w];
    }
    // + the state part, read from the g row before g overwrites it
    const float* ur = gbuf + (((size_t)b * n_q_heads + hq) * ((size_t)n_chunks * chunk) + t0 + qx) * WP;
#pragma unroll
    for (int w = 0; w < W; ++w) acc[w] += ur[w];
    if (active) {
      const float inv = 1.0f / acc[DV];
      const float* dyi = dy + (qrow0 + qx) * DV;
      float ydot = 0.f;
#pragma unroll
      for (int w = 0; w < DV; ++w) {
        const float d = dyi[w];
        g[w] = d * inv;
        ydot = fmaf(d, acc[w] * inv, ydot);
      }
      g[DV] = -ydot * inv;
    }
#pragma unroll
    for (int h = 1; h < SP; ++h) {   // g into every other part's own row
      float* pr = s_dq + (h * chunk + qx) * (DH + 1);
#pragma unroll
      for (int w = 0; w < W; ++w) pr[w] = g[w];
    }
    float* gr = gbuf + (((size_t)b * n_q_heads + hq) * ((size_t)n_chunks * chunk) + t0 + qx) * WP;
#pragma unroll
    for (int i = 0; i < WP / 4; ++i)
      reinterpret_cast<float4*>(gr)[i] = make_float4(g[4 * i], g[4 * i + 1], g[4 * i + 2], g[4 * i + 3]);
  }
  __syncthreads();
  if (half >= 1) {
#pragma unroll
    for (int w = 0; w < W; ++w) g[w] = xrow[w];
#pragma unroll
    for (int w = 0; w <= DH; ++w) xrow[w] = 0.f;   // back to a zero dq row (own row only)
  }

  // ---- 3. the chunk's pairs: alpha_ij and dq_i += alpha_ij k_j o (b' + 2 S p)
  float* arow = alpha + ((((size_t)b * n_q_heads + hq) * n_chunks + c) * chunk + qx) * chunk;
  for (int j0 = 0; j0 < chunk; j0 += TB) {
    const int nj = max(0, min(TB, clen - j0));
    __syncthreads();
    stage_keys(j0, nj);
    __syncthreads();
    const int jmax = active ? max(0, min(nj, qx - j0 + 1)) : 0;
    for (int jj = half; jj < jmax; jj += SP) {
      const float* kj = s_k + jj * (DH + 1);
      const float al = dot_row(s_u + jj * WP, g);
      arow[j0 + jj] = al;
      if (fast) {
        float w[LDIM];
        grouped_pair(qi, kj, gt, w);
        grouped_grad(dqi, al, kj, gt, w);
        continue;
      }
      float p[DH];
#pragma unroll
      for (int t = 0; t < DH; ++t) p[t] = qi[t] * kj[t];
#pragma unroll 1
      for (int r = 0; r < DH; ++r)
        dqi[r] = fmaf(al * kj[r], s_b[r] + 2.f * srow_dot(s_S + r * DH, p), dqi[r]);
    }
    for (int jj = half; jj < TB; jj += SP)
      if (jj >= jmax) arow[j0 + jj] = 0.f;
  }

  __syncthreads();
  if (active) {   // each part writes DH / SP entries, the parts' rows added in order
    float* o = dq + (qrow0 + qx) * DH + half * (DH / SP);
#pragma unroll
    for (int d = 0; d < DH / SP; ++d) {
      float x = 0.f;
#pragma unroll
      for (int h = 0; h < SP; ++h) x += s_dq[(h * chunk + qx) * (DH + 1) + half * (DH / SP) + d];
      o[d] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Pair part of the backward on the fp32 matrix cores, for grouped records at chunk
// 64 (one block per (chunk, query head, batch), four waves).  In a grouped record a
// pair enters only through its group sums s_bar = [1, s_1 .. s_G] ([OAL] Eq. 7), so
// with the chunk's pair matrices (rows i = queries, columns j = keys, zero for
// j > i and past the sequence):
//   S_g = (Q o 1_g) K^T / sqrt(d_h)            group sums, one product chain per group
//   kappa = eps + s_bar^T M s_bar              per entry, on the vector ALUs
//   u~ (pair part) = kappa [V 1],  then g from u~ + the state part and dy
//   alpha = G [V 1]^T,  dv = kappa^T G
//   dq = sum_v (alpha o s_v) (K o m_v),  dk = sum_v (alpha o s_v)^T (Q o m_v)
// with s_0 = 1 and m_v[r] = M_{g(r), v} / 4: the gradient of kappa with respect to
// q_r is k_r w_{g(r)}, w = (2 / sqrt(d_h)) M s_bar, and the sum over v folds the
// group weights into the B operand so that one accumulator takes all G + 1 terms.
// Wave w holds the 32 x 32 quadrant (I, J) = (w / 2, w % 2) of the pair matrices
// and the tiles (I, J) of u~ and dq and (J' = I, J) of dk and dv (32 rows x 32
// columns); quadrant (0, 1) lies above the diagonal.  The group sums run over the
// dimensions in group order (a copy of Q and K with permuted columns), each K-step
// of two dimensions masked to the group whose chain it feeds.  The kernel writes the
// g rows over the state part of u~ that k_bwd_ustate left there, the alpha rows, the
// pair part of dq and this head's part of [dk | dv] (part `slot` of kpart, the
// first of the head's key_split(64) parts); k_bwd_query and k_bwd_key leave grouped
// records at chunk 64 to it, and k_bwd_ksum reads one part instead of four for such
// a head.
constexpr int PR_C = 64;     // chunk of the matrix-core pair kernel
constexpr int PR_RS = 65;    // LDS row stride of its 64-row matrices (odd: column reads spread)

// acc += A B over the 16 K-steps k0, k0 + 2, ..., k0 + 30: a(k), b(k) give this lane's
// operands at K index k + (lane / 32); all 32 loads are issued before the products.
template <typename FA, typename FB>
__device__ __forceinline__ fx16 mm16(fx16 acc, int k0, FA a, FB b) {
  float av[16], bv[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    av[s] = a(k0 + 2 * s);
    bv[s] = b(k0 + 2 * s);
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) acc = mfma_f32(av[s], bv[s], acc);
  return acc;
}

template <typename T>
__global__ void __launch_bounds__(256)
k_bwd_pair(int n_q_heads, int n_kv_heads, int seq_len, int n_chunks, int n_units, int n_parts,
           const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
           const void* __restrict__ coeffs, const float* __restrict__ dy, float* __restrict__ gbuf,
           float* __restrict__ alpha, float* __restrict__ dq, float* __restrict__ kpart) {
  constexpr int C = PR_C, RS = PR_RS, MS = C * RS;
  const int rep = n_q_heads / n_kv_heads;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int uc = (slot / rep) * 8 + xcd;
  if (uc >= n_units * n_chunks) return;
  const int unit = uc / n_chunks, c = uc % n_chunks;
  const int b = unit / n_kv_heads;
  const int hh = slot % rep;
  const int hq = (unit % n_kv_heads) * rep + hh;
  const float* rec = coef_rec(coeffs, hq);
  const int32_t* rec_i = reinterpret_cast<const int32_t*>(rec);
  const int G = min(rec_i[OAL_COEF_NG], GMAX);
  if (G < 1) return;   // dimension-specific record: k_bwd_query and k_bwd_key
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, hf = lane >> 5;
  const int I = wv >> 1, J = wv & 1;
  const bool live = !(I == 0 && J == 1);
  const int t0 = c * C;
  const int clen = min(C, seq_len - t0);
  const size_t bh = (size_t)b * n_q_heads + hq;
  const size_t qrow0 = bh * seq_len + t0;
  const size_t npad = (size_t)n_chunks * C;

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* sQ = smem;         // [C][RS] q rows, zero past the sequence
  float* sK = sQ + MS;      // [C][RS] k rows
  float* sU = sK + MS;      // [C][RS] u = (v, 1) rows, zero past the sequence
  float* sG = sU + MS;      // [C][RS] g rows
  float* sP = sG + MS;      // [C][RS] kappa (masked)
  float* sX = sP + MS;      // [2][C][RS] alpha o s_v; first the permuted q and k, then u~
  __shared__ int s_grp[DH];          // group of each dimension (1 .. G)
  __shared__ int s_pos[DH];          // its place in group order
  __shared__ int s_gofs[LDIM + 1];   // group g's places: s_gofs[g] .. s_gofs[g + 1] - 1
  __shared__ float s_M[LDIM * LDIM];

  if (tid < DH) {
    const int gr = rec_i[OAL_COEF_GMAP + tid];
    s_grp[tid] = gr < 1 ? 1 : (gr > G ? G : gr);
  }
  if (tid < LDIM * LDIM) s_M[tid] = rec[OAL_COEF_M + tid];
  __syncthreads();
  if (tid < DH) {
    const int gr = s_grp[tid];
    int pos = 0;
    for (int r = 0; r < DH; ++r) {
      const int g2 = s_grp[r];
      pos += (g2 < gr || (g2 == gr && r < tid)) ? 1 : 0;
    }
    s_pos[tid] = pos;
  } else if (tid < DH + LDIM + 1) {
    const int g = tid - DH;
    int n = 0;
    for (int r = 0; r < DH; ++r) n += s_grp[r] < g ? 1 : 0;
    s_gofs[g] = n;
  }
  __syncthreads();
  {
    const T* qs = q + qrow0 * DH;
    const T* ks = k + ((size_t)unit * seq_len + t0) * DH;
    const T* vs = v + ((size_t)unit * seq_len + t0) * DV;
    float* sQp = sX;
    float* sKp = sX + MS;
    stage_span<C * DH>(tid, clen * DH, [&](int i) { return Elem<T>::load(qs, i); }, [&](int i, float x) {
      sQ[(i / DH) * RS + i % DH] = x;
      sQp[(i / DH) * RS + s_pos[i % DH]] = x;
    });
    stage_span<C * DH>(tid, clen * DH, [&](int i) { return Elem<T>::load(ks, i); }, [&](int i, float x) {
      sK[(i / DH) * RS + i % DH] = x;
      sKp[(i / DH) * RS + s_pos[i % DH]] = x;
    });
    stage_span<C * DV>(tid, clen * DV, [&](int i) { return Elem<T>::load(vs, i); },
                       [&](int i, float x) { sU[(i / DV) * RS + i % DV] = x; });
    if (tid < C) sU[tid * RS + DV] = tid < clen ? 1.f : 0.f;
  }
  __syncthreads();

  // ---- group sums of this wave's quadrant: sacc[g - 1] = sum_{r in g} q_ir k_jr
  fx16 sacc[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[g][i] = 0.f;
  if (live) {
    const float* qa = sX + (32 * I + col) * RS;        // permuted q row i = 32 I + col
    const float* kb = sX + MS + (32 * J + col) * RS;   // permuted k row j = 32 J + col
#pragma unroll
    for (int g = 1; g <= GMAX; ++g) {
      if (g > G) break;
      const int o0 = __builtin_amdgcn_readfirstlane(s_gofs[g]);
      const int o1 = __builtin_amdgcn_readfirstlane(s_gofs[g + 1]);
      for (int p = o0 & ~1; p < o1; p += 8) {   // four K-steps per round, masked to [o0, o1)
        float av[4], bv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int pos = p + 2 * s + hf;
          const int pc = min(pos, DH - 1);
          av[s] = (pos >= o0 && pos < o1) ? qa[pc] : 0.f;
          bv[s] = kb[pc];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[g - 1] = mfma_f32(av[s], bv[s], sacc[g - 1]);
      }
    }
  }

  // ---- kappa of the quadrant's pairs (zero above the diagonal and past the sequence)
  const float eps = rec[OAL_COEF_EPS];
  float Mr[LDIM][LDIM];
#pragma unroll
  for (int u = 0; u < LDIM; ++u)
#pragma unroll
    for (int w = 0; w < LDIM; ++w) Mr[u][w] = rec[OAL_COEF_M + u * LDIM + w];
  fx16 kap;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ri = 32 * I + mrow(i, hf), cj = 32 * J + col;
    float s[LDIM];
    s[0] = 1.f;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) s[g + 1] = sacc[g][i] * 0.125f;
    float x = eps;
#pragma unroll
    for (int u = 0; u < LDIM; ++u) {
      float tu = 0.f;
#pragma unroll
      for (int w = 0; w < LDIM; ++w) tu = fmaf(Mr[u][w], s[w], tu);
      x = fmaf(s[u], tu, x);
    }
    kap[i] = (live && cj <= ri && ri < clen) ? x : 0.f;
    sP[ri * RS + cj] = kap[i];
  }
  __syncthreads();   // sP complete; the permuted copies in sX are no longer read

  // ---- pair part of u~ (tile (I, J) of kappa [V]) to sX, staged for the rows
  {
    fx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const float* pa = sP + (32 * I + col) * RS + hf;   // A[i][j] = kappa_ij
    const float* ub = sU + hf * RS + 32 * J + col;     // B[j][w] = u_jw
    auto fa = [&](int kk) { return pa[kk]; };
    auto fb = [&](int kk) { return ub[kk * RS]; };
    acc = mm16(acc, 0, fa, fb);
    if (I == 1) acc = mm16(acc, 32, fa, fb);
#pragma unroll
    for (int i = 0; i < 16; ++i) sX[(32 * I + mrow(i, hf)) * RS + 32 * J + col] = acc[i];
  }
  __syncthreads();

  // ---- g rows: four threads per query, 16 channels each
  {
    const int ri = tid >> 2, pp = tid & 3;
    const bool active = ri < clen;
    float* gr = gbuf + (bh * npad + t0 + ri) * WP;
    float u[16], dyv[16];
    float dsum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int w = 16 * pp + e;
      u[e] = sX[ri * RS + w] + gr[w];   // + the state part (k_bwd_ustate)
      dsum += sP[ri * RS + w];          // pair part of the denominator: sum_j kappa_ij
      dyv[e] = dy[(qrow0 + min(ri, clen - 1)) * DV + w];
    }
    const float den_state = gr[DV];
    dsum += lane_xor1(dsum);
    dsum += lane_xor2(dsum);
    const float inv = active ? 1.0f / (dsum + den_state) : 0.f;
    float yd = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) yd = fmaf(dyv[e], u[e] * inv, yd);
    yd += lane_xor1(yd);
    yd += lane_xor2(yd);
    float g[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      g[e] = dyv[e] * inv;
      sG[ri * RS + 16 * pp + e] = g[e];
    }
    const float g64 = -yd * inv;
    if (pp == 0) sG[ri * RS + DV] = g64;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      reinterpret_cast<float4*>(gr + 16 * pp)[e] = make_float4(g[4 * e], g[4 * e + 1], g[4 * e + 2], g[4 * e + 3]);
    if (pp == 0) *reinterpret_cast<float4*>(gr + DV) = make_float4(g64, 0.f, 0.f, 0.f);
  }
  __syncthreads();

  // ---- alpha of the quadrant: G [V 1]^T, masked; to the alpha rows
  fx16 al;
  {
#pragma unroll
    for (int i = 0; i < 16; ++i) al[i] = 0.f;
    if (live) {
      const float* ga = sG + (32 * I + col) * RS + hf;   // A[i][w] = g_iw
      const float* vb = sU + (32 * J + col) * RS + hf;   // B[w][j] = u_jw
      auto fa = [&](int kk) { return ga[kk]; };
      auto fb = [&](int kk) { return vb[kk]; };
      al = mm16(al, 0, fa, fb);
      al = mm16(al, 32, fa, fb);
    }
    float* arow = alpha + ((bh * n_chunks + c) * C) * C;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ri = 32 * I + mrow(i, hf), cj = 32 * J + col;
      al[i] = (live && cj <= ri && ri < clen) ? al[i] + sG[ri * RS + DV] : 0.f;
      arow[(size_t)ri * C + cj] = al[i];
    }
  }

  // ---- dv tile (J' = I, J): kappa^T G
  fx16 dva;
  {
#pragma unroll
    for (int i = 0; i < 16; ++i) dva[i] = 0.f;
    const float* pa = sP + hf * RS + 32 * I + col;   // A[j][i] = kappa_ij
    const float* gb = sG + hf * RS + 32 * J + col;   // B[i][w] = g_iw
    auto fa = [&](int kk) { return pa[kk * RS]; };
    auto fb = [&](int kk) { return gb[kk * RS]; };
    if (I == 0) dva = mm16(dva, 0, fa, fb);   // i >= j: rows from 32 I
    dva = mm16(dva, 32, fa, fb);
  }

  // ---- dq tile (I, J) and dk tile (J' = I, J): sum over v of (alpha o s_v) times
  // (K o m_v) and (Q o m_v)
  fx16 dqa, dka;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    dqa[i] = 0.f;
    dka[i] = 0.f;
  }
  float mv[LDIM];   // m_v of this lane's output column r = 32 J + col
  {
    const int gr = s_grp[32 * J + col];
#pragma unroll
    for (int vv = 0; vv < LDIM; ++vv) mv[vv] = 0.25f * s_M[gr * LDIM + vv];
  }
#pragma unroll
  for (int vv = 0; vv < LDIM; ++vv) {
    if (vv > G) break;
    float* X = sX + (vv & 1) * MS;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float s = vv == 0 ? 1.f : sacc[vv > 0 ? vv - 1 : 0][i] * 0.125f;
      X[(32 * I + mrow(i, hf)) * RS + 32 * J + col] = al[i] * s;
    }
    __syncthreads();   // X_v complete; X_{v-2}'s products (same buffer) came before the last barrier
    const float m = mv[vv];
    {
      const float* xa = X + (32 * I + col) * RS + hf;   // A[i][j] = X_ij
      const float* kb = sK + hf * RS + 32 * J + col;    // B[j][r] = k_jr m_v[r]
      auto fa = [&](int kk) { return xa[kk]; };
      auto fb = [&](int kk) { return kb[kk * RS] * m; };
      dqa = mm16(dqa, 0, fa, fb);
      if (I == 1) dqa = mm16(dqa, 32, fa, fb);
    }
    {
      const float* xt = X + hf * RS + 32 * I + col;     // A[j][i] = X_ij
      const float* qb = sQ + hf * RS + 32 * J + col;    // B[i][r] = q_ir m_v[r]
      auto fa = [&](int kk) { return xt[kk * RS]; };
      auto fb = [&](int kk) { return qb[kk * RS] * m; };
      if (I == 0) dka = mm16(dka, 0, fa, fb);
      dka = mm16(dka, 32, fa, fb);
    }
  }

  // ---- outputs: the pair part of dq (rows in the sequence), this head's [dk | dv] part
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ri = 32 * I + mrow(i, hf);
    if (ri < clen) dq[(qrow0 + ri) * DH + 32 * J + col] = dqa[i];
  }
  float* kp = kpart + (((size_t)unit * n_parts + hh) * npad + t0) * (DH + DV);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rj = 32 * I + mrow(i, hf);
    kp[(size_t)rj * (DH + DV) + 32 * J + col] = dka[i];
    kp[(size_t)rj * (DH + DV) + DH + 32 * J + col] = dva[i];
  }
}

// ---------------------------------------------------------------------------
// State part of dq:  dq_i += sum_f c_f (H_{<c} g_i)_f d psi_f(q_i) / dq_i, added to
// the pair part the query kernel wrote.  Block (32 tokens of a chunk, chunk, query
// head), two waves; the features by the row blocks above.  Per block,
// E[f][tok] = sum_w c_f H_{<c}[f][w] g_tok[w] on the fp32 matrix cores (wave = tile
// of 32 slots, N = the 32 tokens, K = channels): each lane loads its A operands,
// c_f H_{<c}[slot][2 j + lane / 32], straight from the state (the slots of a row run
// are consecutive features, so the loads coalesce), a block ahead of their use; g is
// read once into registers as the B operands.  E goes to LDS by slot, in two
// buffers, so one barrier per block separates the products from the update.  Four
// threads per token each own DH / 4 entries of dq in registers: a pair (m, t) of a
// row adds E q_m to dq[t] (the t side, a masked multiply-add over the thread's
// entries) and E q_t to dq[m] (the m side, a dot product over t summed over the
// parts; every m < DH receives exactly one, stored to LDS).  The diagonal (m, m)
// thus gets 2 E q_m; the linear features' m side (the constant slot q~[64] = 1) is
// dropped.  The blocks of one (unit, chunk) share an XCD (workgroup id % 8), so its
// state is read through one L2.
constexpr int DQ_TG = 32;   // tokens per block
template <typename T>
__global__ void __launch_bounds__(128)
k_bwd_dqstate(int n_q_heads, int n_kv_heads, int seq_len, int chunk, int n_chunks, int n_units,
              const T* __restrict__ q, const void* __restrict__ coeffs,
              const float* __restrict__ gbuf, const float* __restrict__ hc, float* __restrict__ dq) {
  constexpr int TG = DQ_TG;
  constexpr int NTP = DH / 4;            // dq entries per thread
  constexpr int ES = TG + 1;             // E row stride (bank spread)
  constexpr int RS = DH + 1;             // m-side row stride
  constexpr int GS = W + 1;              // g row: channels 0..64 and a zero
  constexpr int NJ = (W + 1) / 2;        // 33 channel pairs
  const int rep = n_q_heads / n_kv_heads;
  const int per = rep * (chunk / TG);    // blocks of one (unit, chunk)
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int uc = (slot / per) * 8 + xcd;
  if (uc >= n_units * n_chunks) return;
  const int unit = uc / n_chunks, c = uc % n_chunks;
  const int b = unit / n_kv_heads;
  const int hq = (unit % n_kv_heads) * rep + (slot % per) % rep;
  const int t0 = c * chunk + ((slot % per) / rep) * TG;
  const int ntok = min(TG, seq_len - t0);
  if (ntok <= 0) return;                 // a group past the sequence (whole block)
  const int tid = threadIdx.x, lane = tid & 63;
  const int FT = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave's feature tile
  const int qx = tid >> 2, half = tid & 3;                    // token and part
  const int hout = lane >> 5, tok = lane & 31;                // matrix-core roles

  // one array, in this order: the masked reads of an E buffer reach up to 63 slots
  // before it (s_rd, or the other buffer) and one slot after it (the other buffer,
  // or the tail)
  __shared__ __attribute__((aligned(16))) float sm[TG * RS + 2 * 64 * ES + TG];
  float* s_rd = sm;                      // [TG][RS] the m-side sums
  float* s_E0 = s_rd + TG * RS;          // [2][64][ES] E[slot][tok]; first the g tile [TG][GS]
  static_assert(TG * GS <= 64 * ES, "the g tile fits an E buffer");
  static_assert(63 * ES <= TG * RS && TG <= 64 * ES, "masked reads stay in the array");
  float* s_g = s_E0;

  const float* rec = coef_rec(coeffs, hq);
  const float* Hc = hc + ((size_t)unit * n_chunks + c) * STATE_FLOATS;
  const size_t row0 = ((size_t)b * n_q_heads + hq) * seq_len + t0;     // q and dq rows
  const float* grow = gbuf + (((size_t)b * n_q_heads + hq) * ((size_t)n_chunks * chunk) + t0) * WP;
  const bool active = qx < ntok;
  const T* qrow = q + (row0 + (active ? qx : 0)) * DH;

  for (int i = tid; i < TG * GS; i += 128) {
    const int r = i / GS, w = i % GS;
    s_g[i] = r < ntok && w < W ? grow[(size_t)r * WP + w] : 0.f;
  }
  float qt[NTP];   // this thread's q entries NTP half + j
#pragma unroll
  for (int j = 0; j < NTP; ++j) qt[j] = active ? Elem<T>::load(qrow, NTP * half + j) : 0.f;
  float dqt[NTP];
#pragma unroll
  for (int j = 0; j < NTP; ++j) dqt[j] = 0.f;
  __syncthreads();
  float gv[NJ];    // B operands: g[tok][2 j + lane / 32] (channel 65: zero)
#pragma unroll
  for (int j = 0; j < NJ; ++j) gv[j] = s_g[tok * GS + 2 * j + hout];

  // A operands, c_f and the multipliers q_m of a row block, loaded two blocks ahead
  // into one of two register sets (the loop is unrolled by two).  Every load is
  // unconditional (clamped index) and its value is kept raw until its block uses
  // it, where the selects drop what is not wanted: a load in a divergent block, or a
  // value used right after its load, is awaited at once, and with it (the counter
  // drains in order) every load still in flight.
  struct Ops {
    float a[NJ], cf;
    T q0, q1;
    bool ok, m0, m1;
  };
  auto fetch_block = [&](int blk, Ops& o) __attribute__((always_inline)) {
    const RowBlk d = row_block(blk);
    const int fs = row_block_feature(blk, d, 32 * FT + tok);
    const float* hp = Hc + max(fs, 0);   // an empty slot reads feature 0
#pragma unroll
    for (int j = 0; j < NJ; ++j) o.a[j] = hp[(size_t)min(2 * j + hout, W - 1) * DS];   // channel 65: any finite value
    o.cf = rec[coef_index(max(fs, 0))];
    o.q0 = qrow[min(d.m0, DH - 1)];
    o.q1 = qrow[min(d.m1, DH - 1)];
    o.ok = fs >= 0;
    o.m0 = d.m0 < DH && active;
    o.m1 = d.m1 < DH && active;
  };
  auto run_block = [&](int blk, Ops& o) __attribute__((always_inline)) {
    const RowBlk d = row_block(blk);
    float* s_E = s_E0 + (blk & 1) * 64 * ES;
    const float cf = o.ok ? o.cf : 0.f;   // zero for an empty slot
    const float q0 = o.m0 ? Elem<T>::load(&o.q0, 0) : 1.f;
    const float q1 = o.m1 ? Elem<T>::load(&o.q1, 0) : 1.f;
    if (32 * FT < d.na + d.nb) {   // else an empty tile (the column block)
      fx16 D;   // one chain: stored as it stands, without an add
#pragma unroll
      for (int i = 0; i < 16; ++i) D[i] = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) D = mfma_f32(cf * o.a[j], gv[j], D);
#pragma unroll
      for (int i = 0; i < 16; ++i)   // every slot of a non-empty tile is used
        s_E[(32 * FT + mrow(i, hout)) * ES + tok] = D[i];
    }
    // the set is free again; unconditional (the last two blocks reload a block),
    // so that the wait before the other set's products counts only its own loads
    fetch_block(min(blk + 2, NRB - 1), o);
    // one barrier: this block's E is complete, and the buffer written next (the
    // block after) was last read two blocks back
    __syncthreads();
    // t side into the registers, m side as dot products, masked to the rows' runs.
    // Slot t - ta0 of row 0 and na + t - tb0 of row 1 are read for every t of the
    // thread; outside a run they lie in [-63, 64] slots from s_E, inside the array,
    // and are dropped.
    float d0 = 0.f, d1 = 0.f;
    {
      const int lo = d.ta0 - NTP * half;           // j of the run's first t
      const float* ep = s_E + (NTP * half - d.ta0) * ES + qx;
#pragma unroll
      for (int j = 0; j < NTP; ++j) {
        const float r = ep[j * ES];
        const float e0 = (unsigned)(j - lo) < (unsigned)d.na ? r : 0.f;
        dqt[j] = fmaf(e0, q0, dqt[j]);
        d0 = fmaf(e0, qt[j], d0);
      }
    }
    if (d.nb > 0) {
      const int lo = d.tb0 - NTP * half;
      const float* ep = s_E + (d.na + NTP * half - d.tb0) * ES + qx;
#pragma unroll
      for (int j = 0; j < NTP; ++j) {
        const float r = ep[j * ES];
        const float e1 = (unsigned)(j - lo) < (unsigned)d.nb ? r : 0.f;
        dqt[j] = fmaf(e1, q1, dqt[j]);
        d1 = fmaf(e1, qt[j], d1);
      }
    }
    d0 += lane_xor1(d0);   // the token's parts are the lanes of one quad
    d1 += lane_xor1(d1);
    d0 += lane_xor2(d0);
    d1 += lane_xor2(d1);
    if (half == 0) {
      if (d.m0 < DH) s_rd[qx * RS + d.m0] = d0;
      if (d.nb > 0) s_rd[qx * RS + d.m1] = d1;
    }
  };
  static_assert(NRB % 2 == 0, "the loop takes the row blocks in pairs");
  Ops oa, ob;
  fetch_block(0, oa);
  fetch_block(1, ob);
  __syncthreads();   // the g tile has been read: the E buffers are free
  for (int blk = 0; blk < NRB; blk += 2) {
    run_block(blk, oa);
    run_block(blk + 1, ob);
  }
  __syncthreads();
  if (active) {
    float* o = dq + (row0 + qx) * DH + NTP * half;
#pragma unroll
    for (int j = 0; j < NTP; ++j) o[j] += dqt[j] + s_rd[qx * RS + NTP * half + j];
  }
}

// ---------------------------------------------------------------------------
// Suffix deltas and the state part of dc.  Block (feature block, chunk, unit).
// Per query head of the unit, the tile R_h[f][w] = sum_i psi_f(q_i) g_i[w] of the
// block's 64 features is formed on the fp32 matrix cores (M = features, N =
// channels, K = tokens; wave = (feature half wave % 2, channel half wave / 2); A =
// psi_f(q) of the lane's own feature, B = the staged g rows; the all-ones channel
// as a multiply-add per product on the waves of channel half 0) and passed through
// LDS to the thread layout below: thread feature f = 64 fb + (tid & 63), columns
// w = 16 (tid >> 6) + j, j < 16, and the all-ones channel on the fourth wave, which
// adds c_f R_h into the suffix delta and H_{<c} . R_h into the state part of dc.
template <typename T>
__global__ void __launch_bounds__(256, 2)   // two blocks per CU: 256 registers a lane
k_bwd_rbuild(int n_q_heads, int n_kv_heads, int seq_len, int chunk, int n_chunks,
             const T* __restrict__ q, const void* __restrict__ coeffs,
             const float* __restrict__ gbuf, const float* __restrict__ hc,
             float* __restrict__ rc, float* __restrict__ dcp) {
  const int fb = blockIdx.x;
  const int c = blockIdx.y;
  const int unit = blockIdx.z;
  const int b = unit / n_kv_heads, kv = unit % n_kv_heads;
  const int rep = n_q_heads / n_kv_heads;
  const int tid = threadIdx.x;
  const int f = fb * FB + (tid & 63);
  const int wq = tid >> 6;
  __shared__ float s_q[TB][DH + 1];                          // q~ = (q, 1) rows, zero past the sequence
  __shared__ __attribute__((aligned(16))) float s_g[TB][WP];
  __shared__ __attribute__((aligned(16))) float s_R[FB][WP];  // R_h of the block
  int r, t;
  const int kind = feat_decode(f, r, t);
  const size_t slot = ((size_t)unit * n_chunks + c) * STATE_FLOATS;
  // columns of this thread: 16 wq .. 16 wq + 15 (read as four 16-byte rows of g),
  // and the all-ones channel W - 1 on wave 3
  auto col_of = [&](int j) { return j < 16 ? 16 * wq + j : (wq == 3 ? W - 1 : -1); };
  float hval[WPT], rd[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = col_of(j);
    hval[j] = w >= 0 ? hc[slot + (size_t)w * DS + f] : 0.f;
    rd[j] = 0.f;
  }
  // the matrix-core roles: this lane's feature (A rows) and channel column (B)
  const int wave = __builtin_amdgcn_readfirstlane(wq), lane = tid & 63;
  const int FT = wave & 1, WT = wave >> 1, kpar = lane >> 5;
  const int fa = fb * FB + 32 * FT + (lane & 31);
  int ra, ta;
  const int kinda = feat_decode(fa, ra, ta);
  const int ia = kinda == 0 ? DH : ra, ib = kinda == 2 ? ta : DH;   // psi = q~[ia] q~[ib]
  const float amask = kinda == 3 ? 0.f : 1.f;
  const int t0 = c * chunk;
  const int t1 = min(seq_len, t0 + chunk);
  const size_t npad = (size_t)n_chunks * chunk;
  // Two barriers per head (chunk 64): one after the staging, one after R_h is in
  // LDS.  The staging of a head follows the last one's reads of s_R in program
  // order, and its products' reads of s_q and s_g precede that head's R_h
  // barrier.  Each wave stores its own part of the state part of dc (its columns);
  // k_bwd_dcoef adds the DC_PARTS parts.
  const size_t dc_stride = (size_t)gridDim.z / n_kv_heads * n_q_heads * n_chunks * DS;   // one part
  for (int hh = 0; hh < rep; ++hh) {
    const int hq = kv * rep + hh;
    const float cf = coef_of(coef_rec(coeffs, hq), f);
    fx16 D[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) D[x][i] = 0.f;
    float d64 = 0.f;   // all-ones channel of the lane's feature, its tokens of parity kpar
    const size_t qrow0 = ((size_t)b * n_q_heads + hq) * seq_len;
    const size_t grow0 = ((size_t)b * n_q_heads + hq) * npad;
    for (int i0 = t0; i0 < t1; i0 += TB) {
      const int ni = min(TB, t1 - i0);
      if (i0 > t0) __syncthreads();   // the previous token tile's products are done
      // the q and g rows of the tile are contiguous in memory, one span each
      const T* qt = q + (qrow0 + i0) * DH;
      const float* gt = gbuf + (grow0 + i0) * WP;
      stage_span<TB * DH>(tid, ni * DH, [&](int i) { return Elem<T>::load(qt, i); },
                          [&](int i, float x) { s_q[i / DH][i % DH] = x; });
      stage_span<TB * WP>(tid, ni * WP, [&](int i) { return gt[i]; },
                          [&](int i, float x) { s_g[i / WP][i % WP] = x; });
      if (tid < TB) s_q[tid][DH] = tid < ni ? 1.f : 0.f;
      __syncthreads();
#pragma unroll
      for (int j0 = 0; j0 < TB / 2; j0 += 8) {
        float av[8], bv[8], gv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int tok = 2 * (j0 + jj) + kpar;
          av[jj] = amask * s_q[tok][ia] * s_q[tok][ib];
          bv[jj] = s_g[tok][32 * WT + (lane & 31)];
          gv[jj] = s_g[tok][W - 1];
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          D[jj & 1] = mfma_f32(av[jj], bv[jj], D[jj & 1]);
          d64 = fmaf(av[jj], gv[jj], d64);
        }
      }
    }
    // R_h to LDS (the previous head's readers are done: the staging barrier)
#pragma unroll
    for (int i = 0; i < 16; ++i) s_R[32 * FT + mrow(i, kpar)][32 * WT + (lane & 31)] = D[0][i] + D[1][i];
    d64 += __shfl_xor(d64, 32, 64);
    if (WT == 0 && kpar == 0) s_R[32 * FT + (lane & 31)][W - 1] = d64;
    __syncthreads();
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int w = col_of(j);
      const float x = w >= 0 ? s_R[tid & 63][w] : 0.f;
      rd[j] = fmaf(cf, x, rd[j]);
      part = fmaf(hval[j], x, part);
    }
    if (dcp != nullptr)
      dcp[wq * dc_stride + (((size_t)b * n_q_heads + hq) * n_chunks + c) * DS + f] = kind == 3 ? 0.f : part;
  }
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = col_of(j);
    if (w >= 0) rc[slot + (size_t)w * DS + f] = rd[j];
  }
}

// Exclusive suffix sums over the chunks of every unit, in place: the loads of RB
// chunks in flight at a time (clamped index, unconditional), so that each thread
// waits out the memory latency n_chunks / RB times rather than n_chunks.
__global__ void __launch_bounds__(256)
k_bwd_rscan(int n_chunks, float* __restrict__ rc) {
  constexpr int RB = 8;
  const int unit = blockIdx.y;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= STATE_FLOATS) return;
  float* p = rc + (size_t)unit * n_chunks * STATE_FLOATS + e;
  float run = 0.f;
  for (int c0 = n_chunks - 1; c0 >= 0; c0 -= RB) {
    float x[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) x[j] = p[(size_t)max(c0 - j, 0) * STATE_FLOATS];
#pragma unroll
    for (int j = 0; j < RB; ++j)
      if (c0 - j >= 0) {
        p[(size_t)(c0 - j) * STATE_FLOATS] = run;
        run += x[j];
      }
  }
}

// ---------------------------------------------------------------------------
// Key side, the chunk's pairs.  One block per (chunk, unit, slot): slot s sums the
// chunk's pairs (i >= j) of query head kv * rep + s.  SP threads per key (thread
// SP j + h for key t0 + j) split the pairs by query index mod SP; each thread writes
// its part of [dk_j | dv_j] to kpart (part h rep + slot of the unit's SP rep + KS_NFS
// parts; the last KS_NFS are k_bwd_kstate's), and k_bwd_ksum adds the parts in order.
template <typename T, int SP>
__global__ void __launch_bounds__(256)
k_bwd_key(int n_q_heads, int n_kv_heads, int seq_len, int chunk, int n_chunks,
          const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
          const void* __restrict__ coeffs, const float* __restrict__ gbuf,
          float* __restrict__ kpart) {
  const int c = blockIdx.x;
  const int rep = n_q_heads / n_kv_heads;
  const int unit = blockIdx.y / rep;
  const int slot = blockIdx.y % rep;
  const int b = unit / n_kv_heads, kv = unit % n_kv_heads;
  if (SP == 4 && reinterpret_cast<const int32_t*>(coef_rec(coeffs, kv * rep + slot))[OAL_COEF_NG] >= 1)
    return;   // chunk 64, grouped record: k_bwd_pair wrote this head's part
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;                // SP * chunk
  const int jx = tid / SP;                    // key of the chunk
  const int half = tid % SP;                  // this thread's part
  const int t0 = c * chunk;
  const int clen = min(chunk, seq_len - t0);
  const bool active = jx < clen;

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* s_k = smem;                          // [chunk][DH + 1]
  float* s_dk = s_k + chunk * (DH + 1);       // [SP][chunk][DH + 1]
  float* s_q = s_dk + SP * chunk * (DH + 1);  // [TB][DH + 1]
  float* s_g = s_q + TB * (DH + 1);           // [TB][WP]
  float* s_b = s_g + TB * WP;                 // [DH]
  float* s_S = s_b + DH;                      // [DH][DH]

  const size_t krow0 = (size_t)unit * seq_len + t0;
  {
    const T* ks = k + krow0 * DH;   // the chunk's key rows, one span (clen >= 1)
    stage_span<(256 / SP) * DH>(tid, clen * DH, [&](int i) { return Elem<T>::load(ks, i); },
                                [&](int i, float x) { s_k[(i / DH) * (DH + 1) + i % DH] = x; });
  }
  for (int i = tid; i < SP * chunk * (DH + 1); i += nthr) s_dk[i] = 0.f;
  float uj[WP];
#pragma unroll
  for (int w = 0; w < WP; ++w) uj[w] = 0.f;
  if (active) {
#pragma unroll
    for (int w = 0; w < DV; ++w) uj[w] = Elem<T>::load(v, (krow0 + jx) * DV + w);
    uj[DV] = 1.f;
  }
  __syncthreads();
  const float* kj = s_k + jx * (DH + 1);
  float* dkj = s_dk + (half * chunk + jx) * (DH + 1);
  float du[WP];
#pragma unroll
  for (int w = 0; w < WP; ++w) du[w] = 0.f;

  // ---- the chunk's pairs (i >= j) of this slot's query head
  const size_t npad = (size_t)n_chunks * chunk;
  __shared__ __attribute__((aligned(16))) GroupTab gt;
  {
    const int hq = kv * rep + slot;
    const float* rec = coef_rec(coeffs, hq);
    const float a = rec[OAL_COEF_A];
    const bool grouped = reinterpret_cast<const int32_t*>(rec)[OAL_COEF_NG] >= 1;
    const size_t qrow0 = ((size_t)b * n_q_heads + hq) * seq_len;
    const size_t grow0 = ((size_t)b * n_q_heads + hq) * npad;
    __syncthreads();
    if (grouped) build_group_tab(gt, rec, tid);
    for (int i = tid; i < DH; i += nthr) s_b[i] = rec[OAL_COEF_BP + i];
    stage_span<DH * DH>(tid, DH * DH, [&](int i) { return rec[OAL_COEF_CM + i]; },
                        [&](int i, float x) { s_S[i] = x; });
    for (int i0 = 0; i0 < clen; i0 += TB) {
      const int ni = min(TB, clen - i0);
      __syncthreads();
      const T* qs = q + (qrow0 + t0 + i0) * DH;        // the tile's q rows and g rows,
      const float* gs = gbuf + (grow0 + t0 + i0) * WP;  // one span each (ni >= 1)
      stage_span<TB * DH>(tid, ni * DH, [&](int i) { return Elem<T>::load(qs, i); },
                          [&](int i, float x) { s_q[(i / DH) * (DH + 1) + i % DH] = x; });
      stage_span<TB * WP>(tid, ni * WP, [&](int i) { return gs[i]; },
                          [&](int i, float x) { s_g[i] = x; });
      __syncthreads();
      const bool fast = grouped && gt.n_out <= MAX_OUT;   // uniform over the block
      if (active) {
        const int ii0 = max(0, jx - i0);
        for (int ii = ii0 + (((half - ii0) % SP) + SP) % SP; ii < ni; ii += SP) {
          const float* qi = s_q + ii * (DH + 1);
          const float* gi = s_g + ii * WP;
          const float al = dot_row(gi, uj);
          if (fast) {
            float w[LDIM];
            const float kap = grouped_pair(qi, kj, gt, w);
            grouped_grad(dkj, al, qi, gt, w);
            axpy_row(du, kap, gi);
            continue;
          }
          float p[DH];
#pragma unroll
          for (int t = 0; t < DH; ++t) p[t] = qi[t] * kj[t];
          float kap = a;
#pragma unroll 1
          for (int r = 0; r < DH; ++r) {
            const float sp = srow_dot(s_S + r * DH, p);
            kap = fmaf(s_b[r] + sp, qi[r] * kj[r], kap);   // p_r from LDS: r is not unrolled
            dkj[r] = fmaf(al * qi[r], s_b[r] + 2.f * sp, dkj[r]);
          }
          axpy_row(du, kap, gi);
        }
      }
    }
  }
  if (active) {
    float* o = kpart + (((size_t)unit * (SP * rep + KS_NFS) + half * rep + slot) * npad + t0 + jx) * (DH + DV);
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] = dkj[d];
#pragma unroll
    for (int w = 0; w < DV; ++w) o[DH + w] = du[w];
  }
}

// ---------------------------------------------------------------------------
// Key side, the later chunks through R = R_{>c} (the suffix states, with c_f and the
// query heads of the group folded in):  dv_j += R^T psi(k_j) and
// dk_j += sum_f (R u_j)_f d psi_f(k_j) / dk_j, u_j = (v_j, 1).  Block (32 keys,
// chunk, unit, feature split): two waves over a quarter of the row blocks.  Per row
// block each lane loads its A operands R[slot][2 j + lane / 32] straight from the
// state a block ahead (the slots of a run are consecutive features: coalesced) and
// copies them to LDS; on the fp32 matrix cores
//   E[slot][tok] = sum_w R[slot][w] u_tok[w]   (wave = tile of 32 slots, K = channels,
//                                               u read once into registers)
//   dv[tok][w] += sum_slot psi_slot(k_tok) R[slot][w]
//                                              (wave = tile of 32 channels, K = slots,
//                                               A = k~[ia] k~[ib] from the key rows and
//                                               the block's slot table, B = R from LDS)
// and E goes through the same t-side / m-side update as the query side (four
// threads per key, 16 entries of dk each in registers).  The block's [dk | dv] is
// one part of kpart (part part0 + split); k_bwd_ksum adds the parts.  The blocks of
// one (unit, chunk) share an XCD (workgroup id % 8).
constexpr int KS_TG = 32;   // keys per block
template <typename T>
__global__ void __launch_bounds__(128)
k_bwd_kstate(int n_kv_heads, int seq_len, int chunk, int n_chunks, int n_units, int part0,
             int nparts, const T* __restrict__ k, const T* __restrict__ v,
             const float* __restrict__ rc, float* __restrict__ kpart) {
  constexpr int TG = KS_TG;
  constexpr int NTP = DH / 4;            // dk entries per thread
  constexpr int ES = TG + 1;             // E row stride (bank spread)
  constexpr int RS = DH + 1;             // m-side row stride
  constexpr int KR = DH + 2;             // key row: k, 1 (the constant slot), 0 (empty slots)
  constexpr int GS = W + 1;              // u row: channels 0..64 and a zero
  constexpr int NJ = (W + 1) / 2;        // 33 channel pairs
  const int per = (chunk / TG) * KS_NFS;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int uc = (slot / per) * 8 + xcd;
  if (uc >= n_units * n_chunks) return;
  const int unit = uc / n_chunks, c = uc % n_chunks;
  const int split = (slot % per) % KS_NFS;
  const int t0 = c * chunk + ((slot % per) / KS_NFS) * TG;
  const int ntok = min(TG, seq_len - t0);
  if (ntok <= 0) return;                 // a group past the sequence (whole block)
  const int blk0 = NRB * split / KS_NFS, blk1 = NRB * (split + 1) / KS_NFS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int FT = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave's tile
  const int qx = tid >> 2, half = tid & 3;                    // key and part
  const int hout = lane >> 5, tok = lane & 31;                // matrix-core roles

  // one array, in this order: the masked reads of an E buffer reach up to 63 slots
  // before it (s_rd, or the other buffer) and one slot after it (the other buffer,
  // or the tail)
  __shared__ __attribute__((aligned(16))) float sm[TG * RS + 2 * 64 * ES + TG + 2 * 64 * WPH + TG * KR];
  __shared__ int s_fd[2][64];            // the block's slots: k~[ia] k~[ib] = ia | ib << 8
  float* s_rd = sm;                      // [TG][RS] the m-side sums
  float* s_E0 = s_rd + TG * RS;          // [2][64][ES] E[slot][tok]; first the u tile [TG][GS]
  float* s_R0 = s_E0 + 2 * 64 * ES + TG; // [2][64][WPH] the block's R rows
  float* s_k = s_R0 + 2 * 64 * WPH;      // [TG][KR] the key rows
  static_assert(TG * GS <= 64 * ES, "the u tile fits an E buffer");
  static_assert(63 * ES <= TG * RS, "masked reads stay in the array");
  float* s_u = s_E0;

  const float* Rs = rc + ((size_t)unit * n_chunks + c) * STATE_FLOATS;
  const size_t row0 = (size_t)unit * seq_len + t0;     // k, v rows
  const bool active = qx < ntok;
  stage_span<TG * DH, 128>(tid, ntok * DH, [&](int i) { return Elem<T>::load(k + row0 * DH, i); },
                           [&](int i, float x) { s_k[(i / DH) * KR + i % DH] = x; });
  stage_span<TG * DV, 128>(tid, ntok * DV, [&](int i) { return Elem<T>::load(v + row0 * DV, i); },
                           [&](int i, float x) { s_u[(i / DV) * GS + i % DV] = x; });
  if (tid < TG) {
    s_k[tid * KR + DH] = 1.f;
    s_k[tid * KR + DH + 1] = 0.f;
    s_u[tid * GS + DV] = tid < ntok ? 1.f : 0.f;
    s_u[tid * GS + DV + 1] = 0.f;
  }
  for (int i = tid; i < TG * RS; i += 128) s_rd[i] = 0.f;   // a split leaves some m-side sums out
  float dkt[NTP];
#pragma unroll
  for (int j = 0; j < NTP; ++j) dkt[j] = 0.f;
  fx16 DVa;   // dv[tok][32 FT + lane % 32] of this split, rows mrow(i, lane / 32)
#pragma unroll
  for (int i = 0; i < 16; ++i) DVa[i] = 0.f;
  // the constant feature (psi = 1, no dk part, so in no row block) adds R[0][w] to
  // every key's dv: split 0 carries it
  const float r0w = split == 0 ? Rs[(size_t)(32 * FT + tok) * DS] : 0.f;
  __syncthreads();
  float kt[NTP];   // this thread's k entries NTP half + j
#pragma unroll
  for (int j = 0; j < NTP; ++j) kt[j] = s_k[qx * KR + NTP * half + j];
  float gv[NJ];    // B operands of E: u[tok][2 j + lane / 32] (channel 65: zero)
#pragma unroll
  for (int j = 0; j < NJ; ++j) gv[j] = s_u[tok * GS + 2 * j + hout];

  // A operands of the next block and the slot's feature; loads unconditional
  // (clamped index), their values used a block later (see k_bwd_dqstate)
  float na[NJ];
  int nfs = 0;
  auto fetch_block = [&](int blk) {
    const RowBlk d = row_block(blk);
    nfs = row_block_feature(blk, d, 32 * FT + tok);
    const float* rp = Rs + max(nfs, 0);   // an empty slot reads feature 0
#pragma unroll
    for (int j = 0; j < NJ; ++j) na[j] = rp[(size_t)min(2 * j + hout, W - 1) * DS];   // channel 65: any finite value
  };
  fetch_block(blk0);
  __syncthreads();   // the u tile has been read: the E buffers are free
  for (int blk = blk0; blk < blk1; ++blk) {
    const RowBlk d = row_block(blk);
    const int bf = (blk - blk0) & 1;
    float* s_E = s_E0 + bf * 64 * ES;
    float* s_R = s_R0 + bf * 64 * WPH;
    // this block's R rows to LDS (for the dv product) and the slot table
    {
      const bool ok = nfs >= 0;
      const int sl = 32 * FT + tok;
      float* rrow = s_R + sl * WPH + hout;
#pragma unroll
      for (int j = 0; j < NJ; ++j) rrow[2 * j] = ok ? na[j] : 0.f;
      if (hout == 0) {
        int r, t;
        const int kind = feat_decode(max(nfs, 0), r, t);
        const int ia = !ok ? DH + 1 : (kind == 0 ? DH : r);
        const int ib = !ok ? DH + 1 : (kind == 2 ? t : DH);
        s_fd[bf][sl] = ia | (ib << 8);
      }
    }
    if (32 * FT < d.na + d.nb) {   // else an empty tile (the column block)
      fx16 D;
#pragma unroll
      for (int i = 0; i < 16; ++i) D[i] = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) D = mfma_f32(na[j], gv[j], D);
#pragma unroll
      for (int i = 0; i < 16; ++i)   // every slot of a non-empty tile is used
        s_E[(32 * FT + mrow(i, hout)) * ES + tok] = D[i];
    }
    fetch_block(min(blk + 1, blk1 - 1));   // unconditional: the last block reloads itself
    // one barrier: this block's E, R rows and slot table are complete, and the
    // buffers written next (the block after) were last read two blocks back
    __syncthreads();
    // dk: t side into the registers, m side as dot products (masked as on the query side)
    const float k0 = s_k[qx * KR + d.m0], k1 = s_k[qx * KR + d.m1];
    float d0 = 0.f, d1 = 0.f;
    {
      const int lo = d.ta0 - NTP * half;
      const float* ep = s_E + (NTP * half - d.ta0) * ES + qx;
#pragma unroll
      for (int j = 0; j < NTP; ++j) {
        const float r = ep[j * ES];
        const float e0 = (unsigned)(j - lo) < (unsigned)d.na ? r : 0.f;
        dkt[j] = fmaf(e0, k0, dkt[j]);
        d0 = fmaf(e0, kt[j], d0);
      }
    }
    if (d.nb > 0) {
      const int lo = d.tb0 - NTP * half;
      const float* ep = s_E + (d.na + NTP * half - d.tb0) * ES + qx;
#pragma unroll
      for (int j = 0; j < NTP; ++j) {
        const float r = ep[j * ES];
        const float e1 = (unsigned)(j - lo) < (unsigned)d.nb ? r : 0.f;
        dkt[j] = fmaf(e1, k1, dkt[j]);
        d1 = fmaf(e1, kt[j], d1);
      }
    }
    d0 += lane_xor1(d0);
    d1 += lane_xor1(d1);
    d0 += lane_xor2(d0);
    d1 += lane_xor2(d1);
    if (half == 0) {
      if (d.m0 < DH) s_rd[qx * RS + d.m0] = d0;
      if (d.nb > 0) s_rd[qx * RS + d.m1] = d1;
    }
    // dv: K = the block's 64 slots, two per product
    {
      const float* krow = s_k + tok * KR;
      const float* rcol = s_R + hout * WPH + 32 * FT + tok;
#pragma unroll
      for (int i0 = 0; i0 < 32; i0 += 8) {
        float av[8], bv[8];
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int dd = s_fd[bf][2 * (i0 + ii) + hout];
          av[ii] = krow[dd & 255] * krow[dd >> 8];
          bv[ii] = rcol[2 * (i0 + ii) * WPH];
        }
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) DVa = mfma_f32(av[ii], bv[ii], DVa);
      }
    }
  }
  __syncthreads();
  float* kp = kpart + ((size_t)unit * nparts + part0 + split) * ((size_t)n_chunks * chunk) * (DH + DV);
  if (active) {
    float* o = kp + (size_t)(t0 + qx) * (DH + DV) + NTP * half;
#pragma unroll
    for (int j = 0; j < NTP; ++j) o[j] = dkt[j] + s_rd[qx * RS + NTP * half + j];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = mrow(i, hout);
    if (r < ntok) kp[(size_t)(t0 + r) * (DH + DV) + DH + 32 * FT + tok] = DVa[i] + r0w;
  }
}

// dk, dv = the sum of the parts of every key, in order.  Parts 0 .. ks rep - 1 are the
// pair parts, part h rep + s the h-th of query head s (k_bwd_key); then the nparts -
// ks rep state parts (k_bwd_kstate).  With pair_mfma set, a head with a grouped
// record has its pair part in part s alone (k_bwd_pair): when every head of the unit
// has one, the parts rep .. ks rep - 1 are skipped as a whole.
__global__ void __launch_bounds__(256)
k_bwd_ksum(int n_kv_heads, int nparts, int ks, int rep, int pair_mfma, const void* __restrict__ coeffs,
           int seq_len, int npad, const float* __restrict__ kpart, float* __restrict__ dk,
           float* __restrict__ dv) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t per_unit = (size_t)seq_len * (DH + DV);
  const int unit = blockIdx.y;
  if (e >= per_unit) return;
  const size_t pos = e / (DH + DV);
  const int comp = (int)(e % (DH + DV));
  const int kv = unit % n_kv_heads;
  auto grouped = [&](int s) {
    return reinterpret_cast<const int32_t*>(coef_rec(coeffs, kv * rep + s))[OAL_COEF_NG] >= 1;
  };
  bool all_grouped = pair_mfma != 0;
  for (int s = 0; s < rep; ++s) all_grouped = all_grouped && grouped(s);
  const float* kp = kpart + ((size_t)unit * nparts * npad + pos) * (DH + DV) + comp;
  const size_t stride = (size_t)npad * (DH + DV);
  float s = 0.f;
  if (all_grouped) {
    for (int sl = 0; sl < rep; ++sl) s += kp[sl * stride];
    for (int sl = ks * rep; sl < nparts; ++sl) s += kp[sl * stride];
  } else {
    for (int sl = 0; sl < nparts; ++sl) {
      if (pair_mfma && sl >= rep && sl < ks * rep && grouped(sl % rep)) continue;
      s += kp[sl * stride];
    }
  }
  if (comp < DH) dk[((size_t)unit * seq_len + pos) * DH + comp] = s;
  else dv[((size_t)unit * seq_len + pos) * DV + comp - DH] = s;
}

// ---------------------------------------------------------------------------
// Pair part of dc: dc_f += sum_i psi_f(q_i) Y[i][f] with Y = alpha Psi(K) over the
// chunk's keys (alpha_ij = 0 for j > i).  One block per (chunk, query head); Y on
// the fp32 matrix cores one 32-feature tile at a time (wave w takes tiles w, w + 4,
// ...): token tiles of 32 rows (A = alpha rows), K = keys two per product, B =
// psi_f(k_j) of the lane's own feature formed in place (psi = k~[ia] k~[ib] with
// k~ = (k, 1)), key steps past a token tile's diagonal skipped; the weighted row
// sum in registers, the two lane halves added at the end.
template <typename T, int CH>
__global__ void __launch_bounds__(256)
k_bwd_dc_intra(int n_q_heads, int n_kv_heads, int seq_len, int n_chunks,
               const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ alpha,
               float* __restrict__ dcp) {
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / n_q_heads, hq = bh % n_q_heads;
  const int unit = b * n_kv_heads + hq / (n_q_heads / n_kv_heads);
  const int t0 = c * CH;
  const int clen = min(CH, seq_len - t0);
  const int tid = threadIdx.x;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* s_a = smem;                          // [CH][CH + 1] (rows padded: the lanes of a
                                              // product read 32 rows at one column)
  float* s_q = s_a + CH * (CH + 1);           // [CH][DH + 1]: q~ = (q, 1), zero past the sequence
  float* s_k = s_q + CH * (DH + 1);           // [CH][DH + 1]: k~ = (k, 1), likewise
  const float* ablk = alpha + ((size_t)bh * n_chunks + c) * CH * CH;
  for (int i = tid; i < CH * CH; i += blockDim.x) s_a[(i / CH) * (CH + 1) + i % CH] = ablk[i];
  const size_t qrow0 = (size_t)bh * seq_len + t0;
  const size_t krow0 = (size_t)unit * seq_len + t0;
  for (int i = tid; i < CH * DH; i += blockDim.x) {
    const int ii = i / DH, d = i % DH;
    s_q[ii * (DH + 1) + d] = ii < clen ? Elem<T>::load(q, (qrow0 + ii) * DH + d) : 0.f;
    s_k[ii * (DH + 1) + d] = ii < clen ? Elem<T>::load(k, (krow0 + ii) * DH + d) : 0.f;
  }
  for (int i = tid; i < CH; i += blockDim.x) {
    s_q[i * (DH + 1) + DH] = i < clen ? 1.f : 0.f;
    s_k[i * (DH + 1) + DH] = i < clen ? 1.f : 0.f;
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, kpar = lane >> 5;
  float* dout = dcp + ((size_t)bh * n_chunks + c) * DS;
  for (int ft = wave; ft < DS / 32; ft += 4) {
    const int f = 32 * ft + col;               // this lane's feature (B column)
    int r, t;
    const int kind = feat_decode(f, r, t);
    const int ia = kind == 0 ? DH : r, ib = kind == 2 ? t : DH;
    const float fm = kind == 3 ? 0.f : 1.f;
    float part = 0.f;
#pragma unroll
    for (int TT = 0; TT < CH / 32; ++TT) {
      fx16 D[2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) D[x][i] = 0.f;
      const float* arow = s_a + (32 * TT + col) * (CH + 1) + kpar;   // alpha[i][2 kk + kpar]
#pragma unroll
      for (int kk0 = 0; kk0 < 16 * (TT + 1); kk0 += 8) {   // keys j < 32 (TT + 1)
        float av[8], bv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = 2 * (kk0 + jj) + kpar;
          av[jj] = arow[2 * (kk0 + jj)];
          const float* kr = s_k + j * (DH + 1);
          bv[jj] = fm * kr[ia] * kr[ib];
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) D[jj & 1] = mfma_f32(av[jj], bv[jj], D[jj & 1]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* qr = s_q + (32 * TT + mrow(i, kpar)) * (DH + 1);
        part = fmaf(qr[ia] * qr[ib], D[0][i] + D[1][i], part);
      }
    }
    part += __shfl_xor(part, 32, 64);
    if (kpar == 0 && f < DCAN) dout[f] += part;
  }
}

// Sum over chunks and batch, then (da, db, dC) of [OAL] Eq. 3: the record's
// b' = b / sqrt(d_h) and c' = m C / d_h give db_r = dc_r / sqrt(d_h) and, for
// either entry of the pair, dC_rt = dc_rt / d_h.
__global__ void __launch_bounds__(256)
k_bwd_dcoef(int batch, int n_q_heads, int n_chunks, const float* __restrict__ dcp,
            float* __restrict__ da, float* __restrict__ db, float* __restrict__ dC) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  const int hq = blockIdx.y;
  if (f >= DCAN) return;
  float s = 0.f;
  const size_t part = (size_t)batch * n_q_heads * n_chunks * DS;
  for (int b = 0; b < batch; ++b) {
    const float* p = dcp + ((size_t)b * n_q_heads + hq) * n_chunks * DS + f;
    for (int c = 0; c < n_chunks; ++c)
#pragma unroll
      for (int k = 0; k < DC_PARTS; ++k) s += p[k * part + (size_t)c * DS];
  }
  int r, t;
  const int kind = feat_decode(f, r, t);
  if (kind == 0) {
    da[hq] = s;
  } else if (kind == 1) {
    db[(size_t)hq * DH + r] = s * 0.125f;
  } else {
    const float x = s * (1.0f / 64.0f);
    dC[(size_t)hq * DH * DH + r * DH + t] = x;
    dC[(size_t)hq * DH * DH + t * DH + r] = x;
  }
}

// ---------------------------------------------------------------------------
// (da, db, dC) -> dL through the grouped map of [OAL] §4.3: in the group sums the
// kernel is eps + sum_uv M_uv s_u s_v, so dM_00 = da, dM_{0,g} = dM_{g,0} =
// sum_{r in g} db_r, dM_{g,h} = sum_{r in g, t in h} dC_rt, and with M = L L^T,
// dL = (dM + dM^T) L on the lower triangle of the leading (G+1) block.
__global__ void __launch_bounds__(64)
k_coeffs_bwd(int g_max, const int32_t* __restrict__ n_groups, const int32_t* __restrict__ group_map,
             const float* __restrict__ Lin, const float* __restrict__ da,
             const float* __restrict__ db, const float* __restrict__ dC, float* __restrict__ dL) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int ld = g_max + 1;
  __shared__ int sg[DH];
  __shared__ float sL[LDIM][LDIM];
  __shared__ double sM[LDIM][LDIM];
  __shared__ int sG;
  if (tid == 0) {
    const int G = n_groups[h];
    sG = G < 1 ? 1 : (G > g_max ? g_max : G);
  }
  __syncthreads();
  const int G = sG;
  {
    const int gr = group_map[(size_t)h * DH + tid];
    sg[tid] = gr < 1 ? 1 : (gr > G ? G : gr);
  }
  if (tid < LDIM * LDIM) {
    const int u = tid / LDIM, w = tid % LDIM;
    sL[u][w] = (u <= G && w <= G && w <= u) ? Lin[(size_t)h * ld * ld + u * ld + w] : 0.f;
  }
  __syncthreads();
  if (tid < LDIM * LDIM) {
    const int u = tid / LDIM, w = tid % LDIM;
    double m = 0.0;
    if (u <= G && w <= G) {
      if (u == 0 && w == 0) {
        m = da[h];
      } else if (u == 0 || w == 0) {
        const int gam = u + w;
        for (int r = 0; r < DH; ++r)
          if (sg[r] == gam) m += db[(size_t)h * DH + r];
      } else {
        for (int r = 0; r < DH; ++r) {
          if (sg[r] != u) continue;
          for (int t = 0; t < DH; ++t)
            if (sg[t] == w) m += dC[(size_t)h * DH * DH + r * DH + t];
        }
      }
    }
    sM[u][w] = m;
  }
  __syncthreads();
  for (int i = tid; i < ld * ld; i += blockDim.x) {
    const int u = i / ld, w = i % ld;
    double x = 0.0;
    if (u <= G && w <= u) {
      for (int p = 0; p <= G; ++p) x += (sM[u][p] + sM[p][u]) * (double)sL[p][w];
    }
    dL[(size_t)h * ld * ld + i] = (float)x;
  }
}

// ---------------------------------------------------------------------------

oal_status launch_prefix_vec(int batch, int n_kv_heads, int seq_len, int chunk, oal_dtype in_dtype,
                             const void* k, const void* v, float* hc, hipStream_t stream);

template <typename T>
static oal_status backward_typed(int batch, int n_q_heads, int n_kv_heads, int seq_len, int chunk,
                                 oal_dtype in_dtype, const void* q, const void* k, const void* v,
                                 const void* coeffs, const float* dy, float* dq, float* dk,
                                 float* dv, float* da, float* db, float* dC, void* ws,
                                 hipStream_t stream) {
  const BwdWs w = bwd_ws(ws, batch, n_q_heads, n_kv_heads, seq_len, chunk);
  const int units = batch * n_kv_heads;
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  const T* qq = reinterpret_cast<const T*>(q);
  const T* kk = reinterpret_cast<const T*>(k);
  const T* vv = reinterpret_cast<const T*>(v);
  const bool want_coef = da != nullptr;
  oal_status st = launch_prefix_vec(batch, n_kv_heads, seq_len, chunk, in_dtype, k, v, w.hc, stream);
  if (st != OAL_OK) return st;
  {
    const int per = (n_q_heads / n_kv_heads) * (chunk / US_TG);
    const dim3 grid((unsigned)(((size_t)units * n_chunks + 7) / 8 * 8 * (size_t)per));
    ProfScope ps("k_bwd_ustate", stream);
    hipLaunchKernelGGL(k_bwd_ustate<T>, grid, dim3(128), 0, stream, n_q_heads, n_kv_heads, seq_len,
                       chunk, n_chunks, units, qq, coeffs, w.hc, w.gbuf);
    if ((st = check_launch("k_bwd_ustate")) != OAL_OK) return st;
  }
  const bool pair_mfma = chunk == PR_C;
  if (pair_mfma) {
    const size_t smem = sizeof(float) * 7 * (size_t)PR_C * PR_RS;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bwd_pair<T>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
      return set_error(OAL_ERR_HIP, "k_bwd_pair: cannot reserve %zu bytes of LDS", smem);
    const int rep = n_q_heads / n_kv_heads;
    const dim3 grid((unsigned)(((size_t)units * n_chunks + 7) / 8 * 8 * (size_t)rep));
    ProfScope ps("k_bwd_pair", stream);
    hipLaunchKernelGGL(k_bwd_pair<T>, grid, dim3(256), smem, stream, n_q_heads, n_kv_heads, seq_len,
                       n_chunks, units, key_split(chunk) * rep + KS_NFS, qq, kk, vv, coeffs, dy, w.gbuf,
                       w.alpha, dq, w.kpart);
    if ((st = check_launch("k_bwd_pair")) != OAL_OK) return st;
  }
  {
    // four threads per query at chunk 64 (256 threads, 143 KB of LDS), two at 128;
    // the kernel's state staging assumes SP * chunk = 256
    const int sp = chunk <= 64 ? 4 : 2;
    if (sp * chunk != 256) return set_error(OAL_ERR_INVALID_ARG, "k_bwd_query: chunk %d", chunk);
    const size_t smem = sizeof(float) * ((size_t)(1 + sp) * chunk * (DH + 1) +
                                         TB * (DH + 1) + TB * WP + DH + DH * DH);
    const void* fn = sp == 4 ? reinterpret_cast<const void*>(&k_bwd_query<T, 4>)
                             : reinterpret_cast<const void*>(&k_bwd_query<T, 2>);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
      return set_error(OAL_ERR_HIP, "k_bwd_query: cannot reserve %zu bytes of LDS", smem);
    const dim3 grid_q((unsigned)(((size_t)units * n_chunks + 7) / 8 * 8 * (size_t)(n_q_heads / n_kv_heads)));
    ProfScope ps("k_bwd_query", stream);
    if (sp == 4)
      hipLaunchKernelGGL((k_bwd_query<T, 4>), grid_q, dim3(4 * chunk), smem,
                         stream, n_q_heads, n_kv_heads, seq_len, chunk, n_chunks, units, qq, kk, vv, coeffs, dy,
                         w.gbuf, w.alpha, dq);
    else
      hipLaunchKernelGGL((k_bwd_query<T, 2>), grid_q, dim3(2 * chunk), smem,
                         stream, n_q_heads, n_kv_heads, seq_len, chunk, n_chunks, units, qq, kk, vv, coeffs, dy,
                         w.gbuf, w.alpha, dq);
    if ((st = check_launch("k_bwd_query")) != OAL_OK) return st;
  }
  {
    const int per = (n_q_heads / n_kv_heads) * (chunk / DQ_TG);
    const dim3 grid((unsigned)(((size_t)units * n_chunks + 7) / 8 * 8 * (size_t)per));
    ProfScope ps("k_bwd_dqstate", stream);
    hipLaunchKernelGGL(k_bwd_dqstate<T>, grid, dim3(128), 0, stream, n_q_heads, n_kv_heads, seq_len,
                       chunk, n_chunks, units, qq, coeffs, w.gbuf, w.hc, dq);
    if ((st = check_launch("k_bwd_dqstate")) != OAL_OK) return st;
  }
  {
    ProfScope ps("k_bwd_rbuild", stream);
    hipLaunchKernelGGL(k_bwd_rbuild<T>, dim3(NFB, n_chunks, units), dim3(256), 0, stream, n_q_heads,
                       n_kv_heads, seq_len, chunk, n_chunks, qq, coeffs, w.gbuf, w.hc, w.rc,
                       want_coef ? w.dcp : nullptr);
    if ((st = check_launch("k_bwd_rbuild")) != OAL_OK) return st;
  }
  {
    ProfScope ps("k_bwd_rscan", stream);
    hipLaunchKernelGGL(k_bwd_rscan, dim3((unsigned)((STATE_FLOATS + 255) / 256), units), dim3(256), 0,
                       stream, n_chunks, w.rc);
    if ((st = check_launch("k_bwd_rscan")) != OAL_OK) return st;
  }
  {
    const int ks = key_split(chunk);
    if (ks * chunk != 256) return set_error(OAL_ERR_INVALID_ARG, "k_bwd_key: chunk %d", chunk);
    const size_t smem = sizeof(float) * ((size_t)(1 + ks) * chunk * (DH + 1) + TB * (DH + 1) +
                                         TB * WP + DH + DH * DH);
    const void* fn = ks == 4 ? reinterpret_cast<const void*>(&k_bwd_key<T, 4>)
                             : reinterpret_cast<const void*>(&k_bwd_key<T, 2>);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
      return set_error(OAL_ERR_HIP, "k_bwd_key: cannot reserve %zu bytes of LDS", smem);
    const int rep = n_q_heads / n_kv_heads;
    {
      ProfScope ps("k_bwd_key", stream);
      if (ks == 4)
        hipLaunchKernelGGL((k_bwd_key<T, 4>), dim3(n_chunks, units * rep), dim3(4 * chunk), smem,
                           stream, n_q_heads, n_kv_heads, seq_len, chunk, n_chunks, qq, kk, vv, coeffs,
                           w.gbuf, w.kpart);
      else
        hipLaunchKernelGGL((k_bwd_key<T, 2>), dim3(n_chunks, units * rep), dim3(2 * chunk), smem,
                           stream, n_q_heads, n_kv_heads, seq_len, chunk, n_chunks, qq, kk, vv, coeffs,
                           w.gbuf, w.kpart);
      if ((st = check_launch("k_bwd_key")) != OAL_OK) return st;
    }
    {
      const int per = (chunk / KS_TG) * KS_NFS;
      const dim3 grid((unsigned)(((size_t)units * n_chunks + 7) / 8 * 8 * (size_t)per));
      ProfScope ps("k_bwd_kstate", stream);
      hipLaunchKernelGGL(k_bwd_kstate<T>, grid, dim3(128), 0, stream, n_kv_heads, seq_len, chunk,
                         n_chunks, units, ks * rep, ks * rep + KS_NFS, kk, vv, w.rc, w.kpart);
      if ((st = check_launch("k_bwd_kstate")) != OAL_OK) return st;
    }
    ProfScope ps("k_bwd_ksum", stream);
    const size_t per_unit = (size_t)seq_len * (DH + DV);
    hipLaunchKernelGGL(k_bwd_ksum, dim3((unsigned)((per_unit + 255) / 256), units), dim3(256), 0,
                       stream, n_kv_heads, ks * rep + KS_NFS, ks, rep, pair_mfma ? 1 : 0, coeffs, seq_len,
                       n_chunks * chunk, w.kpart, dk, dv);
    if ((st = check_launch("k_bwd_ksum")) != OAL_OK) return st;
  }
  if (!want_coef) return OAL_OK;
  {
    const size_t smem = sizeof(float) * ((size_t)chunk * (chunk + 1) + 2 * chunk * (DH + 1));
    const void* fn = chunk == 64 ? reinterpret_cast<const void*>(&k_bwd_dc_intra<T, 64>)
                                 : reinterpret_cast<const void*>(&k_bwd_dc_intra<T, 128>);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
      return set_error(OAL_ERR_HIP, "k_bwd_dc_intra: cannot reserve %zu bytes of LDS", smem);
    ProfScope ps("k_bwd_dc_intra", stream);
    const dim3 grid(n_chunks, batch * n_q_heads);
    if (chunk == 64)
      hipLaunchKernelGGL((k_bwd_dc_intra<T, 64>), grid, dim3(256), smem, stream, n_q_heads, n_kv_heads,
                         seq_len, n_chunks, qq, kk, w.alpha, w.dcp);
    else
      hipLaunchKernelGGL((k_bwd_dc_intra<T, 128>), grid, dim3(256), smem, stream, n_q_heads, n_kv_heads,
                         seq_len, n_chunks, qq, kk, w.alpha, w.dcp);
    if ((st = check_launch("k_bwd_dc_intra")) != OAL_OK) return st;
  }
  ProfScope ps("k_bwd_dcoef", stream);
  hipLaunchKernelGGL(k_bwd_dcoef, dim3((DCAN + 255) / 256, n_q_heads), dim3(256), 0, stream, batch,
                     n_q_heads, n_chunks, w.dcp, da, db, dC);
  return check_launch("k_bwd_dcoef");
}

oal_status launch_backward(int batch, int n_q_heads, int n_kv_heads, int seq_len, int chunk,
                           oal_dtype in_dtype, const void* q, const void* k, const void* v,
                           const void* coeffs, const float* dy, float* dq, float* dk, float* dv,
                           float* da, float* db, float* dC, void* ws, hipStream_t stream) {
  if (in_dtype == OAL_F32)
    return backward_typed<float>(batch, n_q_heads, n_kv_heads, seq_len, chunk, in_dtype, q, k, v,
                                 coeffs, dy, dq, dk, dv, da, db, dC, ws, stream);
  return backward_typed<uint16_t>(batch, n_q_heads, n_kv_heads, seq_len, chunk, in_dtype, q, k, v,
                                  coeffs, dy, dq, dk, dv, da, db, dC, ws, stream);
}

oal_status launch_coeffs_backward(int n_q_heads, int g_max, const int32_t* n_groups,
                                  const int32_t* group_map, const float* L, const float* da,
                                  const float* db, const float* dC, float* dL, hipStream_t stream) {
  ProfScope ps("k_coeffs_bwd", stream);
  hipLaunchKernelGGL(k_coeffs_bwd, dim3(n_q_heads), dim3(64), 0, stream, g_max, n_groups, group_map,
                     L, da, db, dC, dL);
  return check_launch("k_coeffs_bwd");
}

}  // namespace oal
