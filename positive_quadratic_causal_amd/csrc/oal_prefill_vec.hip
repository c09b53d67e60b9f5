// Chunked causal prefill on the vector ALUs in fp32 (the fp32-input path).
//
// [OAL] Algorithm 1 evaluated chunk by chunk (the paper's backend uses 128-token
// blocks, App. E).  For chunk c with tokens T_c:
//   build   dH_c = sum_{j in T_c} phi_k(k_j) u_j^T              ([OAL] Eq. 5)
//   scan    H_{<c} = H_init + sum_{c' < c} dH_{c'}               (exclusive prefix)
//   readout u~_i = phi_q(q_i)^T H_{<c} + sum_{j in T_c, j <= i} kappa(q_i, k_j) u_j
//           y_i = u~_{i,1:64} / u~_{i,65}                         ([OAL] Eq. 6, 7)
// The intra-chunk kernel values of a grouped record use kappa = eps + sum_p t_p^2
// with t_p = L_0p + sum_r ell_p[r] q_r k_r, the expansion of ||L^T s_bar||^2 of
// Eq. 7.  A dimension-specific record (the general kernel of [OAL] Eq. 3) takes
// kappa = a + sum_r p_r (b'_r + sum_t S_rt p_t) with p_r = q_r k_r and S the
// symmetric C / d_h square of the record (equal to the packed-pair sum the state
// readout uses).
// Everything is fp32 with fp32 accumulation; this path favours simplicity over
// speed (the bf16 inputs go through the matrix-core path).
#include "oal_common.h"

namespace oal {

namespace {
constexpr int FB = 64;                 // feature rows per build block
constexpr int NFB = DS / FB;           // 34 build blocks per unit
constexpr int TB = 64;                 // tokens staged per step
constexpr int WPT = (W + 3) / 4;       // 17 columns per thread in the build
constexpr int WP = 68;                 // readout rows of H and u padded to 16 bytes

// acc[0..WP) += s * row[0..WP) for a 16-byte aligned LDS row: the whole row is
// read into registers first (17 wide reads in flight), then the multiply-adds
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
}  // namespace

// dH_c = sum_{j in chunk c} phi_k(k_j) u_j^T of one unit for feature rows
// [fb*64, fb*64+64), stored into the chunk's slot of out: on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: A 32 x 2, lane l holding A[l % 32][l / 32]; B 2 x 32,
// lane l holding B[l / 32][l % 32]; D 32 x 32, register i of lane l holding
// D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]).  M = features, N = channels, K =
// tokens two per product; wave = (feature half wave % 2, channel half wave / 2);
// A = psi_f(k) = k~[ia] k~[ib] (k~ = (k, 1)) of the lane's own feature from the
// staged key rows, B = the staged value rows; the all-ones channel as a
// multiply-add per product.  The tile goes through LDS so that each thread stores
// one feature's columns (consecutive threads, consecutive features).
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float fx16;
template <typename T>
__global__ void __launch_bounds__(256, 3)   // three blocks per CU (51 KB of LDS each)
k_build_mfma(int seq_len, int chunk, int n_chunks, const T* __restrict__ k, const T* __restrict__ v,
             float* __restrict__ out) {
  const int fb = blockIdx.x;
  const int c = blockIdx.y;
  const int unit = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int FT = wave & 1, WT = wave >> 1, kpar = lane >> 5;
  __shared__ float s_k[TB][DH + 1];                           // k~ rows, zero past the sequence
  __shared__ __attribute__((aligned(16))) float s_u[TB][WP];  // v rows
  __shared__ float s_R[FB][W + 1];                            // the block's dH tile
  const int fa = fb * FB + 32 * FT + (lane & 31);
  int ia = DH, ib = DH;
  float amask = 1.f;
  if (fa >= 1 && fa <= DH) {
    ia = fa - 1;
  } else if (fa > DH && fa < DCAN) {
    pair_decode(fa - 1 - DH, ia, ib);
  } else if (fa >= DCAN) {
    amask = 0.f;
  }
  fx16 D[2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < 16; ++i) D[x][i] = 0.f;
  float d64 = 0.f;   // all-ones channel of the lane's feature, its tokens of parity kpar
  const int t0 = c * chunk;
  const int t1 = min(seq_len, t0 + chunk);
  const size_t base = (size_t)unit * seq_len;
  for (int j0 = t0; j0 < t1; j0 += TB) {
    const int nj = min(TB, t1 - j0);
    __syncthreads();
    const T* ks = k + (base + j0) * DH;   // the tile's key and value rows: one span each
    const T* vs = v + (base + j0) * DV;
    stage_span<TB * DH>(tid, nj * DH, [&](int i) { return Elem<T>::load(ks, i); },
                        [&](int i, float x) { s_k[i / DH][i % DH] = x; });
    stage_span<TB * DV>(tid, nj * DV, [&](int i) { return Elem<T>::load(vs, i); },
                        [&](int i, float x) { s_u[i / DV][i % DV] = x; });
    if (tid < TB) s_k[tid][DH] = tid < nj ? 1.f : 0.f;
    __syncthreads();
#pragma unroll
    for (int jp = 0; jp < TB / 2; jp += 8) {
      float av[8], bv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int tok = 2 * (jp + jj) + kpar;
        av[jj] = amask * s_k[tok][ia] * s_k[tok][ib];
        bv[jj] = s_u[tok][32 * WT + (lane & 31)];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        D[jj & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[jj], bv[jj], D[jj & 1], 0, 0, 0);
        d64 += av[jj];   // u[64] = 1 on the sequence; av = 0 past it
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
    s_R[32 * FT + 8 * (i >> 2) + 4 * kpar + (i & 3)][32 * WT + (lane & 31)] = D[0][i] + D[1][i];
  d64 += __shfl_xor(d64, 32, 64);
  if (WT == 0 && kpar == 0) s_R[32 * FT + (lane & 31)][W - 1] = d64;
  __syncthreads();
  const int f = fb * FB + (tid & 63), wq = tid >> 6;
  float* o = out + ((size_t)unit * n_chunks + c) * STATE_FLOATS + f;
#pragma unroll
  for (int j = 0; j < 16; ++j) o[(size_t)(16 * wq + j) * DS] = s_R[tid & 63][16 * wq + j];
  if (wq == 3) o[(size_t)(W - 1) * DS] = s_R[tid & 63][W - 1];
}

// dH over tokens [t0, t1) of one unit for feature rows [fb*64, fb*64+64).
// mode 0: store into out (a per-chunk slot), mode 1: add into out (the state).
template <typename T>
__global__ void __launch_bounds__(256)
k_build_vec(int n_kv_heads, int seq_len, int chunk, int n_chunks, const T* __restrict__ k,
            const T* __restrict__ v, float* __restrict__ out, int mode) {
  const int fb = blockIdx.x;
  const int c = blockIdx.y;
  const int unit = blockIdx.z;
  const int tid = threadIdx.x;
  const int f = fb * FB + (tid & 63);
  const int wq = tid >> 6;
  __shared__ float s_k[TB][DH + 1];
  __shared__ __attribute__((aligned(16))) float s_u[TB][WP];   // [v; 1] rows, 16-byte aligned
  // columns of this thread: 16 wq .. 16 wq + 15 (four 16-byte reads of a u row),
  // and the all-ones channel W - 1 on wave 3
  auto col_of = [&](int j) { return j < 16 ? 16 * wq + j : (wq == 3 ? W - 1 : -1); };

  int r = 0, t = 0, kind;
  if (f == 0) kind = 0;
  else if (f <= DH) { kind = 1; r = f - 1; }
  else if (f < DCAN) { kind = 2; pair_decode(f - 1 - DH, r, t); }
  else kind = 3;

  float acc[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) acc[j] = 0.f;

  const int t0 = c * chunk;
  const int t1 = min(seq_len, t0 + chunk);
  const size_t base = (size_t)unit * seq_len;
  for (int j0 = t0; j0 < t1; j0 += TB) {
    const int nj = min(TB, t1 - j0);
    __syncthreads();
    // the tile's key and value rows are one span each (nj >= 1, 256 threads)
    const T* ks = k + (base + j0) * DH;
    const T* vs = v + (base + j0) * DV;
    stage_span<TB * DH>(tid, nj * DH, [&](int i) { return Elem<T>::load(ks, i); },
                        [&](int i, float x) { s_k[i / DH][i % DH] = x; });
    stage_span<TB * DV>(tid, nj * DV, [&](int i) { return Elem<T>::load(vs, i); },
                        [&](int i, float x) { s_u[i / DV][i % DV] = x; });
    if (tid < TB) s_u[tid][DV] = tid < nj ? 1.f : 0.f;
    __syncthreads();
    for (int jj = 0; jj < nj; ++jj) {
      float phi = kind == 0 ? 1.f : kind == 1 ? s_k[jj][r] : kind == 2 ? s_k[jj][r] * s_k[jj][t] : 0.f;
      const float4* ur = reinterpret_cast<const float4*>(&s_u[jj][16 * wq]);
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const float4 u4 = ur[j4];
        acc[4 * j4 + 0] = fmaf(phi, u4.x, acc[4 * j4 + 0]);
        acc[4 * j4 + 1] = fmaf(phi, u4.y, acc[4 * j4 + 1]);
        acc[4 * j4 + 2] = fmaf(phi, u4.z, acc[4 * j4 + 2]);
        acc[4 * j4 + 3] = fmaf(phi, u4.w, acc[4 * j4 + 3]);
      }
      if (wq == 3) acc[16] = fmaf(phi, s_u[jj][W - 1], acc[16]);
    }
  }
  float* o = out + (mode == 0 ? ((size_t)unit * n_chunks + c) * STATE_FLOATS
                              : (size_t)unit * STATE_FLOATS);
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = col_of(j);
    if (w >= 0) {
      float* p = o + (size_t)w * DS + f;
      if (mode == 0) *p = acc[j];
      else *p += acc[j];
    }
  }
}

// In-place exclusive prefix over chunk slots; optional initial/final state.
__global__ void __launch_bounds__(256)
k_scan_vec(int n_chunks, float* __restrict__ ws, float* __restrict__ state) {
  const int unit = blockIdx.y;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= STATE_FLOATS) return;
  float run = state ? state[(size_t)unit * STATE_FLOATS + e] : 0.f;
  float* p = ws + (size_t)unit * n_chunks * STATE_FLOATS + e;
  for (int c = 0; c < n_chunks; ++c) {
    float x = p[(size_t)c * STATE_FLOATS];
    p[(size_t)c * STATE_FLOATS] = run;
    run += x;
  }
  if (state) state[(size_t)unit * STATE_FLOATS + e] = run;
}

// Upper-triangle 4 x 4 blocks of a 64 x 64 symmetric matrix: block row br, block
// column bc >= br, row-major, at index sblk(br, bc) (compile-time once unrolled).
constexpr int NSB = (DH / 4) * (DH / 4 + 1) / 2;   // 136
__host__ __device__ constexpr int sblk(int br, int bc) { return (DH / 4) * br - br * (br - 1) / 2 + (bc - br); }

// One block per (chunk, query head, batch); thread i owns token i of the chunk.
// DIM: the record is dimension-specific (intra-chunk kappa from b', c');
// otherwise it is grouped, and a record with NG = 0 (dimension-specific) makes
// every output NaN instead of a silently wrong value.
// SPLIT = 2 or 4: that many threads per query (thread SPLIT i + h) split its
// features and its pairs round robin and add their parts of u~_i through LDS at
// the end.
template <typename T, typename O, bool DIM, int SPLIT>
__global__ void __launch_bounds__(SPLIT == 4 ? 512 : 256)
k_readout_vec(int n_q_heads, int n_kv_heads, int seq_len, int chunk, int n_chunks,
              const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
              const void* __restrict__ coeffs, const float* __restrict__ ws, O* __restrict__ y) {
  const int c = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int rep = n_q_heads / n_kv_heads;
  const int kv = hq / rep;
  const int unit = b * n_kv_heads + kv;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;                // SPLIT * chunk
  const int qx = tid / SPLIT, half = tid % SPLIT;
  const int t0 = c * chunk;
  const int clen = min(chunk, seq_len - t0);

  extern __shared__ __attribute__((aligned(16))) float smem[];
  // every array starts at a multiple of 4 floats (chunk and TB are multiples of 64)
  float* s_q = smem;                          // [chunk][DH + 1]
  float* s_H = s_q + chunk * (DH + 1);        // [32][WP]
  float* s_cf = s_H + 32 * WP;                // [32]
  float* s_k = s_cf + 32;                     // [TB][DH + 1]
  float* s_u = s_k + TB * (DH + 1);           // [TB][WP]
  float* s_ell = s_u + TB * WP;               // grouped: [LDIM][DH]; DIM: b' [DH]
  float* s_L0 = s_ell + LDIM * DH;            // grouped: [LDIM]
  float* s_st = s_ell + DH;                   // DIM: S = C / d_h, upper 4 x 4 blocks [NSB][16]

  const float* rec = coef_rec(coeffs, hq);
  const float a = rec[OAL_COEF_A];
  const float eps = rec[OAL_COEF_EPS];
  const int G = reinterpret_cast<const int32_t*>(rec)[OAL_COEF_NG];

  {
    const T* qs = q + (((size_t)b * n_q_heads + hq) * seq_len + t0) * DH;   // the chunk's q rows
    stage_span_rt<8>(tid, nthr, chunk * DH, clen * DH, [&](int i) { return Elem<T>::load(qs, i); },
                     [&](int i, float x) { s_q[(i / DH) * (DH + 1) + i % DH] = x; });
  }
  if constexpr (DIM) {
    for (int i = tid; i < DH; i += nthr) s_ell[i] = rec[OAL_COEF_BP + i];
    // block (br, bc), bc >= br, of S at sblk(br, bc): rows 4 br .., columns 4 bc ..,
    // the blocks above the diagonal doubled (they stand for their mirrors as well)
    for (int i = tid; i < NSB * 16; i += nthr) {
      int br = 0, base = 0;
      while (base + (16 - br) <= i / 16) base += 16 - br++;
      const int bc = br + (i / 16 - base), e = i % 16;
      s_st[i] = (bc > br ? 2.0f : 1.0f) * rec[OAL_COEF_CM + (4 * br + e / 4) * DH + 4 * bc + e % 4];
    }
  } else {
    for (int i = tid; i < LDIM * DH; i += nthr) s_ell[i] = rec[OAL_COEF_ELL + i];
    if (tid < LDIM) s_L0[tid] = rec[OAL_COEF_L + tid];   // row 0 of L: L_{0,p}
  }
  // the pad columns W..WP-1 of the H and u rows are never written again
  for (int i = tid; i < 32 * (WP - W); i += nthr) s_H[(i / (WP - W)) * WP + W + i % (WP - W)] = 0.f;
  for (int i = tid; i < TB * (WP - W); i += nthr) s_u[(i / (WP - W)) * WP + W + i % (WP - W)] = 0.f;
  __syncthreads();

  float acc[WP];
#pragma unroll
  for (int w = 0; w < WP; ++w) acc[w] = 0.f;
  const bool active = qx < clen;
  const float* qi = s_q + qx * (DH + 1);

  // inter-chunk part: phi_q(q_i)^T H_{<c}
  // (the next 32-feature block is fetched into registers while the current one is
  // used; nthr is at least 128 threads with SPLIT 2, 256 otherwise)
  const float* Hc = ws + ((size_t)unit * n_chunks + c) * STATE_FLOATS;
  constexpr int PB = (32 * W + (SPLIT == 2 ? 128 : 256) - 1) / (SPLIT == 2 ? 128 : 256);
  float pre[PB];
  auto fetch_block = [&](int f0) {   // unconditional (clamped): no wait on the loads in flight
#pragma unroll
    for (int e = 0; e < PB; ++e) {
      const int i = min(tid + e * nthr, 32 * W - 1);
      pre[e] = Hc[(size_t)(i / 32) * DS + f0 + i % 32];   // f0 + 31 < DS always
    }
  };
  fetch_block(0);
  for (int f0 = 0; f0 < DCAN; f0 += 32) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PB; ++e) {
      const int i = tid + e * nthr;
      if (i < 32 * W) s_H[(i % 32) * WP + i / 32] = pre[e];
    }
    if (f0 + 32 < DCAN) fetch_block(f0 + 32);
    if (tid < 32) {
      const int f = f0 + tid;
      const float x = rec[coef_index(min(f, DCAN - 1))];   // unconditional, then dropped past DCAN
      s_cf[tid] = f < DCAN ? x : 0.f;
    }
    __syncthreads();
    if (active) {
      const int nf = min(32, DCAN - f0);
      for (int ff = half; ff < nf; ff += SPLIT) {
        int f = f0 + ff;
        float phi;
        if (f == 0) phi = s_cf[ff];
        else if (f <= DH) phi = s_cf[ff] * qi[f - 1];
        else {
          int r, t;
          pair_decode(f - 1 - DH, r, t);
          phi = s_cf[ff] * qi[r] * qi[t];
        }
        axpy_row(acc, phi, s_H + ff * WP);
      }
    }
  }

  // intra-chunk part: direct kernel sum over j <= i inside the chunk
  const size_t kbase = ((size_t)unit * seq_len + t0);
  for (int j0 = 0; j0 < clen; j0 += TB) {
    const int nj = min(TB, clen - j0);
    __syncthreads();
    {
      const T* ks = k + (kbase + j0) * DH;   // the tile's key and value rows, one span each
      const T* vs = v + (kbase + j0) * DV;
      stage_span_rt<8>(tid, nthr, TB * DH, nj * DH, [&](int i) { return Elem<T>::load(ks, i); },
                       [&](int i, float x) { s_k[(i / DH) * (DH + 1) + i % DH] = x; });
      stage_span_rt<8>(tid, nthr, TB * DV, nj * DV, [&](int i) { return Elem<T>::load(vs, i); },
                       [&](int i, float x) { s_u[(i / DV) * WP + i % DV] = x; });
    }
    for (int jj = tid; jj < TB; jj += nthr) s_u[jj * WP + DV] = 1.f;
    __syncthreads();
    if (active) {
      const int jmax = min(nj, qx - j0 + 1);
      for (int jj = half; jj < jmax; jj += SPLIT) {
        const float* kj = s_k + jj * (DH + 1);
        float kap;
        if constexpr (DIM) {
          float pr[DH];
#pragma unroll
          for (int t = 0; t < DH; ++t) pr[t] = qi[t] * kj[t];
          // kappa = a + b' . p + p^T S p over the upper triangle of 4 x 4 blocks of
          // S (2240 multiply-adds instead of 4160), the blocks streamed from LDS as
          // broadcast reads; four row partials per block row
          float kl = a;
#pragma unroll
          for (int i = 0; i < DH / 4; ++i) {
            const float4 b4 = reinterpret_cast<const float4*>(s_ell)[i];
            kl = fmaf(b4.x, pr[4 * i], fmaf(b4.y, pr[4 * i + 1], fmaf(b4.z, pr[4 * i + 2], fmaf(b4.w, pr[4 * i + 3], kl))));
          }
          // the table pointer taken afresh per pair, so that the compiler does
          // not hoist the 544 block reads out of the pair loop into registers
          const float* stp = s_st;
          asm volatile("" : "+v"(stp));
          float kq = 0.f;
#pragma unroll
          for (int br = 0; br < DH / 4; ++br) {
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int bc = br; bc < DH / 4; ++bc) {
              const float4* blk = reinterpret_cast<const float4*>(stp + sblk(br, bc) * 16);
              const float4 b0 = blk[0], b1 = blk[1], b2 = blk[2], b3 = blk[3];
              const float p0 = pr[4 * bc], p1 = pr[4 * bc + 1], p2 = pr[4 * bc + 2], p3 = pr[4 * bc + 3];
              s0 = fmaf(b0.x, p0, fmaf(b0.y, p1, fmaf(b0.z, p2, fmaf(b0.w, p3, s0))));
              s1 = fmaf(b1.x, p0, fmaf(b1.y, p1, fmaf(b1.z, p2, fmaf(b1.w, p3, s1))));
              s2 = fmaf(b2.x, p0, fmaf(b2.y, p1, fmaf(b2.z, p2, fmaf(b2.w, p3, s2))));
              s3 = fmaf(b3.x, p0, fmaf(b3.y, p1, fmaf(b3.z, p2, fmaf(b3.w, p3, s3))));
            }
            kq = fmaf(s0, pr[4 * br], fmaf(s1, pr[4 * br + 1], fmaf(s2, pr[4 * br + 2], fmaf(s3, pr[4 * br + 3], kq))));
          }
          kap = kl + kq;
        } else {
          float tp[LDIM];
#pragma unroll
          for (int p = 0; p < LDIM; ++p) tp[p] = s_L0[p];
          for (int r = 0; r < DH; ++r) {
            float x = qi[r] * kj[r];
#pragma unroll
            for (int p = 0; p < LDIM; ++p) tp[p] = fmaf(s_ell[p * DH + r], x, tp[p]);
          }
          kap = eps;
#pragma unroll
          for (int p = 0; p < LDIM; ++p)
            if (p <= G) kap = fmaf(tp[p], tp[p], kap);
        }
        axpy_row(acc, kap, s_u + jj * WP);
      }
    }
  }

  if (SPLIT == 4) {   // parts 2, 3 onto 0, 1, then 1 onto 0, through the query rows and
                      // the H, k and u staging (chunk x (DH + 1) floats each; done with)
    float* xa = s_q + qx * (DH + 1);
    float* xb = s_H + qx * (DH + 1);
    __syncthreads();
    if (half >= 2) {
      float* xr = half == 2 ? xa : xb;
#pragma unroll
      for (int w = 0; w < W; ++w) xr[w] = acc[w];
    }
    __syncthreads();
    if (half < 2) {
      const float* xr = half == 0 ? xa : xb;
#pragma unroll
      for (int w = 0; w < W; ++w) acc[w] += xr[w];
    }
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int w = 0; w < W; ++w) xa[w] = acc[w];
    }
    __syncthreads();
    if (half != 0) return;
#pragma unroll
    for (int w = 0; w < W; ++w) acc[w] += xa[w];
  }
  if (SPLIT == 2) {   // half 1's share of u~_i through LDS (the query rows are done with)
    float* xrow = s_q + qx * (DH + 1);
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int w = 0; w < W; ++w) xrow[w] = acc[w];
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int w = 0; w < W; ++w) acc[w] += xrow[w];
  }
  if (active) {
    const float inv = (DIM || G >= 1) ? 1.0f / acc[DV] : __builtin_nanf("");
    O* yo = y + (((size_t)b * n_q_heads + hq) * seq_len + t0 + qx) * DV;
#pragma unroll
    for (int w = 0; w < DV; ++w) Elem<O>::store(yo, w, acc[w] * inv);
  }
}

template <typename T, typename O, bool DIM>
static oal_status prefill_vec_typed(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                                    const void* q, const void* k, const void* v,
                                    const void* coeffs, int chunk, float* state, void* y,
                                    float* ws, hipStream_t stream) {
  const int units = batch * n_kv_heads;
  const T* kk = reinterpret_cast<const T*>(k);
  const T* vv = reinterpret_cast<const T*>(v);
  if (y == nullptr) {
    // only advance the state: accumulate all tokens straight into it
    ProfScope ps("k_build_vec", stream);
    hipLaunchKernelGGL(k_build_vec<T>, dim3(NFB, 1, units), dim3(256), 0, stream, n_kv_heads,
                       seq_len, seq_len, 1, kk, vv, state, 1);
    return check_launch("k_build_vec(state)");
  }
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  oal_status st;
  {
    ProfScope ps("k_build_mfma", stream);
    hipLaunchKernelGGL(k_build_mfma<T>, dim3(NFB, n_chunks, units), dim3(256), 0, stream,
                       seq_len, chunk, n_chunks, kk, vv, ws);
    st = check_launch("k_build_mfma");
  }
  if (st != OAL_OK) return st;
  {
    ProfScope ps("k_scan_vec", stream);
    hipLaunchKernelGGL(k_scan_vec, dim3((unsigned)((STATE_FLOATS + 255) / 256), units), dim3(256),
                       0, stream, n_chunks, ws, state);
    st = check_launch("k_scan_vec");
  }
  if (st != OAL_OK) return st;
  size_t smem = sizeof(float) * ((size_t)chunk * (DH + 1) + 32 * WP + 32 + TB * (DH + 1) + TB * WP +
                                 (DIM ? DH + NSB * 16 : LDIM * DH + LDIM));
  // threads per query: 4 for dimension-specific records (their per-pair work is
  // the larger) and 2 for grouped ones up to chunk 128, 1 at chunk 256
  constexpr int SP = DIM ? 4 : 2;
  const bool split = chunk <= 128;
  if (chunk != 64 && chunk != 128 && chunk != 256)   // the state staging's thread counts
    return set_error(OAL_ERR_INVALID_ARG, "k_readout_vec: chunk %d", chunk);
  const void* fn = split ? reinterpret_cast<const void*>(&k_readout_vec<T, O, DIM, SP>)
                         : reinterpret_cast<const void*>(&k_readout_vec<T, O, DIM, 1>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return set_error(OAL_ERR_HIP, "k_readout_vec: cannot reserve %zu bytes of LDS", smem);
  ProfScope ps("k_readout_vec", stream);
  if (split)
    hipLaunchKernelGGL((k_readout_vec<T, O, DIM, SP>), dim3(n_chunks, n_q_heads, batch), dim3(SP * chunk),
                       smem, stream, n_q_heads, n_kv_heads, seq_len, chunk, n_chunks,
                       reinterpret_cast<const T*>(q), kk, vv, coeffs, ws, reinterpret_cast<O*>(y));
  else
    hipLaunchKernelGGL((k_readout_vec<T, O, DIM, 1>), dim3(n_chunks, n_q_heads, batch), dim3(chunk), smem,
                       stream, n_q_heads, n_kv_heads, seq_len, chunk, n_chunks,
                       reinterpret_cast<const T*>(q), kk, vv, coeffs, ws, reinterpret_cast<O*>(y));
  return check_launch("k_readout_vec");
}

oal_status launch_build_vec_chunks(int batch, int n_kv_heads, int seq_len, int chunk,
                                   const void* k, const void* v, float* dh, hipStream_t stream) {
  const int units = batch * n_kv_heads;
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  ProfScope ps("k_build_mfma", stream);
  hipLaunchKernelGGL(k_build_mfma<uint16_t>, dim3(NFB, n_chunks, units), dim3(256), 0, stream,
                     seq_len, chunk, n_chunks, reinterpret_cast<const uint16_t*>(k),
                     reinterpret_cast<const uint16_t*>(v), dh);
  return check_launch("k_build_mfma");
}

// Exclusive per-chunk prefix states H_{<c} of a sequence that starts empty:
// hc[unit][c] = sum of phi_k(k_j) u_j^T over the chunks before c (fp32, the
// state layout), for fp32 or bf16 k and v.
oal_status launch_prefix_vec(int batch, int n_kv_heads, int seq_len, int chunk, oal_dtype in_dtype,
                             const void* k, const void* v, float* hc, hipStream_t stream) {
  const int units = batch * n_kv_heads;
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  {
    ProfScope ps("k_build_mfma", stream);
    if (in_dtype == OAL_F32)
      hipLaunchKernelGGL(k_build_mfma<float>, dim3(NFB, n_chunks, units), dim3(256), 0, stream,
                         seq_len, chunk, n_chunks, reinterpret_cast<const float*>(k),
                         reinterpret_cast<const float*>(v), hc);
    else
      hipLaunchKernelGGL(k_build_mfma<uint16_t>, dim3(NFB, n_chunks, units), dim3(256), 0, stream,
                         seq_len, chunk, n_chunks, reinterpret_cast<const uint16_t*>(k),
                         reinterpret_cast<const uint16_t*>(v), hc);
    oal_status st = check_launch("k_build_mfma");
    if (st != OAL_OK) return st;
  }
  ProfScope ps("k_scan_vec", stream);
  hipLaunchKernelGGL(k_scan_vec, dim3((unsigned)((STATE_FLOATS + 255) / 256), units), dim3(256), 0,
                     stream, n_chunks, hc, nullptr);
  return check_launch("k_scan_vec");
}

size_t prefill_vec_workspace(int batch, int n_kv_heads, int seq_len, int chunk) {
  const size_t n_chunks = (size_t)((seq_len + chunk - 1) / chunk);
  return (size_t)batch * n_kv_heads * n_chunks * STATE_FLOATS * sizeof(float);
}

oal_status launch_prefill_vec(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                              oal_dtype in_dtype, const void* q, const void* k, const void* v,
                              const void* coeffs, int chunk, float* state, void* y,
                              oal_dtype out_dtype, void* ws, bool dim, hipStream_t stream) {
  float* w = reinterpret_cast<float*>(ws);
#define OAL_VEC_CALL(T, O, D) \
  prefill_vec_typed<T, O, D>(batch, n_q_heads, n_kv_heads, seq_len, q, k, v, coeffs, chunk, state, y, w, stream)
  const bool f32_in = in_dtype == OAL_F32, f32_out = out_dtype == OAL_F32;
  if (dim) {
    if (f32_in) return f32_out ? OAL_VEC_CALL(float, float, true) : OAL_VEC_CALL(float, uint16_t, true);
    return f32_out ? OAL_VEC_CALL(uint16_t, float, true) : OAL_VEC_CALL(uint16_t, uint16_t, true);
  }
  if (f32_in) return f32_out ? OAL_VEC_CALL(float, float, false) : OAL_VEC_CALL(float, uint16_t, false);
  return f32_out ? OAL_VEC_CALL(uint16_t, float, false) : OAL_VEC_CALL(uint16_t, uint16_t, false);
#undef OAL_VEC_CALL
}

}  // namespace oal
