// Chunked causal prefill for bf16 inputs on the gfx950 matrix cores.
//
// [OAL] Algorithm 1 evaluated by chunks of C tokens (the paper's backend uses
// 128-token blocks with bf16 tensor-core contractions and fp32 coefficients,
// [OAL] App. E):
//   u~_i = phi_q(q_i)^T H_{<c}  +  sum_{j in chunk, j <= i} kappa(q_i, k_j) u_j
//   y_i  = u~_{i,1:64} / u~_{i,65}
// The inter-chunk term reads the exclusive prefix state H_{<c} of the chunk (a
// bf16 copy in the tiled layout of oal_tile.h, plus fp32 side data for the
// denominator); the intra-chunk term evaluates kappa = eps + sum_p t_p^2,
// t_p = L_0p + sum_r ell_p[r] q_r k_r (the expansion of ||L^T s_bar||^2, Eq. 7)
// on the matrix cores and applies it to [V; 1].
#include "oal_tile.h"

namespace oal {

// ---------------------------------------------------------------------------
// Readout.  Workgroup = 4 waves = (256 / C) query heads of one KV group x C
// tokens of one chunk; wave = one head x 64 tokens.  In the u~^T orientation
// (rows = value channel w, columns = tokens) each wave owns a 64 x 64 tile of
// accumulators (2 x 2 MFMA tiles).
// ---------------------------------------------------------------------------
template <int CH>
struct ReadoutCfg {
  static constexpr int WPH = CH / 64;               // waves per head
  static constexpr int HPW = 4 / WPH;               // heads per workgroup
  static constexpr int QS = 72;                     // bf16 row stride of q / k tiles
  static constexpr int VS = CH + 8;                 // bf16 row stride of v^T
  static constexpr int SK = 8;                      // K-steps per state slab
  static constexpr int NSLAB = (tile::NKS + SK - 1) / SK;
  static constexpr int SLAB_BYTES = SK * tile::KS_BYTES;
  static constexpr int Q_BYTES = HPW * CH * QS * 2;
  static constexpr int K_BYTES = CH * QS * 2;
  static constexpr int V_BYTES = 64 * VS * 2;
  static constexpr int U_BYTES = (2 * SLAB_BYTES > K_BYTES + V_BYTES) ? 2 * SLAB_BYTES
                                                                      : K_BYTES + V_BYTES;
  static constexpr int MG_BYTES = HPW * 2 * LDIM * DH * 4;  // m M_{gamma,g(t)}/d_h, m = 1, 2
  static constexpr int LDS_BYTES = Q_BYTES + U_BYTES + MG_BYTES;
};

// Swizzled LDS offset of the 16-byte half-row (w, h) of a K-step inside a slab
// (avoids bank conflicts between rows w and w + 4).
__device__ __forceinline__ int slab_off(int kk, int w, int h) {
  return kk * tile::KS_BYTES + w * 32 + 16 * (h ^ ((w >> 2) & 1));
}

template <int CH, typename O>
__global__ void __launch_bounds__(256, 2)
k_readout_mfma(int n_q_heads, int n_kv_heads, int seq_len, int n_chunks, int n_hg, int n_uc,
               const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const float* __restrict__ coeffs,
               const uint8_t* __restrict__ ws_tile, O* __restrict__ y) {
  using Cfg = ReadoutCfg<CH>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __bf16* s_q = reinterpret_cast<__bf16*>(smem);
  uint8_t* s_u = smem + Cfg::Q_BYTES;
  __bf16* s_k = reinterpret_cast<__bf16*>(s_u);
  __bf16* s_vt = reinterpret_cast<__bf16*>(s_u + Cfg::K_BYTES);
  float* s_mg = reinterpret_cast<float*>(smem + Cfg::Q_BYTES + Cfg::U_BYTES);

  // ---- which (unit, chunk, head group): the head groups of one (unit, chunk)
  //      share an XCD (blockIdx % 8) so they hit the same L2 for the state.
  const int L = blockIdx.x;
  const int xcd = L & 7, slot = L >> 3;
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
  const int hl = hg * Cfg::HPW + hslot;
  const bool head_ok = hl < rep;
  const int hq = kv * rep + (head_ok ? hl : 0);

  // ---- stage q (all heads of the group), k and v^T of the chunk
  for (int i = tid; i < Cfg::HPW * CH * 8; i += 256) {
    const int hs = i / (CH * 8), rem = i % (CH * 8), tok = rem >> 3, part = rem & 7;
    const int hh = hg * Cfg::HPW + hs;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (hh < rep && tok < clen) {
      const size_t row = ((size_t)b * n_q_heads + kv * rep + hh) * seq_len + t0 + tok;
      val = reinterpret_cast<const uint4*>(q + row * DH)[part];
    }
    *reinterpret_cast<uint4*>(s_q + ((size_t)hs * CH + tok) * Cfg::QS + part * 8) = val;
  }
  const size_t kvrow0 = (size_t)unit * seq_len + t0;
  for (int i = tid; i < CH * 8; i += 256) {
    const int tok = i >> 3, part = i & 7;
    uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (tok < clen) {
      kk = reinterpret_cast<const uint4*>(k + (kvrow0 + tok) * DH)[part];
      vv = reinterpret_cast<const uint4*>(v + (kvrow0 + tok) * DV)[part];
    }
    *reinterpret_cast<uint4*>(s_k + (size_t)tok * Cfg::QS + part * 8) = kk;
    const uint16_t* pv = reinterpret_cast<const uint16_t*>(&vv);
    uint16_t* vt = reinterpret_cast<uint16_t*>(s_vt);
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(size_t)(part * 8 + e) * Cfg::VS + tok] = pv[e];
  }
  for (int i = tid; i < Cfg::HPW * LDIM * DH; i += 256) {
    const int hs = i / (LDIM * DH), e = i % (LDIM * DH);
    const int hh = hg * Cfg::HPW + hs;
    const float x = hh < rep ? coef_rec(coeffs, kv * rep + hh)[OAL_COEF_MG + e] : 0.f;
    s_mg[(hs * 2 + 0) * LDIM * DH + e] = x;          // multiplicity 1 (diagonal block)
    s_mg[(hs * 2 + 1) * LDIM * DH + e] = 2.0f * x;   // multiplicity 2
  }
  __syncthreads();

  const float* rec = coef_rec(coeffs, hq);
  const int G = reinterpret_cast<const int32_t*>(rec)[OAL_COEF_NG];
  const float* ts_side = reinterpret_cast<const float*>(
      ws_tile + ((size_t)unit * n_chunks + chunk) * tile::BYTES + tile::TILE_BYTES);
  const int tok0 = sub * 64;                 // first token of this wave in the chunk
  const __bf16* qw = s_q + (size_t)hslot * CH * Cfg::QS;

  // q fragment (B operand, columns = tokens, K = head dims): exact bf16 inputs
  auto qfrag = [&](int nt, int ks) {
    return *reinterpret_cast<const bf16x8*>(qw + (size_t)(tok0 + 32 * nt + col) * Cfg::QS +
                                            16 * ks + 8 * half);
  };

  float den[2] = {0.f, 0.f};   // this lane's partial denominators of tokens (col, nt)

  // ================= inter-chunk denominator ===============================
  // den = a z0 + sum_r b'_r q_r z1_r + q^T (C / d_h o Z) q: the all-ones channel
  // of the readout; the quadratic part as T = (C/d_h o Z) q^T on the matrix cores,
  // one 32-row block of T at a time.
  if (head_ok) {
    const float* cm = rec + OAL_COEF_CM;
    const float* Zs = ts_side + tile::SIDE_Z;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 T[2] = {splat16(0.f), splat16(0.f)};
      const int n = 32 * mt + col;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = 16 * ks + 8 * half + j;
          x[j] = cm[n * DH + t] * Zs[n * DH + t];
        }
        const bf16x8 az = pack8(x);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) T[nt] = mfma32(az, qfrag(nt, ks), T[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const __bf16* qrow = qw + (size_t)(tok0 + 32 * nt + col) * Cfg::QS;
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) d = fmaf(bf(qrow[32 * mt + acc_row(i, half)]), T[nt][i], d);
        den[nt] += d;
      }
    }
    const float a = rec[OAL_COEF_A];
    const float* bp = rec + OAL_COEF_BP;
    const float* z1 = ts_side + tile::SIDE_Z1;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const __bf16* qrow = qw + (size_t)(tok0 + 32 * nt + col) * Cfg::QS;
      float d = half == 0 ? a * ts_side[tile::SIDE_Z0] : 0.f;
#pragma unroll 8
      for (int r = 32 * half; r < 32 * half + 32; ++r) d = fmaf(bp[r] * bf(qrow[r]), z1[r], d);
      den[nt] += d;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = splat16(0.f);

  // ================= intra-chunk part ======================================
  // kappa^T[key][tok] = eps + sum_p (L_0p + sum_r ell_p[r] k_r q_r)^2 on the matrix
  // cores (A = k o ell_p, B = q^T, the accumulator seeded with L_0p), causal mask,
  // then u~^T += [V; 1]^T kappa^T (values on the matrix cores, the ones channel as
  // column sums into the denominator).  One 32-key tile at a time.
  if (head_ok) {
    const float eps = rec[OAL_COEF_EPS];
    const int n_kt = 2 * (sub + 1);          // key tiles covering keys <= last token
    for (int kt = 0; kt < n_kt; ++kt) {
      f32x16 kap[2] = {splat16(eps), splat16(eps)};
      const __bf16* krow = s_k + (size_t)(32 * kt + col) * Cfg::QS;
      for (int p = 0; p <= G; ++p) {
        const float l0p = rec[OAL_COEF_L + p];          // L_{0,p}
        const float* ell = rec + OAL_COEF_ELL + p * DH;
        bf16x8 ak[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * ks + 8 * half);
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = bf(kf[j]) * ell[16 * ks + 8 * half + j];
          ak[ks] = pack8(x);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          f32x16 sacc = splat16(l0p);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) sacc = mfma32(ak[ks], qfrag(nt, ks), sacc);
#pragma unroll
          for (int i = 0; i < 16; ++i) kap[nt][i] = fmaf(sacc[i], sacc[i], kap[nt][i]);
        }
      }
      // causal mask, denominators, and P [V; 1]
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int tok = tok0 + 32 * nt + col;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kt + acc_row(i, half);
          const float x = key <= tok ? kap[nt][i] : 0.f;
          kap[nt][i] = x;
          den[nt] += x;
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = kap[nt][8 * s2 + j];
          const bf16x8 pb = pack8(x);
          const int key0 = 32 * kt + 16 * s2 + 4 * half;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const __bf16* vr = s_vt + (size_t)(32 * mt + col) * Cfg::VS;
            const uint2 lo = *reinterpret_cast<const uint2*>(vr + key0);
            const uint2 hi = *reinterpret_cast<const uint2*>(vr + key0 + 8);
            uint4 pk = make_uint4(lo.x, lo.y, hi.x, hi.y);
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(&pk);
            acc[mt][nt] = mfma32(av, pb, acc[mt][nt]);
          }
        }
      }
    }
  }

  // ================= inter-chunk numerator: main K loop ======================
  __syncthreads();   // the slab buffers reuse the k / v^T staging area
  const uint8_t* tsrc = ws_tile + ((size_t)unit * n_chunks + chunk) * tile::BYTES;
  constexpr int NST = Cfg::SLAB_BYTES / (256 * 16);   // 16-byte pieces per thread per slab
  uint4 stage[NST];
  auto load_slab = [&](int s) {
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int piece = tid + 256 * i;                // 16-byte piece within the slab
      const int ks = s * Cfg::SK + (piece >> 7);
      stage[i] = ks < tile::NKS ? reinterpret_cast<const uint4*>(tsrc)[(size_t)s * Cfg::SK * 128 + piece]
                                : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_slab = [&](int buf) {
    uint8_t* base = s_u + buf * Cfg::SLAB_BYTES;
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int piece = tid + 256 * i;
      const int kk = piece >> 7, w = (piece >> 1) & 63, h = piece & 1;
      *reinterpret_cast<uint4*>(base + slab_off(kk, w, h)) = stage[i];
    }
  };
  load_slab(0);
  store_slab(0);
  __syncthreads();

  const int32_t* gmap = reinterpret_cast<const int32_t*>(rec) + OAL_COEF_GMAP;   // g(r), uniform
  const float* mgw = s_mg + hslot * 2 * LDIM * DH;
  const __bf16* qrow0 = qw + (size_t)(tok0 + col) * Cfg::QS;        // token of N-tile 0
  const __bf16* qrow1 = qw + (size_t)(tok0 + 32 + col) * Cfg::QS;   // token of N-tile 1
  float qt0[8], qt1[8];   // q_t of this lane's 8 t's of the current t-block (c)
  float qh0[8], qh1[8];   // qhat[t] = m q_t M_{g(r), g(t)} / d_h for the current (g(r), m)
  int cur_c = -1, cur_key = -1;

  for (int s = 0; s < Cfg::NSLAB; ++s) {
    const int buf = s & 1;
    if (s + 1 < Cfg::NSLAB) load_slab(s + 1);
    if (head_ok) {
      const uint8_t* sb = s_u + buf * Cfg::SLAB_BYTES;
      // Two half-slabs of 4 K-steps.  A new t-block starts at K-step 4 + 8 c (c + 1),
      // i.e. always at a half-slab boundary, and the 4 r's of a half-slab are the
      // consecutive, 4-aligned values r0 .. r0 + 3.
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ks0 = s * Cfg::SK + 4 * hh;
        if (ks0 >= tile::NKS) break;
        if (ks0 < tile::NKS_LIN) {
          // linear rows (slab 0, first half): phi = b'_r q_r, r = 16 ks + 8 half + j
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ks = ks0 + i;
            float b8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) b8[j] = rec[OAL_COEF_BP + 16 * ks + 8 * half + j];
            const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(qrow0 + 16 * ks + 8 * half);
            const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(qrow1 + 16 * ks + 8 * half);
            float x0[8], x1[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              x0[j] = b8[j] * bf(q0[j]);
              x1[j] = b8[j] * bf(q1[j]);
            }
            const bf16x8 b0 = pack8(x0), b1 = pack8(x1);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
              const bf16x8 af = *reinterpret_cast<const bf16x8*>(sb + slab_off(4 * hh + i, 32 * mt + col, half));
              acc[mt][0] = mfma32(af, b0, acc[mt][0]);
              acc[mt][1] = mfma32(af, b1, acc[mt][1]);
            }
          }
          continue;
        }
        const int c = tile::ks_block(ks0);
        const int r0 = ks0 - tile::quad_base(c);
        if (c != cur_c) {
          cur_c = c;
          cur_key = -1;
          const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(qrow0 + 16 * c + 8 * half);
          const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(qrow1 + 16 * c + 8 * half);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            qt0[j] = bf(q0[j]);
            qt1[j] = bf(q1[j]);
          }
        }
        // q_r for r0 .. r0 + 3 of both tokens (one 8-byte read each)
        const uint2 qa = *reinterpret_cast<const uint2*>(qrow0 + r0);
        const uint2 qb = *reinterpret_cast<const uint2*>(qrow1 + r0);
        const float qr0[4] = {__uint_as_float(qa.x << 16), __uint_as_float(qa.x & 0xffff0000u),
                              __uint_as_float(qa.y << 16), __uint_as_float(qa.y & 0xffff0000u)};
        const float qr1[4] = {__uint_as_float(qb.x << 16), __uint_as_float(qb.x & 0xffff0000u),
                              __uint_as_float(qb.y << 16), __uint_as_float(qb.y & 0xffff0000u)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          const int gam = __builtin_amdgcn_readfirstlane(gmap[r]);
          const int key = 2 * gam + (r >= 16 * c ? 0 : 1);     // (group, multiplicity)
          if (key != cur_key) {
            cur_key = key;
            const float4* mrow = reinterpret_cast<const float4*>(
                mgw + ((key & 1) * LDIM + gam) * DH + 16 * c + 8 * half);
            const float4 ma = mrow[0], mb = mrow[1];
            const float m8[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              qh0[j] = qt0[j] * m8[j];
              qh1[j] = qt1[j] * m8[j];
            }
          }
          // quadratic rows of item (r, c): phi = q_r * qhat[t]
          float x0[8], x1[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x0[j] = qr0[i] * qh0[j];
            x1[j] = qr1[i] * qh1[j];
          }
          const bf16x8 b0 = pack8(x0), b1 = pack8(x1);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(sb + slab_off(4 * hh + i, 32 * mt + col, half));
            acc[mt][0] = mfma32(af, b0, acc[mt][0]);
            acc[mt][1] = mfma32(af, b1, acc[mt][1]);
          }
        }
      }
    }
    if (s + 1 < Cfg::NSLAB) store_slab(buf ^ 1);
    __syncthreads();
  }

  // ================= epilogue: + a H0, normalise, store ======================
  if (!head_ok) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) den[nt] += __shfl_xor(den[nt], 32, 64);
  const float a = rec[OAL_COEF_A];
  const float* h0 = ts_side + tile::SIDE_H0;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int tok = tok0 + 32 * nt + col;
    if (tok >= clen) continue;
    const float inv = 1.0f / den[nt];
    O* yr = y + (((size_t)b * n_q_heads + hq) * seq_len + t0 + tok) * DV;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int w0 = 32 * mt + 8 * g4 + 4 * half;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (acc[mt][nt][4 * g4 + e] + a * h0[w0 + e]) * inv;
#pragma unroll
        for (int e = 0; e < 4; ++e) Elem<O>::store(yr, w0 + e, o[e]);
      }
  }
}

// ---------------------------------------------------------------------------

size_t state_mfma_workspace(int batch, int n_kv_heads, int seq_len, int chunk, bool with_tiles);
oal_status launch_state_mfma(int batch, int n_kv_heads, int seq_len, int chunk, const void* k,
                             const void* v, float* state, uint8_t* ts, void* ws,
                             hipStream_t stream);

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
  const long long blocks = 8LL * n_hg * ((n_uc + 7) / 8);
  auto kern = &k_readout_mfma<CH, O>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS_BYTES) != hipSuccess)
    return set_error(OAL_ERR_HIP, "k_readout_mfma: cannot reserve %d bytes of LDS", Cfg::LDS_BYTES);
  ProfScope ps("k_readout_mfma", stream);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), Cfg::LDS_BYTES, stream, n_q_heads,
                     n_kv_heads, seq_len, n_chunks, n_hg, n_uc,
                     reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
                     reinterpret_cast<const uint16_t*>(v), reinterpret_cast<const float*>(coeffs), ts,
                     reinterpret_cast<O*>(y));
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
                               int chunk, float* state, void* y, oal_dtype out_dtype, void* ws,
                               hipStream_t stream) {
  const int units = batch * n_kv_heads;
  const int n_chunks = (seq_len + chunk - 1) / chunk;
  // workspace: the per-chunk prefix tiles (with output), then the builder's scratch
  if (y == nullptr)   // state only: no per-chunk prefixes are needed
    return launch_state_mfma(batch, n_kv_heads, seq_len, chunk, k, v, state, nullptr, ws, stream);
  uint8_t* ts = reinterpret_cast<uint8_t*>(ws);
  uint8_t* scratch = ts + (size_t)units * n_chunks * tile::BYTES;
  oal_status st = launch_state_mfma(batch, n_kv_heads, seq_len, chunk, k, v, state, ts, scratch,
                                    stream);
  if (st != OAL_OK) return st;
  if (out_dtype == OAL_F32)
    return readout_dispatch<float>(chunk, batch, n_q_heads, n_kv_heads, seq_len, n_chunks, q, k, v,
                                   coeffs, ts, y, stream);
  return readout_dispatch<uint16_t>(chunk, batch, n_q_heads, n_kv_heads, seq_len, n_chunks, q, k, v,
                                    coeffs, ts, y, stream);
}

}  // namespace oal
