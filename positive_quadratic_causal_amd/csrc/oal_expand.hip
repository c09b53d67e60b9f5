// Coefficient expansion: (L, g, eps) -> the dimension-wise coefficients of the
// grouped positive kernel, [OAL] §4.3 ("Positive group-aware kernel"):
//   M = L L^T,  a = eps + M_00,  b_r = 2 M_{0,g(r)},  C_rt = M_{g(r),g(t)}
// together with the derived tables the kernels read (scaled by 1/sqrt d_h and
// 1/d_h as in the readout of [OAL] Eq. 6, and the packed multiplicities of
// App. D).  EXPAND_SPLIT workgroups per query head, each forming the head's
// (tiny) L and M and writing a disjoint part of its record: rows 8 j .. 8 j + 7
// of the C square and of the packed pairs for workgroup j, the short fields and
// the padding words for workgroup 0, ell for 1 and the M_{gamma,g(t)} table for 2.
// The record layout is in oal.h.
#include "oal_common.h"

namespace oal {

constexpr int EXPAND_SPLIT = DH / 8;

__global__ void __launch_bounds__(256)
k_expand(int g_max, const int32_t* __restrict__ n_groups, const int32_t* __restrict__ group_map,
         const float* __restrict__ Lin, float eps, float* __restrict__ coeffs) {
  const int h = blockIdx.x, part = blockIdx.y;
  const int tid = threadIdx.x;
  const int ld = g_max + 1;
  __shared__ float sL[LDIM][LDIM];
  __shared__ float sM[LDIM][LDIM];
  __shared__ int sg[DH];
  float* rec = coeffs + (size_t)h * OAL_COEF_WORDS;

  // Every input load is issued before the first barrier; L is read only inside
  // the g_max + 1 square of the head.
  const int G_in = n_groups[h];
  float lval = 0.f;
  const int lu = tid / LDIM, lv = tid % LDIM;
  if (tid < LDIM * LDIM && lu <= g_max && lv <= g_max) lval = Lin[(size_t)h * ld * ld + lu * ld + lv];
  const int gr_in = tid < DH ? group_map[(size_t)h * DH + tid] : 1;
  const int G = G_in < 1 ? 1 : (G_in > g_max ? g_max : G_in);
  if (tid < LDIM * LDIM) sL[lu][lv] = (lu <= G && lv <= G && lv <= lu) ? lval : 0.f;
  if (tid < DH) sg[tid] = gr_in < 1 ? 1 : (gr_in > G ? G : gr_in);
  __syncthreads();
  if (tid < LDIM * LDIM) {
    double m = 0.0;
    for (int p = 0; p < LDIM; ++p) m += (double)sL[lu][p] * (double)sL[lv][p];
    sM[lu][lv] = (float)m;
  }
  __syncthreads();

  const float inv_sqrt_d = 0.125f;   // 1 / sqrt(64)
  const float inv_d = 1.0f / 64.0f;
  // C_rt / d_h of rows 8 part .. + 7 over the full square, and with the
  // multiplicity of the packed pair (r <= t) at pair_index(r, t)
  for (int i = tid; i < 8 * DH; i += blockDim.x) {
    const int r = 8 * part + i / DH, t = i % DH;
    const float c = sM[sg[r]][sg[t]] * inv_d;
    rec[OAL_COEF_CM + r * DH + t] = c;
    if (t >= r) rec[OAL_COEF_CP + pair_index(r, t)] = (r == t ? 1.0f : 2.0f) * c;
  }
  if (part == 0) {
    if (tid == 0) {
      rec[OAL_COEF_A] = eps + sM[0][0];
      rec[OAL_COEF_EPS] = eps;
      reinterpret_cast<int32_t*>(rec)[OAL_COEF_NG] = G;
    }
    if (tid < DH) {
      const int gr = sg[tid];
      rec[OAL_COEF_BP + tid] = 2.0f * sM[0][gr] * inv_sqrt_d;
      reinterpret_cast<int32_t*>(rec)[OAL_COEF_GMAP + tid] = gr;
    }
    if (tid < DH / 8) {
      uint32_t word = 0;
      for (int i = 0; i < 8; ++i) word |= (uint32_t)sg[8 * tid + i] << (4 * i);
      reinterpret_cast<uint32_t*>(rec)[OAL_COEF_GPACK + tid] = word;
    }
    if (tid < LDIM * LDIM) {
      rec[OAL_COEF_M + tid] = sM[lu][lv];
      rec[OAL_COEF_L + tid] = sL[lu][lv];
    }
    // the padding words between and after the fields
    auto zero = [&](int w0, int w1) {
      for (int i = w0 + tid; i < w1; i += blockDim.x) rec[i] = 0.f;
    };
    zero(OAL_COEF_NG + 1, OAL_COEF_BP);
    zero(OAL_COEF_M + LDIM * LDIM, OAL_COEF_L);
    zero(OAL_COEF_L + LDIM * LDIM, OAL_COEF_ELL);
    zero(OAL_COEF_GPACK + DH / 8, OAL_COEF_WORDS);
  } else if (part == 1) {
    for (int i = tid; i < LDIM * DH; i += blockDim.x) {
      const int p = i / DH, r = i % DH;
      rec[OAL_COEF_ELL + i] = sL[sg[r]][p] * inv_sqrt_d;
    }
  } else if (part == 2) {
    for (int i = tid; i < LDIM * DH; i += blockDim.x) {
      const int gam = i / DH, t = i % DH;
      rec[OAL_COEF_MG + i] = (gam <= G ? sM[gam][sg[t]] : 0.f) * inv_d;
    }
  }
}
static_assert(OAL_COEF_BP > OAL_COEF_NG && OAL_COEF_ELL == OAL_COEF_L + 64 &&
                  OAL_COEF_CM == OAL_COEF_ELL + LDIM * DH && OAL_COEF_CP == OAL_COEF_CM + DH * DH &&
                  OAL_COEF_MG == OAL_COEF_CP + DH * (DH + 1) / 2 &&
                  OAL_COEF_GPACK == OAL_COEF_MG + LDIM * DH && OAL_COEF_GMAP == OAL_COEF_BP + DH &&
                  OAL_COEF_M == OAL_COEF_GMAP + DH && OAL_COEF_L == OAL_COEF_M + 64,
              "the fields and padding words of the record tile it without gaps");

// Dimension-specific coefficients, the general kernel of [OAL] §4.1 (Eq. 3):
//   kappa_dim(q, k) = a + sum_r b_r x_r + sum_{r,t} C_rt x_r x_t,  x_r = q_r k_r / sqrt(d_h)
// with arbitrary a, b_r, C_rt (no group structure).  x^T C x depends only on the
// symmetric part of C, so the record holds S = (C + C^T) / 2: the full square in
// CM and the packed pairs, weighted 1 on the diagonal and 2 off it, in CP.  The
// group fields stay zero and NG = 0 marks the record as dimension-specific.
__global__ void __launch_bounds__(256)
k_dim_coeffs(const float* __restrict__ a, const float* __restrict__ b,
             const float* __restrict__ C, float* __restrict__ coeffs) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  float* rec = coeffs + (size_t)h * OAL_COEF_WORDS;
  const float* Ch = C + (size_t)h * DH * DH;
  for (int i = tid; i < OAL_COEF_WORDS; i += blockDim.x) rec[i] = 0.f;
  __syncthreads();
  const float inv_sqrt_d = 0.125f;   // 1 / sqrt(64)
  const float inv_d = 1.0f / 64.0f;
  if (tid == 0) rec[OAL_COEF_A] = a[h];   // NG and EPS stay 0
  if (tid < DH) rec[OAL_COEF_BP + tid] = b[(size_t)h * DH + tid] * inv_sqrt_d;
  for (int i = tid; i < DH * DH; i += blockDim.x) {
    const int r = i / DH, t = i % DH;
    const float sym = 0.5f * (Ch[r * DH + t] + Ch[t * DH + r]);
    rec[OAL_COEF_CM + i] = sym * inv_d;
    if (t >= r) rec[OAL_COEF_CP + pair_index(r, t)] = (r == t ? 1.0f : 2.0f) * sym * inv_d;
  }
}

oal_status launch_dim_coeffs(int n_q_heads, const float* a, const float* b, const float* C,
                             void* coeffs, hipStream_t stream) {
  ProfScope ps("k_dim_coeffs", stream);
  hipLaunchKernelGGL(k_dim_coeffs, dim3(n_q_heads), dim3(256), 0, stream, a, b, C,
                     reinterpret_cast<float*>(coeffs));
  return check_launch("k_dim_coeffs");
}

oal_status launch_expand(int n_q_heads, int g_max, const int32_t* n_groups,
                         const int32_t* group_map, const float* L, float eps, void* coeffs,
                         hipStream_t stream) {
  ProfScope ps("k_expand", stream);
  hipLaunchKernelGGL(k_expand, dim3(n_q_heads, EXPAND_SPLIT), dim3(256), 0, stream, g_max, n_groups,
                     group_map, L, eps, reinterpret_cast<float*>(coeffs));
  return check_launch("k_expand");
}

}  // namespace oal
