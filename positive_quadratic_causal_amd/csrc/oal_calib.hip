// Coefficient calibration by output matching, [OAL] App. B (Eq. 20): per query
// head, fit the lower-triangular L so that the causal OAL output matches softmax
// attention on sampled query positions, with Adam (Kingma and Ba, Algorithm 1)
// under gradient-norm clipping.
//
// One update's gradient needs only the sampled rows, so they are evaluated
// directly in the grouped form of [OAL] Eq. 7 (no chunked prefill): for row i of
// head h, with s_bar_ij = [1, s_1, .., s_G] (s_g = sum_{r in g} q_ir k_jr / sqrt d_h),
//   kappa_ij = eps + s_bar^T M s_bar,  M = L L^T,
//   y_i = sum_{j<=i} kappa_ij v_j / den_i,  den_i = sum_{j<=i} kappa_ij,
//   loss_i = ||y_i - y_ref_i||^2 / (2 n_pos),  dy_i = (y_i - y_ref_i) / n_pos,
//   g_i = [dy_i / den_i ; -(dy_i . y_i) / den_i],  alpha_ij = g_i . [v_j; 1],
//   dM += sum_j alpha_ij s_bar_ij s_bar_ij^T,
// and per head dL = (dM + dM^T) L on the parameters (lower triangle of the
// leading (G+1) block).
//
//   k_calib_rows    block (sampled row, head): two passes over the row's keys
//   k_calib_reduce  per head: rows summed in order, loss, dL
//   k_adam          per head: clip to the norm, one Adam step
//   k_output_mse    per head: mean squared error of a whole output (validation)
#include "oal_common.h"

namespace oal {

namespace {
constexpr int CT = 256;   // threads of the row kernel

// tree reduction of n floats per thread over the block: red [CT][n] in LDS; the
// result is left in red[0][:]
__device__ __forceinline__ void block_sum_rows(float* red, int n, int tid) {
  for (int stride = CT / 2; stride > 0; stride >>= 1) {
    __syncthreads();
    if (tid < stride)
      for (int c = 0; c < n; ++c) red[tid * n + c] += red[(tid + stride) * n + c];
  }
  __syncthreads();
}
}  // namespace

template <typename T>
__global__ void __launch_bounds__(CT)
k_calib_rows(int n_q_heads, int n_kv_heads, int seq_len, const T* __restrict__ q,
             const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ y_ref,
             const int32_t* __restrict__ positions, int n_pos, int g_max,
             const int32_t* __restrict__ n_groups, const int32_t* __restrict__ group_map,
             const float* __restrict__ Lin, float eps, float* __restrict__ dm_part,
             float* __restrict__ loss_part) {
  const int pi = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int kv = h / (n_q_heads / n_kv_heads);
  const int ld = g_max + 1;
  __shared__ float s_qm[LDIM][DH];     // q_r / sqrt(d_h) on the dims of group gamma, else 0
  __shared__ float s_M[LDIM][LDIM];
  __shared__ float s_L[LDIM][LDIM];
  __shared__ float s_red[CT * LDIM * LDIM];
  __shared__ float s_kap[CT];
  __shared__ float s_g[DV + 1];
  __shared__ int s_G;
  const int i = positions[pi];
  float* dmo = dm_part + ((size_t)pi * n_q_heads + h) * LDIM * LDIM;
  if (i < 0 || i >= seq_len) {   // a position outside the sequence contributes nothing
    for (int c = tid; c < LDIM * LDIM; c += CT) dmo[c] = 0.f;
    if (tid == 0) loss_part[(size_t)pi * n_q_heads + h] = 0.f;
    return;
  }
  if (tid == 0) {
    const int G = n_groups[h];
    s_G = G < 1 ? 1 : (G > g_max ? g_max : G);
  }
  __syncthreads();
  const int G = s_G;
  if (tid < LDIM * LDIM) {
    const int u = tid / LDIM, w = tid % LDIM;
    s_L[u][w] = (u <= G && w <= G && w <= u) ? Lin[(size_t)h * ld * ld + u * ld + w] : 0.f;
  }
  const size_t qrow = ((size_t)h * seq_len + i) * DH;
  for (int c = tid; c < LDIM * DH; c += CT) {
    const int gam = c / DH, r = c % DH;
    int gr = group_map[(size_t)h * DH + r];
    gr = gr < 1 ? 1 : (gr > G ? G : gr);
    s_qm[gam][r] = (gam >= 1 && gr == gam) ? Elem<T>::load(q, qrow + r) * 0.125f : 0.f;
  }
  __syncthreads();
  if (tid < LDIM * LDIM) {
    const int u = tid / LDIM, w = tid % LDIM;
    float m = 0.f;
#pragma unroll
    for (int p = 0; p < LDIM; ++p) m = fmaf(s_L[u][p], s_L[w][p], m);
    s_M[u][w] = m;
  }
  __syncthreads();

  const size_t kvrow0 = (size_t)kv * seq_len;
  // s_bar of key j: the key row streamed in blocks of 8 into the group sums (a
  // rolled block loop: unrolled, the 448 loop-invariant s_qm loads would be hoisted
  // out of the key loop into registers and spill)
  auto sbar = [&](int j, float (&s)[LDIM]) {
    const T* kp = k + (kvrow0 + j) * DH;
    s[0] = 1.f;
#pragma unroll
    for (int gam = 1; gam < LDIM; ++gam) s[gam] = 0.f;
#pragma unroll 1
    for (int r0 = 0; r0 < DH; r0 += 8) {
      float kb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kb[e] = Elem<T>::load(kp, r0 + e);
#pragma unroll
      for (int gam = 1; gam < LDIM; ++gam) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[gam] = fmaf(s_qm[gam][r0 + e], kb[e], s[gam]);
      }
    }
  };

  // ---- pass 1: numerator and denominator of row i.  Per block of CT keys, each
  //      thread puts one key's kappa in LDS; then thread (w, part) adds channel w
  //      of 64 of those keys (the 64 threads of a wave read one v row together).
  const int wch = tid & 63, part = tid >> 6;
  float den_acc = 0.f, num_acc = 0.f;
  for (int j0 = 0; j0 <= i; j0 += CT) {
    const int j = j0 + tid;
    float kap = 0.f;
    if (j <= i) {
      float s[LDIM];
      sbar(j, s);
      kap = eps;
#pragma unroll
      for (int u = 0; u < LDIM; ++u) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < LDIM; ++w) t = fmaf(s_M[u][w], s[w], t);
        kap = fmaf(s[u], t, kap);
      }
    }
    den_acc += kap;
    __syncthreads();
    s_kap[tid] = kap;
    __syncthreads();
    const int jb = j0 + part * 64;
    const int nk = min(64, i + 1 - jb);
    for (int jj = 0; jj < nk; ++jj)
      num_acc = fmaf(s_kap[part * 64 + jj], Elem<T>::load(v, (kvrow0 + jb + jj) * DV + wch), num_acc);
  }
  __syncthreads();
  s_red[tid] = num_acc;
  s_red[CT + tid] = den_acc;
  for (int stride = CT / 2; stride > 0; stride >>= 1) {
    __syncthreads();
    if (tid < stride) s_red[CT + tid] += s_red[CT + tid + stride];
  }
  __syncthreads();
  if (tid < 64) s_red[tid] = (s_red[tid] + s_red[64 + tid]) + (s_red[128 + tid] + s_red[192 + tid]);
  if (tid == 0) s_red[DV] = s_red[CT];   // the denominator after the 64 channels
  __syncthreads();
  if (tid < 64) {   // one wave: y_i, dy_i, g_i and the loss
    const float den = s_red[DV];
    const float inv = 1.0f / den;
    const float y = s_red[tid] * inv;
    const float diff = y - y_ref[qrow + tid];
    const float dy = diff / (float)n_pos;
    s_g[tid] = dy * inv;
    float sq = diff * diff, yd = dy * y;
    for (int off = 32; off > 0; off >>= 1) {
      sq += __shfl_xor(sq, off, 64);
      yd += __shfl_xor(yd, off, 64);
    }
    if (tid == 0) {
      s_g[DV] = -yd * inv;
      loss_part[(size_t)pi * n_q_heads + h] = sq / (2.0f * (float)n_pos);
    }
  }
  __syncthreads();

  // ---- pass 2: dM = sum_j alpha_ij s_bar s_bar^T
  float dm[LDIM][LDIM];
#pragma unroll
  for (int u = 0; u < LDIM; ++u)
#pragma unroll
    for (int w = 0; w < LDIM; ++w) dm[u][w] = 0.f;
  for (int j = tid; j <= i; j += CT) {
    float s[LDIM];
    sbar(j, s);
    const T* vp = v + (kvrow0 + j) * DV;
    float al = s_g[DV];
#pragma unroll
    for (int w = 0; w < DV; ++w) al = fmaf(s_g[w], Elem<T>::load(vp, w), al);
#pragma unroll
    for (int u = 0; u < LDIM; ++u)
#pragma unroll
      for (int w = 0; w < LDIM; ++w) dm[u][w] = fmaf(al * s[u], s[w], dm[u][w]);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < LDIM; ++u)
#pragma unroll
    for (int w = 0; w < LDIM; ++w) s_red[tid * LDIM * LDIM + u * LDIM + w] = dm[u][w];
  block_sum_rows(s_red, LDIM * LDIM, tid);
  for (int c = tid; c < LDIM * LDIM; c += CT) dmo[c] = s_red[c];
}

// Per head: sum the rows' dM (in row order) and losses; dL = (dM + dM^T) L on
// the parameter entries, zero elsewhere.
__global__ void __launch_bounds__(64)
k_calib_reduce(int n_q_heads, int n_pos, int g_max, const int32_t* __restrict__ n_groups,
               const float* __restrict__ Lin, const float* __restrict__ dm_part,
               const float* __restrict__ loss_part, float* __restrict__ dL, float* __restrict__ loss) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int ld = g_max + 1;
  __shared__ float s_dM[LDIM][LDIM];
  __shared__ float s_L[LDIM][LDIM];
  int G = n_groups[h];
  G = G < 1 ? 1 : (G > g_max ? g_max : G);
  if (tid < LDIM * LDIM) {
    const int u = tid / LDIM, w = tid % LDIM;
    float acc = 0.f;
    for (int p = 0; p < n_pos; ++p) acc += dm_part[((size_t)p * n_q_heads + h) * LDIM * LDIM + tid];
    s_dM[u][w] = acc;
    s_L[u][w] = (u <= G && w <= G && w <= u) ? Lin[(size_t)h * ld * ld + u * ld + w] : 0.f;
  }
  if (tid == 0) {
    float acc = 0.f;
    for (int p = 0; p < n_pos; ++p) acc += loss_part[(size_t)p * n_q_heads + h];
    loss[h] = acc;
  }
  __syncthreads();
  if (tid < ld * ld) {
    const int u = tid / ld, w = tid % ld;
    float x = 0.f;
    if (u <= G && w <= u)
      for (int p = 0; p <= G; ++p) x = fmaf(s_dM[u][p] + s_dM[p][u], s_L[p][w], x);
    dL[(size_t)h * ld * ld + tid] = x;
  }
}

// Per head: clip the gradient to Euclidean norm <= clip over the parameter
// entries, then one Adam step (bias-corrected moments; t is the 1-based step).
__global__ void __launch_bounds__(64)
k_adam(int g_max, const int32_t* __restrict__ n_groups, float* __restrict__ L,
       const float* __restrict__ dL, float* __restrict__ m, float* __restrict__ v, int t, float lr,
       float beta1, float beta2, float eps, float clip) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int ld = g_max + 1;
  int G = n_groups[h];
  G = G < 1 ? 1 : (G > g_max ? g_max : G);
  const int u = tid / ld, w = tid % ld;
  const bool param = tid < ld * ld && u <= G && w <= u;
  const size_t e = (size_t)h * ld * ld + tid;
  const float g = param ? dL[e] : 0.f;
  float sq = g * g;
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
  const float norm = sqrtf(sq);
  const float scale = norm > clip ? clip / norm : 1.0f;
  if (!param) return;
  const float gc = g * scale;
  const float mt = beta1 * m[e] + (1.0f - beta1) * gc;
  const float vt = beta2 * v[e] + (1.0f - beta2) * gc * gc;
  m[e] = mt;
  v[e] = vt;
  const float mhat = mt / (1.0f - powf(beta1, (float)t));
  const float vhat = vt / (1.0f - powf(beta2, (float)t));
  L[e] -= lr * mhat / (sqrtf(vhat) + eps);
}

// Per head: sum over batch, positions and channels of (y - y_ref)^2, divided by
// their count.  One 1024-thread block per head, float4 loads when d_v is a
// multiple of 4, a fixed-order tree at the end (deterministic).
constexpr int MSE_T = 1024;
__global__ void __launch_bounds__(MSE_T)
k_output_mse(int batch, int n_q_heads, int seq_len, int d_v, const float* __restrict__ y,
             const float* __restrict__ y_ref, float* __restrict__ mse) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ float s_red[MSE_T];
  const size_t per = (size_t)seq_len * d_v;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int b = 0; b < batch; ++b) {
    const float* a = y + ((size_t)b * n_q_heads + h) * per;
    const float* r = y_ref + ((size_t)b * n_q_heads + h) * per;
    if ((d_v & 3) == 0) {
      const float4* a4 = reinterpret_cast<const float4*>(a);
      const float4* r4 = reinterpret_cast<const float4*>(r);
      for (size_t e = tid; e < per / 4; e += MSE_T) {
        const float4 x = a4[e], z = r4[e];
        a0 = fmaf(x.x - z.x, x.x - z.x, a0);
        a1 = fmaf(x.y - z.y, x.y - z.y, a1);
        a2 = fmaf(x.z - z.z, x.z - z.z, a2);
        a3 = fmaf(x.w - z.w, x.w - z.w, a3);
      }
    } else {
      for (size_t e = tid; e < per; e += MSE_T) {
        const float d = a[e] - r[e];
        a0 = fmaf(d, d, a0);
      }
    }
  }
  s_red[tid] = (a0 + a1) + (a2 + a3);
  for (int stride = MSE_T / 2; stride > 0; stride >>= 1) {
    __syncthreads();
    if (tid < stride) s_red[tid] += s_red[tid + stride];
  }
  if (tid == 0) mse[h] = s_red[0] / (float)((size_t)batch * per);
}

// The learned global quadratic ([OAL] App. D, Eq. 23: eps + [1 s] M_g [1 s]^T,
// s = q . k / sqrt(d_h)) embedded into the grouped parameterisation: M_00 = m00,
// M_{0g} = M_{g0} = m01, M_{gh} = m11 for all groups 1..G, factored as L with
// row 0 = (l00, 0, ..) and rows 1..G = (l10, l11, 0, ..), l00 = sqrt(m00),
// l10 = m01 / l00, l11 = sqrt(max(m11 - l10^2, 0)); M_g = L_g L_g^T from the
// 2 x 2 lower triangle L_g of each head (the G = 1 calibration's L).
__global__ void __launch_bounds__(64)
k_embed_global(int g_max, int g_ld, const int32_t* __restrict__ n_groups,
               const float* __restrict__ Lg, float* __restrict__ L) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int ld = g_max + 1;
  int G = n_groups[h];
  G = G < 1 ? 1 : (G > g_max ? g_max : G);
  const float* lg = Lg + (size_t)h * g_ld * g_ld;
  const double a = lg[0], b = lg[g_ld], c = lg[g_ld + 1];   // lower triangle of L_g
  const double m00 = a * a, m01 = a * b, m11 = b * b + c * c;
  const double l00 = sqrt(m00);
  const double l10 = l00 > 0.0 ? m01 / l00 : 0.0;
  const double l11 = sqrt(fmax(m11 - l10 * l10, 0.0));
  if (tid < ld * ld) {
    const int u = tid / ld, w = tid % ld;
    float x = 0.f;
    if (u == 0 && w == 0) x = (float)l00;
    else if (u >= 1 && u <= G && w == 0) x = (float)l10;
    else if (u >= 1 && u <= G && w == 1) x = (float)l11;
    L[(size_t)h * ld * ld + tid] = x;
  }
}

oal_status launch_embed_global(int n_q_heads, int g_max, int g_ld, const int32_t* n_groups,
                               const float* Lg, float* L, hipStream_t stream) {
  ProfScope ps("k_embed_global", stream);
  hipLaunchKernelGGL(k_embed_global, dim3(n_q_heads), dim3(64), 0, stream, g_max, g_ld, n_groups, Lg, L);
  return check_launch("k_embed_global");
}

// ---------------------------------------------------------------------------

size_t calib_workspace(int n_q_heads, int n_pos) {
  const size_t a = (((size_t)n_pos * n_q_heads * LDIM * LDIM * sizeof(float)) + 255) & ~(size_t)255;
  const size_t b = (((size_t)n_pos * n_q_heads * sizeof(float)) + 255) & ~(size_t)255;
  return a + b;
}

oal_status launch_calib_grad(int n_q_heads, int n_kv_heads, int seq_len, oal_dtype in_dtype,
                             const void* q, const void* k, const void* v, const float* y_ref,
                             const int32_t* positions, int n_pos, int g_max,
                             const int32_t* n_groups, const int32_t* group_map, const float* L,
                             float eps, float* dL, float* loss, void* ws, hipStream_t stream) {
  float* dm_part = reinterpret_cast<float*>(ws);
  float* loss_part = reinterpret_cast<float*>(
      reinterpret_cast<uint8_t*>(ws) +
      ((((size_t)n_pos * n_q_heads * LDIM * LDIM * sizeof(float)) + 255) & ~(size_t)255));
  {
    ProfScope ps("k_calib_rows", stream);
    const dim3 grid(n_pos, n_q_heads);
    if (in_dtype == OAL_F32)
      hipLaunchKernelGGL(k_calib_rows<float>, grid, dim3(CT), 0, stream, n_q_heads, n_kv_heads, seq_len,
                         reinterpret_cast<const float*>(q), reinterpret_cast<const float*>(k),
                         reinterpret_cast<const float*>(v), y_ref, positions, n_pos, g_max, n_groups,
                         group_map, L, eps, dm_part, loss_part);
    else
      hipLaunchKernelGGL(k_calib_rows<uint16_t>, grid, dim3(CT), 0, stream, n_q_heads, n_kv_heads,
                         seq_len, reinterpret_cast<const uint16_t*>(q),
                         reinterpret_cast<const uint16_t*>(k), reinterpret_cast<const uint16_t*>(v),
                         y_ref, positions, n_pos, g_max, n_groups, group_map, L, eps, dm_part,
                         loss_part);
    oal_status st = check_launch("k_calib_rows");
    if (st != OAL_OK) return st;
  }
  ProfScope ps("k_calib_reduce", stream);
  hipLaunchKernelGGL(k_calib_reduce, dim3(n_q_heads), dim3(64), 0, stream, n_q_heads, n_pos, g_max,
                     n_groups, L, dm_part, loss_part, dL, loss);
  return check_launch("k_calib_reduce");
}

oal_status launch_adam(int n_q_heads, int g_max, const int32_t* n_groups, float* L, const float* dL,
                       float* m, float* v, int t, float lr, float beta1, float beta2, float eps,
                       float clip, hipStream_t stream) {
  ProfScope ps("k_adam", stream);
  hipLaunchKernelGGL(k_adam, dim3(n_q_heads), dim3(64), 0, stream, g_max, n_groups, L, dL, m, v, t, lr,
                     beta1, beta2, eps, clip);
  return check_launch("k_adam");
}

oal_status launch_output_mse(int batch, int n_q_heads, int seq_len, int d_v, const float* y,
                             const float* y_ref, float* mse, hipStream_t stream) {
  ProfScope ps("k_output_mse", stream);
  hipLaunchKernelGGL(k_output_mse, dim3(n_q_heads), dim3(MSE_T), 0, stream, batch, n_q_heads, seq_len,
                     d_v, y, y_ref, mse);
  return check_launch("k_output_mse");
}

}  // namespace oal
