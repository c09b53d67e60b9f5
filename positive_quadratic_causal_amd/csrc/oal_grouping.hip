// Dimension grouping of [OAL]: contribution scores (§3.1, Eq. 2) and the
// bootstrap tail-cut grouping of App. B (Eq. 16-19).
//
// Eq. 2 averages |q_ir k_jr| / sqrt(d_h) over the causal pairs j <= i of a prompt;
// the pair sum factorises as sum_i |q_ir| sum_{j<=i} |k_jr|, so one thread per
// dimension walks the prompt once with a running sum of |k_jr| (double
// accumulation).  The grouping of a head then needs only its P x d_h scores:
//   pi      dimensions by increasing chi (stable: rank = #smaller + #equal before)
//   rho_k   chi_{pi_{k+1}} / max(chi_{pi_k}, eps) for the candidate cuts
//           k = max(1, d - ceil(alpha d)) .. d - 1                     (Eq. 16)
//   S_k     fraction of bootstrap replicates (prompt multisets given by the
//           caller) whose mean scores, in the fixed order pi, keep
//           min(upper side) >= tau max(max(lower side), eps)           (Eq. 17-18)
//   cuts    rho_k >= tau and S_k >= gamma; below g_min groups, unused candidates
//           by descending (S_k, rho_k), ties in candidate order
//   labels  group g = pi_{k_{g-1}+1} .. pi_{k_g}                         (Eq. 19)
// Decisions are taken in double precision.
#include "oal_common.h"

namespace oal {

namespace {
constexpr int GT = 1024;         // threads of the grouping kernel (16 waves)
constexpr int MAX_PROMPTS = 256; // per-prompt scores of one head staged in LDS
}  // namespace

// chi_prompt[p][h][r] for prompt p = tokens offsets[p] .. offsets[p+1]-1.
template <typename T>
__global__ void __launch_bounds__(64)
k_contrib(int n_q_heads, int n_kv_heads, int total, const T* __restrict__ q,
          const T* __restrict__ k, const int32_t* __restrict__ offsets,
          float* __restrict__ chi_prompt) {
  const int p = blockIdx.x;
  const int h = blockIdx.y;
  const int r = threadIdx.x;
  const int kv = h / (n_q_heads / n_kv_heads);
  const int s = min(max(offsets[p], 0), total);
  const int e = min(max(offsets[p + 1], s), total);
  const T* qh = q + (size_t)h * total * DH;
  const T* kh = k + (size_t)kv * total * DH;
  double cum = 0.0, acc = 0.0;
  for (int i = s; i < e; ++i) {
    cum += fabs((double)Elem<T>::load(kh, (size_t)i * DH + r));
    acc += fabs((double)Elem<T>::load(qh, (size_t)i * DH + r)) * cum;
  }
  const double n = (double)(e - s);
  const double pairs = n * (n + 1.0) / 2.0;
  chi_prompt[((size_t)p * n_q_heads + h) * DH + r] = pairs > 0.0 ? (float)(acc / (pairs * 8.0)) : 0.f;
}

// chi[h][r] = mean over the prompts (equal weights), summed in prompt order.
__global__ void __launch_bounds__(64)
k_contrib_mean(int n_q_heads, int n_prompts, const float* __restrict__ chi_prompt,
               float* __restrict__ chi) {
  const int h = blockIdx.x;
  const int r = threadIdx.x;
  double s = 0.0;
  for (int p = 0; p < n_prompts; ++p) s += chi_prompt[((size_t)p * n_q_heads + h) * DH + r];
  chi[(size_t)h * DH + r] = (float)(s / n_prompts);
}

// double-precision wave shuffles (two 32-bit halves)
__device__ __forceinline__ double shfl_up_d(double x, int d) {
  const int lo = __shfl_up(__double2loint(x), d, 64), hi = __shfl_up(__double2hiint(x), d, 64);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double shfl_down_d(double x, int d) {
  const int lo = __shfl_down(__double2loint(x), d, 64), hi = __shfl_down(__double2hiint(x), d, 64);
  return __hiloint2double(hi, lo);
}

// One block per head: order, gaps, bootstrap support, cuts and labels.  The
// bootstrap runs one replicate per wave at a time, lane u holding the u-th
// dimension of the fixed order pi: the replicate's score sums, a prefix maximum
// and a suffix minimum by wave scans, and lane k counts the replicates that keep
// cut k (no atomics; the per-wave counts are added in wave order).
__global__ void __launch_bounds__(GT)
k_group(int n_q_heads, int n_prompts, const float* __restrict__ chi_prompt, int n_boot,
        const int32_t* __restrict__ boot_idx, float alpha, float tau, float gamma, int g_min,
        float eps, int32_t* __restrict__ group_map, int32_t* __restrict__ n_groups,
        float* __restrict__ support_out, float* __restrict__ gap_out) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ float s_cp[MAX_PROMPTS][DH];   // this head's per-prompt scores, then in pi order
  __shared__ double s_chi[DH];
  __shared__ int s_pi[DH];
  __shared__ double s_rho[DH];
  __shared__ int s_wcnt[GT / 64][DH];
  __shared__ int s_cnt[DH];
  const int m = (int)ceil((double)alpha * DH);
  const int kmin = max(1, DH - m);           // candidates kmin .. DH-1
  for (int i = tid; i < n_prompts * DH; i += GT)
    s_cp[i / DH][i % DH] = chi_prompt[((size_t)(i / DH) * n_q_heads + h) * DH + i % DH];
  __syncthreads();
  if (tid < DH) {
    double s = 0.0;
    for (int p = 0; p < n_prompts; ++p) s += s_cp[p][tid];
    s_chi[tid] = s / n_prompts;
  }
  __syncthreads();
  if (tid < DH) {   // stable ascending rank
    const double c = s_chi[tid];
    int rank = 0;
    for (int r = 0; r < DH; ++r) rank += (s_chi[r] < c) || (s_chi[r] == c && r < tid);
    s_pi[rank] = tid;
  }
  __syncthreads();
  if (tid < DH)
    s_rho[tid] = tid >= kmin ? s_chi[s_pi[tid]] / fmax(s_chi[s_pi[tid - 1]], (double)eps) : 0.0;
  {   // permute every prompt's row into pi order (through registers, one pass)
    constexpr int PER = MAX_PROMPTS * DH / GT;
    float tmp[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * GT;
      tmp[e] = i < n_prompts * DH ? s_cp[i / DH][s_pi[i % DH]] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * GT;
      if (i < n_prompts * DH) s_cp[i / DH][i % DH] = tmp[e];
    }
  }
  __syncthreads();

  // cut k at lane k: lower side = lanes 0..k-1, upper side = lanes k..63; both
  // sums carry the factor 1 / n_prompts, which the ratio test does not need
  int cnt = 0;
  const double tau_d = tau, floor_d = (double)eps * n_prompts;
  for (int b = wave; b < n_boot; b += GT / 64) {
    const int32_t* idx = boot_idx + (size_t)b * n_prompts;
    double sum = 0.0;
    for (int t = 0; t < n_prompts; ++t) {
      const int p = min(max(idx[t], 0), n_prompts - 1);
      sum += s_cp[p][lane];
    }
    double pmax = sum, smin = sum;
    for (int d = 1; d < 64; d <<= 1) {
      const double up = shfl_up_d(pmax, d);
      const double dn = shfl_down_d(smin, d);
      if (lane >= d) pmax = fmax(pmax, up);
      if (lane + d < 64) smin = fmin(smin, dn);
    }
    const double lower = shfl_up_d(pmax, 1);   // max over lanes 0..lane-1
    if (lane >= kmin && smin >= tau_d * fmax(lower, floor_d)) ++cnt;
  }
  s_wcnt[wave][lane] = cnt;
  __syncthreads();
  if (tid < DH) {
    int c = 0;
    for (int wv = 0; wv < GT / 64; ++wv) c += s_wcnt[wv][tid];
    s_cnt[tid] = c;
  }
  __syncthreads();

  if (tid == 0) {
    bool chosen[DH];
    int n_cuts = 0;
    for (int kk = 0; kk < DH; ++kk) {
      const double sk = (double)s_cnt[kk] / n_boot;
      chosen[kk] = kk >= kmin && s_rho[kk] >= (double)tau && sk >= (double)gamma;
      n_cuts += chosen[kk];
    }
    while (n_cuts + 1 < g_min) {   // fallback: best unused (S_k, rho_k), first in order on ties
      int best = -1;
      for (int kk = kmin; kk < DH; ++kk) {
        if (chosen[kk]) continue;
        if (best < 0 || s_cnt[kk] > s_cnt[best] ||
            (s_cnt[kk] == s_cnt[best] && s_rho[kk] > s_rho[best]))
          best = kk;
      }
      if (best < 0) break;
      chosen[best] = true;
      ++n_cuts;
    }
    int g = 1;
    for (int t = 0; t < DH; ++t) {
      if (t > 0 && chosen[t]) ++g;   // a cut at k starts a new group at pi_{k+1} = s_pi[k]
      group_map[(size_t)h * DH + s_pi[t]] = g;
    }
    n_groups[h] = g;
  }
  if (tid < DH) {
    if (support_out) support_out[(size_t)h * DH + tid] = tid >= kmin ? (float)s_cnt[tid] / n_boot : 0.f;
    if (gap_out) gap_out[(size_t)h * DH + tid] = (float)s_rho[tid];
  }
}

// ---------------------------------------------------------------------------

oal_status launch_contrib(int n_q_heads, int n_kv_heads, int n_prompts, int total,
                          oal_dtype in_dtype, const void* q, const void* k, const int32_t* offsets,
                          float* chi_prompt, float* chi, hipStream_t stream) {
  {
    ProfScope ps("k_contrib", stream);
    const dim3 grid(n_prompts, n_q_heads);
    if (in_dtype == OAL_F32)
      hipLaunchKernelGGL(k_contrib<float>, grid, dim3(64), 0, stream, n_q_heads, n_kv_heads, total,
                         reinterpret_cast<const float*>(q), reinterpret_cast<const float*>(k), offsets,
                         chi_prompt);
    else
      hipLaunchKernelGGL(k_contrib<uint16_t>, grid, dim3(64), 0, stream, n_q_heads, n_kv_heads, total,
                         reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
                         offsets, chi_prompt);
    oal_status st = check_launch("k_contrib");
    if (st != OAL_OK || chi == nullptr) return st;
  }
  ProfScope ps("k_contrib_mean", stream);
  hipLaunchKernelGGL(k_contrib_mean, dim3(n_q_heads), dim3(64), 0, stream, n_q_heads, n_prompts,
                     chi_prompt, chi);
  return check_launch("k_contrib_mean");
}

oal_status launch_grouping(int n_q_heads, int n_prompts, const float* chi_prompt, int n_boot,
                           const int32_t* boot_idx, float alpha, float tau, float gamma, int g_min,
                           float eps, int32_t* group_map, int32_t* n_groups, float* support,
                           float* gap, hipStream_t stream) {
  ProfScope ps("k_group", stream);
  hipLaunchKernelGGL(k_group, dim3(n_q_heads), dim3(GT), 0, stream, n_q_heads, n_prompts, chi_prompt,
                     n_boot, boot_idx, alpha, tau, gamma, g_min, eps, group_map, n_groups, support, gap);
  return check_launch("k_group");
}

int grouping_max_prompts() { return MAX_PROMPTS; }

}  // namespace oal
