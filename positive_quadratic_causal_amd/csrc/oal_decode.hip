// Single-token decode step: [OAL] Algorithm 1 loop body for one new token per
// (batch, KV head) unit:  u = [v; 1];  H += phi_k(k) u^T  (H0, H1_r, H2_rt of
// Eq. 5, packed-symmetric rows of App. D);  then for every query head of the
// grouped-query group  u~_h = phi_q^h(q_h)^T H  (Eq. 6) and y_h = u~_{1:64} / u~_65.
// The state is shared by the query heads of a group because it depends only on
// k and v ([OAL] App. D).
//
// MI355X design: the step is a pure stream over the fp32 state (557 KB per unit
// read and written once), so it is HBM-bound.  One workgroup per unit; each wave
// owns a set of state columns (column-major layout, 8.5 KB contiguous per
// column), reads them with 16-byte loads, updates them in registers, writes them
// back and accumulates the readout of all query heads of the group from the same
// registers.  The key- and query-side feature vectors are built once per
// workgroup in LDS and read as float4; per-column readout sums are reduced across
// the wave with lane shuffles.
#include "oal_common.h"

namespace oal {

template <typename T, typename O, int HG>
__global__ void __launch_bounds__(256)
k_decode(int n_q_heads, int n_kv_heads, int head0, int nh, int update,
         const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
         const void* __restrict__ coeffs, float* __restrict__ state, O* __restrict__ y) {
  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int kv = unit % n_kv_heads;
  const int rep = n_q_heads / n_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  __shared__ float4 s_phik4[DS / 4];
  __shared__ float4 s_phiq4[HG][DS / 4];
  __shared__ float s_k[DH];
  __shared__ float s_u[W];
  __shared__ float s_q[HG][DH];
  __shared__ float s_ut[HG][W];

  if (tid < DH) {
    s_k[tid] = Elem<T>::load(k, (size_t)unit * DH + tid);
    s_u[tid] = Elem<T>::load(v, (size_t)unit * DV + tid);
  }
  if (tid == 0) s_u[DV] = 1.0f;
  {
    // the q rows of the group's nh heads are one span (blockDim.x = 256); loads
    // unconditional (clamped), all issued before the first is awaited
    const T* qs = q + ((size_t)b * n_q_heads + kv * rep + head0) * DH;
    float x[HG * DH / 256 > 0 ? HG * DH / 256 : 1];
    constexpr int QE = HG * DH / 256 > 0 ? HG * DH / 256 : 1;
#pragma unroll
    for (int e = 0; e < QE; ++e) x[e] = Elem<T>::load(qs, min(tid + 256 * e, nh * DH - 1));
#pragma unroll
    for (int e = 0; e < QE; ++e) {
      const int i = tid + 256 * e;
      if (i < nh * DH) s_q[i / DH][i % DH] = x[e];
    }
  }
  __syncthreads();

  // feature decode by arithmetic (no table loads), a constant trip count
  constexpr int FIT = (DS + 255) / 256;   // features per thread
  float* phik = reinterpret_cast<float*>(s_phik4);
#pragma unroll
  for (int i = 0; i < FIT; ++i) {
    const int f = tid + 256 * i;
    if (f >= DS) break;
    float pk;
    if (f == 0) {
      pk = 1.0f;
    } else if (f <= DH) {
      pk = s_k[f - 1];
    } else if (f < DCAN) {
      int r, t;
      pair_decode(f - 1 - DH, r, t);
      pk = s_k[r] * s_k[t];
    } else {
      pk = 0.f;
    }
    phik[f] = pk;
  }
  // query features of every head: the coefficient of feature f (a, b'_r or the
  // packed c'_rt) comes from the head's record; all of a thread's coefficient
  // loads are issued before the first is used
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    if (hh >= nh) break;
    const float* rec = coef_rec(coeffs, kv * rep + head0 + hh);
    float cf[FIT];
#pragma unroll
    for (int i = 0; i < FIT; ++i) {
      const int f = tid + 256 * i;
      // record offset of feature f's coefficient: A, BP + r, CP + pair (f < DCAN)
      const int off = f == 0 ? OAL_COEF_A : f <= DH ? OAL_COEF_BP + f - 1 : OAL_COEF_CP + min(f, DCAN - 1) - 1 - DH;
      cf[i] = rec[off];
    }
    float* phiq = reinterpret_cast<float*>(s_phiq4[hh]);
#pragma unroll
    for (int i = 0; i < FIT; ++i) {
      const int f = tid + 256 * i;
      if (f >= DS) break;
      float pq;
      if (f == 0) {
        pq = cf[i];
      } else if (f <= DH) {
        pq = cf[i] * s_q[hh][f - 1];
      } else if (f < DCAN) {
        int r, t;
        pair_decode(f - 1 - DH, r, t);
        pq = cf[i] * s_q[hh][r] * s_q[hh][t];
      } else {
        pq = 0.f;
      }
      phiq[f] = pq;
    }
  }
  __syncthreads();

  constexpr int N4 = DS / 4;               // 544 float4 per column
  constexpr int IT = (N4 + 63) / 64;       // 9 iterations, the last one half full
  float4* st4 = reinterpret_cast<float4*>(state + (size_t)unit * STATE_FLOATS);
  // columns col, col + 4, ..: the next column's loads are issued before the
  // current one is processed (two columns in flight per wave)
  float4 hn[IT];
  auto load_col = [&](int c) {   // unconditional (clamped): a load inside a branch
    const float4* src = st4 + (size_t)c * N4;   // would be awaited on the spot
#pragma unroll
    for (int it = 0; it < IT; ++it) hn[it] = src[min(lane + 64 * it, N4 - 1)];
  };
  if (wave < W) load_col(wave);
  for (int col = wave; col < W; col += 4) {
    float4* hc = st4 + (size_t)col * N4;
    const float uc = s_u[col];
    float4 hv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) hv[it] = hn[it];
    if (col + 4 < W) load_col(col + 4);
    float acc[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) acc[hh] = 0.f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      int i4 = lane + 64 * it;
      if (i4 < N4) {
        float4 x = hv[it];
        if (update) {
          float4 pk = s_phik4[i4];
          x.x = fmaf(uc, pk.x, x.x);
          x.y = fmaf(uc, pk.y, x.y);
          x.z = fmaf(uc, pk.z, x.z);
          x.w = fmaf(uc, pk.w, x.w);
          hc[i4] = x;
        }
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float4 pq = s_phiq4[hh][i4];
          acc[hh] = fmaf(pq.x, x.x, acc[hh]);
          acc[hh] = fmaf(pq.y, x.y, acc[hh]);
          acc[hh] = fmaf(pq.z, x.z, acc[hh]);
          acc[hh] = fmaf(pq.w, x.w, acc[hh]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      float s = acc[hh];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      if (lane == 0) s_ut[hh][col] = s;
    }
  }
  __syncthreads();
  for (int i = tid; i < nh * DV; i += blockDim.x) {
    int hh = i / DV, w = i % DV;
    int hq = kv * rep + head0 + hh;
    float val = s_ut[hh][w] / s_ut[hh][DV];
    Elem<O>::store(y, ((size_t)b * n_q_heads + hq) * DV + w, val);
  }
}

template <typename T, typename O>
static oal_status decode_typed(int batch, int n_q_heads, int n_kv_heads, const void* q,
                               const void* k, const void* v, const void* coeffs,
                               float* state, void* y, hipStream_t stream) {
  const int rep = n_q_heads / n_kv_heads;
  const int units = batch * n_kv_heads;
  // Heads are handled 8 at a time; the first pass also updates the state.
  for (int head0 = 0; head0 < rep; head0 += 8) {
    int nh = rep - head0 < 8 ? rep - head0 : 8;
    int update = head0 == 0;
    const T* qq = reinterpret_cast<const T*>(q);
    const T* kk = reinterpret_cast<const T*>(k);
    const T* vv = reinterpret_cast<const T*>(v);
    O* yy = reinterpret_cast<O*>(y);
    ProfScope ps("k_decode", stream);
    if (nh <= 1)
      hipLaunchKernelGGL((k_decode<T, O, 1>), dim3(units), dim3(256), 0, stream, n_q_heads,
                         n_kv_heads, head0, nh, update, qq, kk, vv, coeffs, state, yy);
    else if (nh <= 2)
      hipLaunchKernelGGL((k_decode<T, O, 2>), dim3(units), dim3(256), 0, stream, n_q_heads,
                         n_kv_heads, head0, nh, update, qq, kk, vv, coeffs, state, yy);
    else if (nh <= 4)
      hipLaunchKernelGGL((k_decode<T, O, 4>), dim3(units), dim3(256), 0, stream, n_q_heads,
                         n_kv_heads, head0, nh, update, qq, kk, vv, coeffs, state, yy);
    else
      hipLaunchKernelGGL((k_decode<T, O, 8>), dim3(units), dim3(256), 0, stream, n_q_heads,
                         n_kv_heads, head0, nh, update, qq, kk, vv, coeffs, state, yy);
    oal_status st = check_launch("k_decode");
    if (st != OAL_OK) return st;
  }
  return OAL_OK;
}

oal_status launch_decode(int batch, int n_q_heads, int n_kv_heads, oal_dtype in_dtype,
                         const void* q, const void* k, const void* v, const void* coeffs,
                         float* state, void* y, oal_dtype out_dtype, hipStream_t stream) {
  if (in_dtype == OAL_F32) {
    if (out_dtype == OAL_F32)
      return decode_typed<float, float>(batch, n_q_heads, n_kv_heads, q, k, v, coeffs, state, y, stream);
    return decode_typed<float, uint16_t>(batch, n_q_heads, n_kv_heads, q, k, v, coeffs, state, y, stream);
  }
  if (out_dtype == OAL_F32)
    return decode_typed<uint16_t, float>(batch, n_q_heads, n_kv_heads, q, k, v, coeffs, state, y, stream);
  return decode_typed<uint16_t, uint16_t>(batch, n_q_heads, n_kv_heads, q, k, v, coeffs, state, y, stream);
}

}  // namespace oal
