// State management kernels: zero fill and the export to canonical packed order
// ([OAL] Eq. 5 states; packed-symmetric rows of App. D).
#include "oal_common.h"

namespace oal {

__global__ void __launch_bounds__(256) k_fill_zero(float4* __restrict__ p, size_t n4) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n4; i += stride) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// dst[unit][f][w] = src[unit][w][f] for f < DCAN.
__global__ void __launch_bounds__(256)
k_export(const float* __restrict__ src, float* __restrict__ dst) {
  const int unit = blockIdx.y;
  const int f0 = blockIdx.x * 32;
  __shared__ float tile[W][33];
  const float* s = src + (size_t)unit * STATE_FLOATS;
  for (int i = threadIdx.x; i < W * 32; i += blockDim.x) {
    int w = i / 32, ff = i % 32;
    int f = f0 + ff;
    tile[w][ff] = (f < DS) ? s[(size_t)w * DS + f] : 0.f;
  }
  __syncthreads();
  float* d = dst + (size_t)unit * DCAN * W;
  for (int i = threadIdx.x; i < W * 32; i += blockDim.x) {
    int ff = i / W, w = i % W;
    int f = f0 + ff;
    if (f < DCAN) d[(size_t)f * W + w] = tile[w][ff];
  }
}

oal_status launch_fill_zero(float* p, size_t n_floats, hipStream_t stream) {
  size_t n4 = n_floats / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return OAL_OK;
  ProfScope ps("k_fill_zero", stream);
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(p), n4);
  return check_launch("k_fill_zero");
}

oal_status launch_export(const oal_state* st, float* dst, hipStream_t stream) {
  int units = st->batch * st->n_kv_heads;
  dim3 grid((DCAN + 31) / 32, units);
  ProfScope ps("k_export", stream);
  hipLaunchKernelGGL(k_export, grid, dim3(256), 0, stream, st->data, dst);
  return check_launch("k_export");
}

}  // namespace oal
