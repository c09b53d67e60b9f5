// Exact causal softmax attention on the gfx950 matrix cores: the reference that
// OAL approximates ([OAL] §3: weights exp(q_i . k_j / sqrt(d_h)) over j <= i,
// normalised per row), for the frozen-attention fidelity metrics of [OAL] App. C.
//
// One workgroup per (unit, 128-query block, pair of query heads of the unit's
// GQA group); wave w handles head w / 2 and queries 64 (w % 2) .. + 63.  The
// keys 0 .. end of the query block stream through LDS in blocks of 64 (k rows and
// v^T rows, double buffered, loaded into registers one block ahead).  Per
// 32-key tile and 32-query tile: S^T = K Q^T on the matrix cores (bf16 inputs,
// fp32 accumulation), the causal mask, an online softmax per query (running
// maximum m and sum l, the output rescaled by exp(m_old - m_new)), then
// O^T += V^T P with P in bf16.  Finally y = O / l.  Query blocks are dealt out
// last first: their key ranges are the longest.
#include "oal_tile.h"

namespace oal {

namespace sm {
constexpr int QB = 128;                 // queries per workgroup and head
constexpr int HPW = 2;                  // query heads per workgroup
constexpr int KB = 64;                  // keys per staged block
constexpr int Q_BYTES = HPW * QB * 128;
constexpr int ROW_BYTES = KB * 128;     // 64 rows of 64 bf16
constexpr float LOG2E = 1.4426950408889634f;
}  // namespace sm

namespace {

__device__ __forceinline__ float wave_max32x2(float x) {   // with the lane 32 apart
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

}  // namespace

template <typename O>
__global__ void __launch_bounds__(256, 2)
k_softmax(int n_q_heads, int n_kv_heads, int seq_len, int n_qb, int n_hg,
          const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
          const uint16_t* __restrict__ v, O* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t s_q[sm::Q_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[sm::ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[sm::ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_v0[sm::ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_v1[sm::ROW_BYTES];

  const int per_unit = n_qb * n_hg;
  const int unit = blockIdx.x / per_unit, rem = blockIdx.x % per_unit;
  const int qblk = n_qb - 1 - rem / n_hg, hg = rem % n_hg;
  const int b = unit / n_kv_heads, kv = unit % n_kv_heads;
  const int rep = n_q_heads / n_kv_heads;
  const int q0 = qblk * sm::QB;
  const int qlen = min(sm::QB, seq_len - q0);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int hslot = wave >> 1, sub = wave & 1;
  const int hl = hg * sm::HPW + hslot;
  const bool head_ok = hl < rep;
  const int hq = kv * rep + (head_ok ? hl : 0);

  // ---- q of both heads (rows swizzled by row_key), zero past the sequence
  constexpr int QIT = sm::HPW * sm::QB * 8 / 256;
  uint4 qv[QIT];
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int hs = it * 256 / (sm::QB * 8);
    const int r = tid + 256 * it - hs * sm::QB * 8, tok = r >> 3, part = r & 7;
    const int hh = min(hg * sm::HPW + hs, rep - 1);
    const size_t row = ((size_t)b * n_q_heads + kv * rep + hh) * seq_len + q0 + min(tok, qlen - 1);
    qv[it] = reinterpret_cast<const uint4*>(q + row * DH)[part];
  }
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int hs = it * 256 / (sm::QB * 8);
    const int r = tid + 256 * it - hs * sm::QB * 8, tok = r >> 3, part = r & 7;
    const bool ok = hg * sm::HPW + hs < rep && tok < qlen;
    *reinterpret_cast<uint4*>(s_q + (hs * sm::QB + tok) * 128 + ((part ^ row_key(tok)) << 4)) =
        ok ? qv[it] : make_uint4(0, 0, 0, 0);
  }

  // ---- key blocks: thread t holds dims 8 (t & 7) .. + 7 of keys 2 (t >> 3) + e
  const size_t kvrow0 = (size_t)unit * seq_len;
  const int kpart = tid & 7, kpair = tid >> 3;
  const int n_kb = (q0 + qlen - 1) / sm::KB + 1;
  uint4 kq[2], vq[2];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = kb * sm::KB + 2 * kpair + e;
      const size_t row = kvrow0 + min(key, seq_len - 1);
      kq[e] = reinterpret_cast<const uint4*>(k + row * DH)[kpart];
      vq[e] = reinterpret_cast<const uint4*>(v + row * DV)[kpart];
      if (key >= seq_len) {
        kq[e] = make_uint4(0, 0, 0, 0);
        vq[e] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // k rows as read by the S product; v^T rows with the keys of each 16-block
  // permuted (position 8 h + 4 a + e holds key 8 a + 4 h + e, the key order of
  // the S accumulator rows)
  auto deposit = [&](uint8_t* ka, uint8_t* va) {
    const int tok = 2 * kpair;
    *reinterpret_cast<uint4*>(ka + tok * 128 + ((kpart ^ row_key(tok)) << 4)) = kq[0];
    *reinterpret_cast<uint4*>(ka + (tok + 1) * 128 + ((kpart ^ row_key(tok + 1)) << 4)) = kq[1];
    const int pk = (tok & ~15) | (((tok >> 2) & 1) << 3) | (((tok >> 3) & 1) << 2) | (tok & 3);
    const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&vq[0]);
    const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&vq[1]);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int w = kpart * 8 + x;
      const uint32_t word = (x & 1) ? (a0[x >> 1] >> 16) | (a1[x >> 1] & 0xffff0000u)
                                    : (a0[x >> 1] & 0xffffu) | (a1[x >> 1] << 16);
      *reinterpret_cast<uint32_t*>(va + w * 128 + (((pk >> 3) ^ row_key(w)) << 4) + ((pk & 7) << 1)) = word;
    }
  };
  fetch(0);
  deposit(s_k0, s_v0);
  __syncthreads();

  const int tok0 = q0 + sub * 64;               // this wave's first query
  const uint8_t* qw = s_q + hslot * sm::QB * 128;
  const SwRow qrow0(qw, sub * 64 + col), qrow1(qw, sub * 64 + 32 + col);
  const float sc = 0.125f * sm::LOG2E;          // 1/sqrt(d_h), in base 2
  float mx[2] = {-INFINITY, -INFINITY}, sum[2] = {0.f, 0.f};
  f32x16 acc[2][2];                             // O^T[w][query]: [w tile][query tile]
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = splat16(0.f);

  for (int kb = 0; kb < n_kb; ++kb) {
    const uint8_t* ka = (kb & 1) ? s_k1 : s_k0;
    const uint8_t* va = (kb & 1) ? s_v1 : s_v0;
    if (kb + 1 < n_kb) fetch(kb + 1);
    if (head_ok) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key0 = kb * sm::KB + 32 * kt;
        if (key0 > tok0 + 63) continue;         // later than every query of the wave
        const SwRow krow(ka, 32 * kt + col);
        bf16x8 kr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kr[ks] = *reinterpret_cast<const bf16x8*>(krow.chunk(2 * ks + half));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int qt0 = tok0 + 32 * nt;       // first query of the tile
          if (key0 > qt0 + 31) continue;
          const SwRow& qr = nt ? qrow1 : qrow0;
          f32x16 s = splat16(0.f);
          // products at raised wave priority: a wave with its operands ready issues
          // them ahead of the co-resident waves' exponentials (about 1 %, measured)
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            s = mfma32(kr[ks], *reinterpret_cast<const bf16x8*>(qr.chunk(2 * ks + half)), s);
          __builtin_amdgcn_s_setprio(0);
          // scores in base 2; keys after the query are masked
          const int query = qt0 + col;
          float tmax = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const bool vis = key0 + acc_row(i, half) <= query;
            s[i] = vis ? s[i] * sc : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
          }
          tmax = wave_max32x2(tmax);
          const float mnew = fmaxf(mx[nt], tmax);
          const float alpha = exp2f(mx[nt] - mnew);   // 0 while mx is -inf
          mx[nt] = mnew;
          float ps = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[i] = exp2f(s[i] - mnew);
            ps += s[i];
          }
          sum[nt] = sum[nt] * alpha + ps + __shfl_xor(ps, 32, 64);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] *= alpha;
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = s[8 * s2 + j];
            const bf16x8 pb = pack8(x);
            const int kc8 = 4 * kt + 2 * s2 + half;   // 16-byte chunk of the v^T row
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
              const SwRow vr(va, 32 * mt + col);
              acc[mt][nt] = mfma32(*reinterpret_cast<const bf16x8*>(vr.chunk(kc8)), pb, acc[mt][nt]);
            }
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }
    }
    if (kb + 1 < n_kb) deposit((kb & 1) ? s_k0 : s_k1, (kb & 1) ? s_v0 : s_v1);
    __syncthreads();
  }

  // ---- y = O / l
  if (!head_ok) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int tok = sub * 64 + 32 * nt + col;
    if (tok >= qlen) continue;
    const float inv = 1.0f / sum[nt];
    O* yr = y + (((size_t)b * n_q_heads + hq) * seq_len + q0 + tok) * DV;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int w0 = 32 * mt + 8 * g4 + 4 * half;
        const float o[4] = {acc[mt][nt][4 * g4] * inv, acc[mt][nt][4 * g4 + 1] * inv,
                            acc[mt][nt][4 * g4 + 2] * inv, acc[mt][nt][4 * g4 + 3] * inv};
        Elem<O>::store4(yr, w0, o);
      }
  }
}

oal_status launch_softmax(int batch, int n_q_heads, int n_kv_heads, int seq_len, const void* q,
                          const void* k, const void* v, void* y, oal_dtype out_dtype,
                          hipStream_t stream) {
  const int units = batch * n_kv_heads;
  const int rep = n_q_heads / n_kv_heads;
  const int n_hg = (rep + sm::HPW - 1) / sm::HPW;
  const int n_qb = (seq_len + sm::QB - 1) / sm::QB;
  const long long blocks = (long long)units * n_qb * n_hg;
  if (blocks > 0x7fffffff) return set_error(OAL_ERR_UNSUPPORTED, "problem too large");
  const auto* qq = reinterpret_cast<const uint16_t*>(q);
  const auto* kk = reinterpret_cast<const uint16_t*>(k);
  const auto* vv = reinterpret_cast<const uint16_t*>(v);
  ProfScope ps("k_softmax", stream);
  if (out_dtype == OAL_F32)
    hipLaunchKernelGGL(k_softmax<float>, dim3((unsigned)blocks), dim3(256), 0, stream, n_q_heads,
                       n_kv_heads, seq_len, n_qb, n_hg, qq, kk, vv, reinterpret_cast<float*>(y));
  else
    hipLaunchKernelGGL(k_softmax<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream, n_q_heads,
                       n_kv_heads, seq_len, n_qb, n_hg, qq, kk, vv, reinterpret_cast<uint16_t*>(y));
  return check_launch("k_softmax");
}

}  // namespace oal
