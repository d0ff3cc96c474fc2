// Block-causal attention, fp32 path (all of Q, K, V, O in fp32).
//
// Same visibility rule as the MFMA path (explainer "wan-streamer-realtime-av",
// block-causal figure caption): query at position p sees key j iff
// j / B <= p / B.  One lane per query row, exact online softmax in fp32
// (running max, rescale on every new maximum), K/V tiles of 64 keys staged in
// LDS.  This path exists for fp32 caches (small heads, tight tolerances); it
// is not tuned for throughput.
#include <math.h>

#include "bca_internal.h"

namespace bca {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float kt[kKeyTile][D + 1];
  __shared__ float vt[kKeyTile][D + 1];
  const int h = blockIdx.y;
  const int H = a.n_heads;
  const int64_t row0 = (int64_t)blockIdx.x * 64;
  const int64_t row = row0 + threadIdx.x;
  const bool active = row < a.n_q;
  const int64_t B = a.block_size;
  const int64_t rlast = min(row0 + 63, a.n_q - 1);
  const int64_t lim_last = min(a.n_kv, ((a.q_pos0 + rlast) / B + 1) * B);
  const int64_t lim = active ? min(a.n_kv, ((a.q_pos0 + row) / B + 1) * B) : 0;
  const float* q = static_cast<const float*>(a.q);
  const float* kp = static_cast<const float*>(a.k_pages);
  const float* vp = static_cast<const float*>(a.v_pages);
  const int psm = (1 << a.ps_log2) - 1;

  float qv[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = active ? q[(row * H + h) * D + d] : 0.0f;
    o[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  for (int64_t k0 = 0; k0 < lim_last; k0 += kKeyTile) {
    __syncthreads();
    {
      const int r = threadIdx.x;
      const int64_t key = k0 + r;
      if (key < a.n_kv) {
        const int64_t page = a.page_table[key >> a.ps_log2];
        const int64_t slot = key & psm;
        const float* ksrc = kp + (((page * H + h) << a.ps_log2) | slot) * D;
        const float* vsrc = vp + (((page * H + h) * D) << a.ps_log2) + slot;
        for (int d = 0; d < D; ++d) {
          kt[r][d] = ksrc[d];
          vt[r][d] = vsrc[(int64_t)d << a.ps_log2];
        }
      } else {
        for (int d = 0; d < D; ++d) { kt[r][d] = 0.0f; vt[r][d] = 0.0f; }
      }
    }
    __syncthreads();
    const int jn = (int)min((int64_t)kKeyTile, lim - k0);
    for (int j = 0; j < jn; ++j) {
      float sdot = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) sdot = fmaf(qv[d], kt[j][d], sdot);
      const float sc = sdot * a.scale;
      const float mn = fmaxf(m, sc);
      const float corr = expf(m - mn);
      const float p = expf(sc - mn);
      l = l * corr + p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, vt[j][d], o[d] * corr);
      m = mn;
    }
  }
  if (!active) return;
  const float inv = 1.0f / l;
  float* out = static_cast<float*>(a.out) + (row * H + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = o[d] * inv;
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.n_q + 63) / 64), (unsigned)a.n_heads);
  switch (a.head_dim) {
    case 32: attn_f32_kernel<32><<<grid, 64, 0, s>>>(a); break;
    case 64: attn_f32_kernel<64><<<grid, 64, 0, s>>>(a); break;
    case 128: attn_f32_kernel<128><<<grid, 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bca
