// Flow-matching Euler step with a fused velocity projection.
//
// The interpolant z_tau = (1 - tau) z0 + tau eps has velocity dz/dtau =
// eps - z0 (deep read "全双工语音模型精读⑫：Wan-Streamer", section 3.2);
// integrating from tau = 1 (noise) toward tau = 0 (clean latents) an explicit
// Euler step is z <- z - dtau * v.  Here v is the attention output of the
// unit projected by a fixed matrix W: v[i][c] = sum_k x[i][k] W[k][c].
//
// bf16 x, n_ch = 16: the product runs on v_mfma_f32_16x16x32_bf16 with W
// split into bf16 high and low halves (W = hi + lo to ~2^-16 relative), two
// MFMAs per k-step, fp32 accumulation.  The kernel is bound by reading x
// from HBM; W (fp32) is re-read from L2 and staged transposed in LDS.  k is
// split across workgroups; the last workgroup of a token block (atomic
// counter) sums the partials in split order and applies the update, then
// resets the counter, so results do not depend on arrival order.
#include "bca_internal.h"

namespace bca {

namespace {
constexpr int kThreads = 256;
constexpr int kMaxSteps = 20;       // k-steps of 32 per split (kchunk <= 640)
constexpr int kWPitch = kMaxSteps * 32 + 8;   // LDS row pitch (bf16), +16 bytes

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}
}  // namespace

__global__ __launch_bounds__(kThreads) void euler_bf16_proj_kernel(EulerArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t whi[16 * kWPitch];
  __shared__ __attribute__((aligned(16))) uint16_t wlo[16 * kWPitch];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tb = blockIdx.x, sp = blockIdx.y;
  const int kbeg = sp * a.kchunk;
  const int kend = min(a.k, kbeg + a.kchunk);
  const int nsteps = (kend - kbeg) / 32;
  const int64_t row = (int64_t)tb * kEulerTokens + wave * 16 + (lane & 15);
  const bool rv = row < a.n_tok;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);

  // issue every x load of this split first (A operand: row, 8 k per lane)
  u32x4 xr[kMaxSteps];
  const uint16_t* xp = x + row * a.k + kbeg + 8 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < kMaxSteps; ++j)
    xr[j] = (rv && j < nsteps) ? *reinterpret_cast<const u32x4*>(xp + 32 * j) : u32x4{0, 0, 0, 0};

  // W[kbeg:kend, 0:16] -> LDS as W^T hi/lo bf16, rows = channel
  for (int u = tid; u < 16 * nsteps * 4; u += kThreads) {
    const int c = u & 15, oct = u >> 4;
    const float* wp = a.w + (int64_t)(kbeg + 8 * oct) * 16 + c;
    uint16_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = wp[16 * e];
      hi[e] = bf16_rne(f);
      lo[e] = bf16_rne(f - __uint_as_float((uint32_t)hi[e] << 16));
    }
    *reinterpret_cast<u32x4*>(&whi[c * kWPitch + 8 * oct]) = *reinterpret_cast<const u32x4*>(hi);
    *reinterpret_cast<u32x4*>(&wlo[c * kWPitch + 8 * oct]) = *reinterpret_cast<const u32x4*>(lo);
  }
  __syncthreads();

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int wrow = (lane & 15) * kWPitch + 8 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < kMaxSteps; ++j) {
    if (j < nsteps) {
      const bf16x8 xa = __builtin_bit_cast(bf16x8, xr[j]);
      const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&whi[wrow + 32 * j]));
      const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&wlo[wrow + 32 * j]));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bl, acc, 0, 0, 0);
    }
  }

  // acc[e] = v[token 4*(lane>>4)+e of this wave's 16][channel lane&15]
  const int c = lane & 15;
  const int64_t tok0 = (int64_t)tb * kEulerTokens + wave * 16 + 4 * (lane >> 4);
  if (a.ksplit == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (tok0 + e < a.n_tok) {
        float* zp = a.z + (tok0 + e) * 16 + c;
        *zp = __builtin_fmaf(-a.dtau, acc[e], *zp);
      }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (tok0 + e < a.n_tok) a.ws_part[((int64_t)sp * a.n_tok + tok0 + e) * 16 + c] = acc[e];
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&a.counters[tb], 1) == a.ksplit - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int i = tid; i < kEulerTokens * 16; i += kThreads) {
    const int64_t tok = (int64_t)tb * kEulerTokens + i / 16;
    if (tok >= a.n_tok) continue;
    float v = 0.0f;
    for (int s = 0; s < a.ksplit; ++s) v += a.ws_part[((int64_t)s * a.n_tok + tok) * 16 + (i & 15)];
    float* zp = a.z + tok * 16 + (i & 15);
    *zp = __builtin_fmaf(-a.dtau, v, *zp);
  }
  if (tid == 0) a.counters[tb] = 0;
}

// Any x dtype / n_ch <= 64 / k: one workgroup per token, fp32 FMA, fixed
// reduction order.  Used for fp32 attention outputs and odd shapes.
template <bool XF32>
__global__ __launch_bounds__(kThreads) void euler_generic_kernel(EulerArgs a) {
  __shared__ float red[4][64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) acc[c] = 0.0f;
  for (int kk = tid; kk < a.k; kk += kThreads) {
    float xv;
    if constexpr (XF32) xv = static_cast<const float*>(a.x)[row * a.k + kk];
    else xv = __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.x)[row * a.k + kk] << 16);
    const float* wp = a.w + (int64_t)kk * a.n_ch;
#pragma unroll
    for (int c = 0; c < 64; ++c)
      if (c < a.n_ch) acc[c] = fmaf(xv, wp[c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    if (c >= a.n_ch) break;
    float v = acc[c];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[wave][c] = v;
  }
  __syncthreads();
  if (tid < a.n_ch) {
    const float v = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    float* zp = a.z + row * a.n_ch + tid;
    *zp = __builtin_fmaf(-a.dtau, v, *zp);
  }
}

// v given: z <- z - dtau * v, elementwise.
__global__ __launch_bounds__(kThreads) void euler_plain_kernel(EulerArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.n_tok * a.n_ch) return;
  a.z[i] = __builtin_fmaf(-a.dtau, static_cast<const float*>(a.x)[i], a.z[i]);
}

hipError_t launch_euler_bf16_proj(const EulerArgs& a, hipStream_t s) {
  if (a.n_ch != 16 || a.k % 32 != 0 || a.kchunk % 32 != 0 || a.kchunk > kMaxSteps * 32)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.n_tok + kEulerTokens - 1) / kEulerTokens), (unsigned)a.ksplit);
  euler_bf16_proj_kernel<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_euler_generic(const EulerArgs& a, bool x_f32, hipStream_t s) {
  if (a.n_ch > 64) return hipErrorInvalidValue;
  if (x_f32) euler_generic_kernel<true><<<(unsigned)a.n_tok, kThreads, 0, s>>>(a);
  else euler_generic_kernel<false><<<(unsigned)a.n_tok, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_euler_plain(const EulerArgs& a, hipStream_t s) {
  const int64_t n = a.n_tok * a.n_ch;
  euler_plain_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bca
