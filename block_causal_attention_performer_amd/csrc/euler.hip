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
// MFMAs per k-step, fp32 accumulation.  W is first rewritten transposed,
// as hi/lo bf16 rows per channel (w_prep_kernel, 64 bytes per row of W, into
// the caller's workspace), so every MFMA operand is one 16-byte load.  The
// main kernel is bound by reading x from HBM once: one workgroup per 16
// tokens, its sixteen waves split k (many loads in flight per CU, since a
// unit has only a few hundred such token groups) and add their 16x16
// partials through LDS in a fixed order before the update.
#include "bca_internal.h"

namespace bca {

namespace {
constexpr int kThreads = 256;
constexpr int kTok = 16;       // tokens per workgroup
constexpr int kProjWaves = 16; // waves per projection workgroup (split k)
constexpr int kBatch = 8;      // k-steps loaded ahead per wave

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}
}  // namespace

// W [k][16] fp32 -> wt_hi / wt_lo [16][k] bf16 with W = hi + lo (+ O(2^-16)).
__global__ __launch_bounds__(kThreads) void w_prep_kernel(const float* w, uint16_t* wt_hi,
                                                          uint16_t* wt_lo, int k) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= k * 16) return;
  const int kk = i >> 4, c = i & 15;
  const float f = w[i];
  const uint16_t hi = bf16_rne(f);
  wt_hi[(int64_t)c * k + kk] = hi;
  wt_lo[(int64_t)c * k + kk] = bf16_rne(f - __uint_as_float((uint32_t)hi << 16));
}

__global__ __launch_bounds__(kProjWaves * 64) void euler_proj_kernel(EulerArgs a) {
  __shared__ float part[kProjWaves][kTok * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = (int64_t)blockIdx.x * kTok + (lane & 15);
  const bool rv = row < a.n_tok;
  const int nsteps = a.k / 32;
  const int s0 = wave * nsteps / kProjWaves, s1 = (wave + 1) * nsteps / kProjWaves;
  const int oct = 8 * (lane >> 4);
  const uint16_t* xp = static_cast<const uint16_t*>(a.x) + row * a.k + oct;
  const uint16_t* hp = a.wt_hi + (int64_t)(lane & 15) * a.k + oct;
  const uint16_t* lp = a.wt_lo + (int64_t)(lane & 15) * a.k + oct;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int sb = s0; sb < s1; sb += kBatch) {
    u32x4 xr[kBatch], hr[kBatch], lr[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int st = sb + j;
      const bool ok = st < s1;
      xr[j] = (ok && rv) ? *reinterpret_cast<const u32x4*>(xp + 32 * st) : u32x4{0, 0, 0, 0};
      hr[j] = ok ? *reinterpret_cast<const u32x4*>(hp + 32 * st) : u32x4{0, 0, 0, 0};
      lr[j] = ok ? *reinterpret_cast<const u32x4*>(lp + 32 * st) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bf16x8 xa = __builtin_bit_cast(bf16x8, xr[j]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, hr[j]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, lr[j]), acc, 0, 0, 0);
    }
  }
  // acc[e] = partial v[token 4*(lane>>4)+e][channel lane&15]
#pragma unroll
  for (int e = 0; e < 4; ++e) part[wave][(4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[e];
  __syncthreads();
  if (tid >= kTok * 16) return;
  const int64_t tok = (int64_t)blockIdx.x * kTok + (tid >> 4);
  if (tok < a.n_tok) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kProjWaves; ++w) v += part[w][tid];
    float* zp = a.z + tok * 16 + (tid & 15);
    *zp = __builtin_fmaf(-a.dtau, v, *zp);
  }
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

hipError_t launch_w_prep(const float* w, uint16_t* wt_hi, uint16_t* wt_lo, int k, hipStream_t s) {
  const int n = k * 16;
  w_prep_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, s>>>(w, wt_hi, wt_lo, k);
  return hipGetLastError();
}

hipError_t launch_euler_proj(const EulerArgs& a, hipStream_t s) {
  if (a.n_ch != 16 || a.k % 32 != 0 || !a.wt_hi || !a.wt_lo) return hipErrorInvalidValue;
  euler_proj_kernel<<<(unsigned)((a.n_tok + kTok - 1) / kTok), kProjWaves * 64, 0, s>>>(a);
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
