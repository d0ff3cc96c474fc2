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
// MFMAs per k-step, fp32 accumulation.  The launch is bound by reading x
// from HBM once.  A workgroup takes 64 tokens and an eighth of k: it loads
// its eighth of W (fp32, from L2), starts all its x loads, splits W into
// hi/lo bf16 rows per channel in LDS while x streams in, then runs the MFMAs and sums its
// eight waves' partials in a fixed order into the workspace; a second small
// kernel adds the eight parts (fixed order) and updates z.  Splitting k
// keeps each CU's share of W small: with every workgroup reading all of W,
// W was twice the bytes of x per CU and the CUs' outstanding loads, not
// HBM, set the pace; with 120 registers per lane two workgroups share a CU.
#include <algorithm>

#include "bca_internal.h"

namespace bca {

namespace {
constexpr int kThreads = 256;
constexpr int kRows = 64;      // tokens per projection workgroup (4 MFMA row tiles)
constexpr int kPWaves = 8;     // waves per projection workgroup (split the k-steps)
constexpr int kMaxSteps = 4;   // k-steps of 32 per wave kept in registers
}  // namespace

__global__ __launch_bounds__(kPWaves * 64) void euler_proj_kernel(EulerArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kch = a.k / kEulerChunks;        // k per workgroup
  const int kc = blockIdx.y;
  const int nst = kch / 32;                  // k-steps of the chunk
  const int pitch = kch + 8;                 // bf16 per LDS row (16-byte pad: no bank conflicts)
  uint16_t* whi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* wlo = whi + 16 * pitch;
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  const int g = lane >> 4, ln = lane & 15;

  // W's eighth first (from L2, it lands before the x stream), then every x
  // fragment of this wave's k-steps (st = wave + kPWaves * j, all four row
  // tiles); W is split and written to LDS while x is in flight.
  // Unit u = 8 k-rows x 4 channels: hi = RNE(w), lo = RNE(w - hi).
  const float* wb = a.w + (int64_t)kc * kch * 16;
  const int nunit = (kch / 8) * 4;
  static_assert(kEulerMaxK / kEulerChunks / 8 * 4 <= kPWaves * 64, "one W unit per thread");
  f32x4 f[8];
  if (tid < nunit) {
    const int r8 = tid >> 2, q = tid & 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = *reinterpret_cast<const f32x4*>(wb + (8 * r8 + i) * 16 + 4 * q);
  }
  u32x4 xr[kMaxSteps][4];
  const uint16_t* xb = static_cast<const uint16_t*>(a.x) + (int64_t)kc * kch + 8 * g;
#pragma unroll
  for (int j = 0; j < kMaxSteps; ++j) {
    const int st = wave + kPWaves * j;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int64_t row = r0 + 16 * rt + ln;
      xr[j][rt] = (st < nst && row < a.n_tok)
                      ? *reinterpret_cast<const u32x4*>(xb + row * a.k + 32 * st)
                      : u32x4{0, 0, 0, 0};
    }
  }
  if (tid < nunit) {
    const int r8 = tid >> 2, q = tid & 3;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 hv, lv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 h = (__bf16)f[i][c];
        hv[i] = h;
        lv[i] = (__bf16)(f[i][c] - (float)h);
      }
      *reinterpret_cast<bf16x8*>(whi + (4 * q + c) * pitch + 8 * r8) = hv;
      *reinterpret_cast<bf16x8*>(wlo + (4 * q + c) * pitch + 8 * r8) = lv;
    }
  }
  __syncthreads();

  f32x4 acc[4] = {};
#pragma unroll
  for (int j = 0; j < kMaxSteps; ++j) {
    const int st = wave + kPWaves * j;
    if (st < nst) {
      const bf16x8 h = *reinterpret_cast<const bf16x8*>(whi + ln * pitch + 32 * st + 8 * g);
      const bf16x8 l = *reinterpret_cast<const bf16x8*>(wlo + ln * pitch + 32 * st + 8 * g);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const bf16x8 xa = __builtin_bit_cast(bf16x8, xr[j][rt]);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, h, acc[rt], 0, 0, 0);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, l, acc[rt], 0, 0, 0);
      }
    }
  }
  // acc[rt][e] = partial v[token 16 rt + 4 g + e][channel ln]; sum the
  // waves in order through LDS (reusing the W rows)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(wave * kRows + 16 * rt + 4 * g + e) * 16 + ln] = acc[rt][e];
  __syncthreads();
  for (int i = tid; i < kRows * 16; i += kPWaves * 64) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kPWaves; ++w) v += red[w * kRows * 16 + i];
    const int64_t row = r0 + (i >> 4);
    if (row < a.n_tok) a.part[((int64_t)kc * a.n_tok + row) * 16 + (i & 15)] = v;
  }
}

// z <- z - dtau * (sum of the k-part partials, in order)
__global__ __launch_bounds__(kThreads) void euler_reduce_kernel(EulerArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.n_tok * 16) return;
  float v = 0.0f;
#pragma unroll
  for (int c = 0; c < kEulerChunks; ++c) v += a.part[c * a.n_tok * 16 + i];
  a.z[i] = __builtin_fmaf(-a.dtau, v, a.z[i]);
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

hipError_t launch_euler_proj(const EulerArgs& a, hipStream_t s) {
  const int kch = a.k / kEulerChunks;
  static_assert(kEulerMaxK / kEulerChunks / 32 <= kPWaves * kMaxSteps, "k-steps per part");
  if (a.n_ch != 16 || a.k % (32 * kEulerChunks) != 0 || a.k > kEulerMaxK || !a.part)
    return hipErrorInvalidValue;
  const size_t lds = std::max<size_t>((size_t)2 * 16 * (kch + 8) * 2, (size_t)kPWaves * kRows * 16 * 4);
  const dim3 grid((unsigned)((a.n_tok + kRows - 1) / kRows), kEulerChunks);
  hipError_t e = hipSuccess;
  if (lds > 65536) {                         // only k above 7936 needs more than the default
    e = hipFuncSetAttribute((const void*)euler_proj_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  euler_proj_kernel<<<grid, kPWaves * 64, lds, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  euler_reduce_kernel<<<(unsigned)((a.n_tok * 16 + kThreads - 1) / kThreads), kThreads, 0, s>>>(a);
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
