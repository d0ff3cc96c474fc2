// kv_append kernels: write a unit's K/V slice into the paged cache.
//
// The performer appends every received KV slice to its own full-history
// cache (deep read "全双工语音模型精读⑫：Wan-Streamer", section 4, step 3).
// K pages are token-major [page][h][slot][d]; V pages are d-major
// [page][h][d][slot] so that the attention kernel reads 16-byte runs along
// the key axis.  The bf16/fp32 copy is pure data movement (HBM bound): each
// lane moves a 16-byte-square block of K and of V, transposing V in
// registers, so every load and store is a 16-byte vector.
#include "bca_internal.h"

namespace bca {
namespace {

constexpr int kThreads = 256;               // fp8 append kernel
constexpr int kCopyThreads = 256;           // bf16 / f32 copy kernel

// Transpose an E x E block held as E rows of 16 bytes (row = token,
// column = head dim) into E rows of head dims, each holding E tokens.
template <typename T>
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[16 / sizeof(T)],
                                                u32x4 (&out)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    // out[d].word[w] = (token 2w, token 2w+1) of column d
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        out[d][w] = __builtin_amdgcn_perm(in[2 * w + 1][d >> 1], in[2 * w][d >> 1],
                                          (d & 1) ? 0x07060302u : 0x05040100u);
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int w = 0; w < 4; ++w) out[d][w] = in[w][d];
  }
}

// One workgroup of four waves per (TPW consecutive tokens, head), over the
// tokens [g0, g1) of the slice whose E-aligned groups it covers fully (four
// waves rather than one: a workgroup's V^T stores then cover 256 bytes of
// each head-dim row, so a slice that starts off a 64-byte boundary writes
// fewer partial lines; 38 against 44 us for the v0.2 slice at such a
// start, the same 32 us at an aligned one).  Thread (to, j) moves the
// E tokens t0 = g0 + to*E .. +E-1, head dims j*E .. +E-1: E 16-byte loads of
// K and of V; K rows are stored as they are, the V block is transposed in
// registers and stored as E runs of E tokens of the V^T rows.  The E tokens
// lie in one page (pages hold >= 16 tokens, groups are E-aligned).
// T: element type (uint16_t for bf16, float for f32); D: head dim.
template <typename T, int D>
__global__ __launch_bounds__(kCopyThreads) void append_copy_kernel(AppendArgs a, int64_t g0, int64_t g1) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte vector
  constexpr int JO = D / E;                  // 16-byte chunks per token row
  constexpr int TO = kCopyThreads / JO;      // token groups per workgroup
  constexpr int TPW = TO * E;                // tokens per workgroup
  const int lane = threadIdx.x;
  const int j = lane % JO, to = lane / JO;
  const int h = blockIdx.y;
  const int H = a.n_heads;
  const int64_t t0 = g0 + (int64_t)blockIdx.x * TPW + to * E;
  if (t0 >= g1) return;
  const int64_t page = a.page_table[t0 >> a.ps_log2];
  const int64_t slot0 = t0 & ((1 << a.ps_log2) - 1);
  const T* kin = static_cast<const T*>(a.k_new) + ((t0 - a.n0) * H + h) * D + j * E;
  const T* vin = static_cast<const T*>(a.v_new) + ((t0 - a.n0) * H + h) * D + j * E;
  const int64_t in_stride = (int64_t)H * D;

  u32x4 kr[E], vr[E], vt[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kr[e] = *reinterpret_cast<const u32x4*>(kin + e * in_stride);
    vr[e] = *reinterpret_cast<const u32x4*>(vin + e * in_stride);
  }
  T* krow = static_cast<T*>(a.k_pages) + (((page * H + h) << a.ps_log2) + slot0) * D + j * E;
#pragma unroll
  for (int e = 0; e < E; ++e) *reinterpret_cast<u32x4*>(krow + e * D) = kr[e];
  transpose_block<T>(vr, vt);
  T* vcol = static_cast<T*>(a.v_pages) + ((((page * H + h) * D + j * E) << a.ps_log2) + slot0);
#pragma unroll
  for (int e = 0; e < E; ++e) *reinterpret_cast<u32x4*>(vcol + (e << a.ps_log2)) = vt[e];
}

// Tokens of the slice outside [g0, g1) (fewer than E at each end): one
// workgroup per (token, head), one element per thread.
template <typename T>
__global__ void append_edge_kernel(AppendArgs a, int64_t g0, int64_t g1) {
  const int64_t lo = a.n0, hi = a.n0 + a.n_new;
  const int64_t n_head_edge = (g0 < hi ? g0 : hi) - lo;
  const int64_t t = blockIdx.x < n_head_edge ? lo + blockIdx.x
                                             : (g1 > g0 ? g1 : g0) + (blockIdx.x - n_head_edge);
  const int d = threadIdx.x;
  if (t >= hi || d >= a.head_dim) return;
  const int h = blockIdx.y, H = a.n_heads, D = a.head_dim;
  const int64_t page = a.page_table[t >> a.ps_log2];
  const int64_t slot = t & ((1 << a.ps_log2) - 1);
  const int64_t src = ((t - lo) * H + h) * D + d;
  static_cast<T*>(a.k_pages)[(((page * H + h) << a.ps_log2) + slot) * D + d] =
      static_cast<const T*>(a.k_new)[src];
  static_cast<T*>(a.v_pages)[(((page * H + h) * D + d) << a.ps_log2) + slot] =
      static_cast<const T*>(a.v_new)[src];
}

// ------------------------------------------------------------------ fp8

// Round-to-nearest-even onto the finite OCP E4M3FN values (OCP 8-bit
// floating point spec: bias 7, 3 mantissa bits, subnormal quantum 2^-9,
// S.1111.111 reserved for NaN), saturating at 448, two values at once by the
// hardware conversion (v_cvt_pk_fp8_f32) into bytes 0-1 (HI = false) or 2-3
// (HI = true) of `old`.  The inputs are clamped to +-448 first (the
// saturation).  The append tests check the codes bit for bit against the
// oracle's encoder (ties, subnormals, saturation).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_rne_sat(float x, float y, uint32_t old) {
  x = fminf(fmaxf(x, -448.0f), 448.0f);
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, y, (int)old, HI);
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
  // wave reduction then across the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The values of rows a page already holds: its E4M3 codes (exact in fp32
// through the hardware conversion) times the page's scale, rounded to fp32.
__device__ __forceinline__ void held8(uint2 codes, float sc, float (&x)[8]) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(codes.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(codes.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(codes.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(codes.y, true);
  x[0] = a[0] * sc; x[1] = a[1] * sc; x[2] = b[0] * sc; x[3] = b[1] * sc;
  x[4] = c[0] * sc; x[5] = c[1] * sc; x[6] = d[0] * sc; x[7] = d[1] * sc;
}

// One workgroup per (logical page touched, head).  The slice fills rows
// [n_old, r1) of the page; rows [0, n_old) (first page of an append that
// starts inside a page) already hold codes, whose values enter the block as
// they are held, so the whole page is quantised afresh over its valid rows;
// rows past r1 get code 0.  Each thread reads the held codes of its own
// 8-value chunk before it writes the chunk, and every thread reads the
// page's old scale before the barrier after which thread 0 replaces it.
template <int D>
__global__ __launch_bounds__(kThreads) void append_fp8_kernel(AppendArgs a) {
  const int ps = 1 << a.ps_log2;
  const int h = blockIdx.y;
  const int H = a.n_heads;
  const int64_t lp = (a.n0 >> a.ps_log2) + blockIdx.x;
  const int64_t t0 = lp << a.ps_log2;
  const int64_t r1l = a.n0 + a.n_new - t0;
  const int r1 = (int)(r1l < ps ? r1l : ps);
  const int n_old = a.n0 > t0 ? (int)(a.n0 - t0) : 0;
  const int64_t page = a.page_table[lp];
  const uint16_t* src_k = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* src_v = static_cast<const uint16_t*>(a.v_new);
  uint8_t* kp = static_cast<uint8_t*>(a.k_pages) + ((page * H + h) << a.ps_log2) * D;
  uint8_t* vp = static_cast<uint8_t*>(a.v_pages) + ((page * H + h) << a.ps_log2) * D;
  __shared__ float red[4];
  __shared__ uint8_t vt[D * 260];   // V^T codes staged [d][slot], pitch ps+4 (ps <= 256)

  for (int which = 0; which < 2; ++which) {
    const uint16_t* src = which == 0 ? src_k : src_v;
    float* scales = which == 0 ? a.k_scales : a.v_scales;
    const float old_sc = n_old > 0 ? scales[page * H + h] : 1.0f;
    // the 8 values of row r, head dims 8c .. 8c+7, as the block holds them
    auto row8 = [&](int r, int c, float (&x)[8]) {
      if (r < n_old) {
        uint2 codes;
        if (which == 0) {
          codes = *reinterpret_cast<const uint2*>(kp + (int64_t)r * D + c * 8);
        } else {
          uint32_t w[2] = {0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e >> 2] |= (uint32_t)vp[(int64_t)(c * 8 + e) * ps + r] << (8 * (e & 3));
          codes = make_uint2(w[0], w[1]);
        }
        held8(codes, old_sc, x);
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + ((t0 - a.n0 + r) * H + h) * D + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(v[e] << 16);
          x[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
        }
      }
    };
    // amax over the valid rows
    float amax = 0.0f;
    for (int i = threadIdx.x; i < r1 * (D / 8); i += kThreads) {
      float x[8];
      row8(i / (D / 8), i % (D / 8), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    }
    amax = block_max_256(amax, red);
    const float scale = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
    const float inv = amax == 0.0f ? 0.0f : __fdiv_rn(448.0f, amax);
    if (threadIdx.x == 0) scales[page * H + h] = scale;
    // codes: 8 values (one 16-byte bf16 vector) per thread per pass
    for (int i = threadIdx.x; i < ps * (D / 8); i += kThreads) {
      const int r = i / (D / 8), c = i % (D / 8);
      uint32_t dw[2] = {0u, 0u};             // codes 0..3, 4..7 (byte e of dw[e / 4])
      if (r < r1 && amax != 0.0f) {           // an all-zero block (-0 too) gets codes 0
        float x[8];
        row8(r, c, x);
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          dw[e >> 2] = e4m3x2_rne_sat<false>(x[e] * inv, x[e + 1] * inv, 0u);
          dw[e >> 2] = e4m3x2_rne_sat<true>(x[e + 2] * inv, x[e + 3] * inv, dw[e >> 2]);
        }
      }
      if (which == 0) {
        *reinterpret_cast<uint2*>(kp + (int64_t)r * D + c * 8) = make_uint2(dw[0], dw[1]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(c * 8 + e) * (ps + 4) + r] = (uint8_t)(dw[e >> 2] >> (8 * (e & 3)));
      }
    }
    if (which == 1) {
      __syncthreads();
      // write V^T rows: 16 slots (bytes) per store
      for (int i = threadIdx.x; i < D * (ps / 16); i += kThreads) {
        const int d = i / (ps / 16), c = i % (ps / 16);
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint8_t* s = &vt[d * (ps + 4) + c * 16 + 4 * e];
          w4[e] = s[0] | s[1] << 8 | s[2] << 16 | s[3] << 24;
        }
        *reinterpret_cast<u32x4*>(vp + (int64_t)d * ps + c * 16) = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_copy_t(const AppendArgs& a, hipStream_t s) {
  constexpr int E = 16 / (int)sizeof(T);
  constexpr int TPW = kCopyThreads / (D / E) * E;
  const int64_t lo = a.n0, hi = a.n0 + a.n_new;
  const int64_t g0 = (lo + E - 1) / E * E, g1 = hi / E * E;
  if (g1 > g0) {
    dim3 grid((unsigned)((g1 - g0 + TPW - 1) / TPW), (unsigned)a.n_heads);
    append_copy_kernel<T, D><<<grid, kCopyThreads, 0, s>>>(a, g0, g1);
  }
  const int64_t n_edge = g1 > g0 ? (g0 - lo) + (hi - g1) : a.n_new;
  if (n_edge > 0) {
    dim3 grid((unsigned)n_edge, (unsigned)a.n_heads);
    append_edge_kernel<T><<<grid, D, 0, s>>>(a, g0, g1);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_copy(const AppendArgs& a, int elem_bytes, hipStream_t s) {
  if (elem_bytes == 2) {
    switch (a.head_dim) {
      case 64: return launch_copy_t<uint16_t, 64>(a, s);
      case 128: return launch_copy_t<uint16_t, 128>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.head_dim) {
    case 32: return launch_copy_t<float, 32>(a, s);
    case 64: return launch_copy_t<float, 64>(a, s);
    case 128: return launch_copy_t<float, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t s) {
  const int ps = 1 << a.ps_log2;
  // logical pages from the one holding n0 to the one holding n0 + n_new - 1
  const int64_t npages = ((a.n0 & (ps - 1)) + a.n_new + ps - 1) / ps;
  dim3 grid((unsigned)npages, (unsigned)a.n_heads);
  if (a.head_dim != 128 || ps > 256) return hipErrorInvalidValue;
  append_fp8_kernel<128><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bca
