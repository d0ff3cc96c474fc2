// kv_append kernels: write a unit's K/V slice into the paged cache.
//
// The performer appends every received KV slice to its own full-history
// cache (deep read "全双工语音模型精读⑫：Wan-Streamer", section 4, step 3).
// K pages are token-major [page][h][slot][d]; V pages are d-major
// [page][h][d][slot] so that the attention kernel reads 16-byte runs along
// the key axis.  Both copies are pure data movement (HBM bound): every
// workgroup moves one 64-token logical chunk of one head.
#include "bca_internal.h"

namespace bca {
namespace {

constexpr int kChunk = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ int64_t page_slot_offset(const int32_t* pt, int64_t t,
                                                    int ps_log2, int h, int H,
                                                    int row_elems) {
  // element offset of (token t, head h) row start in a [page][h][ps][row] array
  const int64_t page = pt[t >> ps_log2];
  const int64_t slot = t & ((1 << ps_log2) - 1);
  return ((page * H + h) << ps_log2 | slot) * (int64_t)row_elems;
}

// T: element type (uint16_t for bf16, float for f32); D: head dim.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void append_copy_kernel(AppendArgs a) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte vector
  constexpr int RV = D / E;                  // 16-byte vectors per K row
  constexpr int LD = D + 4 / sizeof(T);      // LDS row pitch (+4 bytes: spreads banks)
  __shared__ T tile[kChunk * LD];

  const int h = blockIdx.y;
  const int H = a.n_heads;
  const int64_t base = (a.n0 & ~(int64_t)(kChunk - 1)) + (int64_t)blockIdx.x * kChunk;
  const int64_t lo = a.n0, hi = a.n0 + a.n_new;
  const T* kin = static_cast<const T*>(a.k_new);
  const T* vin = static_cast<const T*>(a.v_new);
  T* kp = static_cast<T*>(a.k_pages);
  T* vp = static_cast<T*>(a.v_pages);

  // K rows: straight copy, one 16-byte vector per thread per pass.
  for (int i = threadIdx.x; i < kChunk * RV; i += kThreads) {
    const int r = i / RV, c = i % RV;
    const int64_t t = base + r;
    if (t < lo || t >= hi) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(kin + ((t - lo) * H + h) * D + c * E);
    *reinterpret_cast<u32x4*>(kp + page_slot_offset(a.page_table, t, a.ps_log2, h, H, D) + c * E) = v;
  }
  // V rows into LDS (rows outside the slice are never written out).
  for (int i = threadIdx.x; i < kChunk * RV; i += kThreads) {
    const int r = i / RV, c = i % RV;
    const int64_t t = base + r;
    if (t < lo || t >= hi) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(vin + ((t - lo) * H + h) * D + c * E);
    const T* pv = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int e = 0; e < E; ++e) tile[r * LD + c * E + e] = pv[e];
  }
  __syncthreads();
  // V^T: for each d, E consecutive tokens form one 16-byte run of a page row.
  constexpr int RUNS = kChunk / E;           // runs per d-row of the chunk
  const int ps = 1 << a.ps_log2;
  for (int i = threadIdx.x; i < D * RUNS; i += kThreads) {
    const int d = i / RUNS, run = i % RUNS;
    const int64_t t0 = base + run * E;
    if (t0 + E <= lo || t0 >= hi) continue;
    // E tokens never straddle a page (page_size >= 16 >= E)
    const int64_t page = a.page_table[t0 >> a.ps_log2];
    const int64_t slot = t0 & (ps - 1);
    T* dst = vp + (((page * H + h) * D + d) << a.ps_log2) + slot;
    if (t0 >= lo && t0 + E <= hi) {
      T buf[E];
#pragma unroll
      for (int e = 0; e < E; ++e) buf[e] = tile[(run * E + e) * LD + d];
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(buf);
    } else {
      for (int e = 0; e < E; ++e) {
        const int64_t t = t0 + e;
        if (t >= lo && t < hi) dst[e] = tile[(run * E + e) * LD + d];
      }
    }
  }
}

// ------------------------------------------------------------------ fp8

// Round-to-nearest-even onto the finite OCP E4M3FN values, saturating at
// 448 (OCP 8-bit floating point spec: bias 7, 3 mantissa bits, subnormal
// quantum 2^-9, S.1111.111 reserved for NaN).  Sign copied from x.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  if (a < 0x1p-6f) {
    // subnormal range: code = round-half-even(a / 2^-9); a * 512 is exact
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  const uint32_t b = __float_as_uint(a);
  const uint32_t m = b & 0x7FFFFFu;
  uint32_t keep = m >> 20;
  const uint32_t rem = m & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
  uint32_t e = (b >> 23) - 127 + 7;
  if (keep == 8) { keep = 0; ++e; }
  return sign | (e << 3) | keep;
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

// One workgroup per (logical page touched, head).  Rows of the page that
// the slice covers are [r0, r1); the page starts fresh (appends to an fp8
// cache start at a page boundary), rows past r1 get code 0.
template <int D>
__global__ __launch_bounds__(kThreads) void append_fp8_kernel(AppendArgs a) {
  const int ps = 1 << a.ps_log2;
  const int h = blockIdx.y;
  const int H = a.n_heads;
  const int64_t lp = (a.n0 >> a.ps_log2) + blockIdx.x;
  const int64_t t0 = lp << a.ps_log2;
  const int64_t r1l = a.n0 + a.n_new - t0;
  const int r1 = (int)(r1l < ps ? r1l : ps);
  const int64_t page = a.page_table[lp];
  const uint16_t* src_k = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* src_v = static_cast<const uint16_t*>(a.v_new);
  uint8_t* kp = static_cast<uint8_t*>(a.k_pages) + ((page * H + h) << a.ps_log2) * D;
  uint8_t* vp = static_cast<uint8_t*>(a.v_pages) + ((page * H + h) << a.ps_log2) * D;
  __shared__ float red[4];
  __shared__ uint8_t vt[D * 260];   // V^T codes staged [d][slot], pitch ps+4 (ps <= 256)

  for (int which = 0; which < 2; ++which) {
    const uint16_t* src = which == 0 ? src_k : src_v;
    // amax over the valid rows
    float amax = 0.0f;
    for (int i = threadIdx.x; i < r1 * (D / 8); i += kThreads) {
      const int r = i / (D / 8), c = i % (D / 8);
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + ((t0 - a.n0 + r) * H + h) * D + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(__uint_as_float(v[e] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(v[e] & 0xFFFF0000u)));
      }
    }
    amax = block_max_256(amax, red);
    const float scale = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
    const float inv = amax == 0.0f ? 0.0f : __fdiv_rn(448.0f, amax);
    if (threadIdx.x == 0) {
      float* sc = which == 0 ? a.k_scales : a.v_scales;
      sc[page * H + h] = scale;
    }
    // codes: 8 values (one 16-byte bf16 vector) per thread per pass
    for (int i = threadIdx.x; i < ps * (D / 8); i += kThreads) {
      const int r = i / (D / 8), c = i % (D / 8);
      uint32_t code[8];
      if (r < r1) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + ((t0 - a.n0 + r) * H + h) * D + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          code[2 * e] = e4m3_rne_sat(__uint_as_float(v[e] << 16) * inv);
          code[2 * e + 1] = e4m3_rne_sat(__uint_as_float(v[e] & 0xFFFF0000u) * inv);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) code[e] = 0;
      }
      if (which == 0) {
        uint32_t lo = code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24;
        uint32_t hi = code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24;
        *reinterpret_cast<uint2*>(kp + (int64_t)r * D + c * 8) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(c * 8 + e) * (ps + 4) + r] = (uint8_t)code[e];
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

}  // namespace

hipError_t launch_append_copy(const AppendArgs& a, int elem_bytes, hipStream_t s) {
  const int64_t first = a.n0 & ~(int64_t)(kChunk - 1);
  const int64_t nchunks = (a.n0 + a.n_new - first + kChunk - 1) / kChunk;
  dim3 grid((unsigned)nchunks, (unsigned)a.n_heads);
  if (elem_bytes == 2) {
    switch (a.head_dim) {
      case 64: append_copy_kernel<uint16_t, 64><<<grid, kThreads, 0, s>>>(a); break;
      case 128: append_copy_kernel<uint16_t, 128><<<grid, kThreads, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.head_dim) {
      case 32: append_copy_kernel<float, 32><<<grid, kThreads, 0, s>>>(a); break;
      case 64: append_copy_kernel<float, 64><<<grid, kThreads, 0, s>>>(a); break;
      case 128: append_copy_kernel<float, 128><<<grid, kThreads, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t s) {
  const int ps = 1 << a.ps_log2;
  const int64_t npages = (a.n_new + ps - 1) / ps;   // n0 is page aligned
  dim3 grid((unsigned)npages, (unsigned)a.n_heads);
  if (a.head_dim != 128 || ps > 256) return hipErrorInvalidValue;
  append_fp8_kernel<128><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bca
