// Block-causal attention over the paged KV cache, bf16 MFMA path (gfx950).
//
// Visibility (explainer "wan-streamer-realtime-av", listening-while-speaking
// section and its figure caption; youleyou.com article section 3.1): query
// at global position p sees key j iff j / B <= p / B.  For a query tile the
// key range splits into tiles that every row sees (no mask work), tiles that
// straddle the diagonal block or the n_kv tail (masked per element) and
// tiles no row sees (never visited).
//
// Kernel shape: one workgroup = 8 waves x 32 query rows of one head (two
// waves per SIMD); key tiles of 64.
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys on the MFMA rows, queries
//   on its columns, so a lane owns one query column and the row softmax
//   needs only one swap between the two 32-lane halves (v_permlane32_swap).
//   O^T += V^T P^T with the same MFMA: P^T is the S^T accumulator converted
//   to bf16 in place, because the key order on the MFMA rows is permuted
//   (sigma32) so that each lane half holds 8 consecutive keys per 16-key
//   chunk -- exactly the B-operand layout of the next MFMA.
//   K tiles are staged in LDS token-major, V tiles d-major (the cache stores
//   V d-major), both XOR-swizzled by row so 16-byte reads are conflict free.
//
// Ping-pong: the 8 waves form two groups (waves 0-3 and 4-7, one wave of
// each per SIMD); group B runs one phase behind group A (one extra barrier
// at the start), so on every SIMD one wave's matrix phase (S(t) = K(t) Q^T
// and O += V(t-1)^T P(t-1)^T) overlaps the other wave's vector phase
// (softmax of tile t).  Group A stages K tiles (2-slot ring), group B V^T
// tiles (3-slot ring), each loading one tile ahead into registers during its
// vector phase and writing them to LDS in the next.
//
// Softmax in base 2 against a fixed per-row reference m: m is the exact
// maximum of the row over the first key tile, and every later tile uses
// p = 2^(s*c - m) without taking a maximum.  That is exact (O / l does not
// depend on m) as long as nothing overflows; a tile whose row sum exceeds
// 2^40 (or is not finite) raises a flag for its query tile, and the
// exact-rescaling kernel recomputes every flagged query tile afterwards.
//
// Optional split of the key range (nsplit workgroups per query tile) writes
// unnormalised partials merged by a fixed-order log-sum-exp combine.
#include <math.h>

#include "bca_internal.h"

namespace bca {
namespace {

constexpr int BN = kKeyTile;      // keys per tile
constexpr int QW = 32;            // query rows per wave
constexpr int NW = 8;             // waves per workgroup (two groups of four)
constexpr int NT = NW * 64;
constexpr int GT = NT / 2;        // threads per group
constexpr int BM = NW * QW;       // query rows per workgroup
constexpr float kSlowSum = 1099511627776.0f;   // 2^40
static_assert(NW == kAttnFlagWaves, "one overflow flag per wave");

__device__ __forceinline__ int sigma32(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

// 16-byte chunk swizzle for LDS rows of R chunks (R = 8 or 16): the 8 (or
// 16) rows read by one group of lanes land in distinct banks.
template <int R>
__device__ __forceinline__ int swz(int row) {
  if constexpr (R == 16) {
    return (row & 3) | ((row >> 1) & 4) | ((row << 1) & 8);
  } else {
    return ((row >> 1) & 1) | ((row >> 2) & 2) | (((row ^ (row >> 2)) & 1) << 2);
  }
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// fp8 E4M3FN -> bf16 bits for 4 codes packed in a u32.  Exact (3 mantissa
// bits fit in bf16's 7; the E4M3 exponent range fits bf16's).
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  uint32_t a = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
  uint32_t b = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
  return make_uint2(a, b);
}

// Workgroup barrier that waits only for this wave's LDS traffic, not for
// global loads still in flight (they land in registers and are waited for
// at their use).  The asm clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unchanged
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int D, bool FP8, bool SMALLPAGE>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KK = D / 16;                 // k-steps of S^T
  constexpr int DB = D / 32;                 // head-dim blocks of O^T
  constexpr int RK = D / 8;                  // bf16 16-byte chunks per LDS K row
  constexpr int EB = FP8 ? 1 : 2;            // bytes per element in HBM
  constexpr int TG = BN * D * EB / 16 / GT;  // 16-byte global loads per group thread per tile
  constexpr int KPR = D * EB / 16;           // global loads per K row
  constexpr int VPR = BN * EB / 16;          // global loads per V^T row
  static_assert(TG >= 1, "tile too small");

  // LDS: K tiles in a 2-slot ring, V^T tiles in a 3-slot ring
  __shared__ __attribute__((aligned(16))) uint16_t lk[2 * BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t lv[3 * D * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= NW / 2;
  const int gt = tid & (GT - 1);             // thread index inside the group

  // XCD-aware mapping: hardware hands consecutive block ids to the 8 XCDs in
  // turn; give each XCD a contiguous run of (head, split, q-tile) ids so the
  // q-tiles of one head run side by side on one L2 and share its K/V tiles.
  const int G = gridDim.x;
  const int lid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int H = a.n_heads;
  const int nqt = (int)((a.n_q + BM - 1) / BM);
  if (lid >= nqt * H * a.nsplit) return;
  const int qt = lid % nqt;
  const int rest = lid / nqt;
  const int split = rest % a.nsplit;
  const int h = rest / a.nsplit;

  const int64_t B = a.block_size;
  const int64_t r0 = (int64_t)qt * BM;
  const int64_t rlast = (r0 + BM < a.n_q ? r0 + BM : a.n_q) - 1;
  const int64_t lim_first = min(a.n_kv, ((a.q_pos0 + r0) / B + 1) * B);
  const int64_t lim_last = min(a.n_kv, ((a.q_pos0 + rlast) / B + 1) * B);
  const int ntile = (int)((lim_last + BN - 1) / BN);
  const int t_begin = (int)((int64_t)split * ntile / a.nsplit);
  const int t_end = (int)((int64_t)(split + 1) * ntile / a.nsplit);

  const int64_t qrow = r0 + wave * QW + col;
  const int64_t lim = min(a.n_kv, ((a.q_pos0 + qrow) / B + 1) * B);

  // Q fragments (B operand of S^T = K Q^T): lane holds query column `col`,
  // head-dim elements 16*kk + 8*half .. +7.
  bf16x8 qf[KK];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow * H + h) * D + 8 * half;
    const bool ok = qrow < a.n_q;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(qp + 16 * kk) : u32x4{0, 0, 0, 0});
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  bool overflow = false;     // a tile exceeded the first tile's maximum by > 2^40

  // per-lane LDS read offsets (elements within one slot); +32 rows per MFMA
  // row block is a constant offset.
  const int kr = sigma32(col);
  int koff[KK], voff[4];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = kr * D + (((2 * kk + half) ^ swz<RK>(kr)) * 8);
#pragma unroll
  for (int c = 0; c < 4; ++c) voff[c] = kr * BN + (((2 * c + half) ^ swz<8>(kr)) * 8);

  const int ps_log2 = a.ps_log2;
  const int psm = (1 << ps_log2) - 1;
  const uint8_t* kpages = static_cast<const uint8_t*>(a.k_pages);
  const uint8_t* vpages = static_cast<const uint8_t*>(a.v_pages);

  // ------------------------------------------------------------ tile staging
  // HBM -> registers -> LDS by one group (256 threads); fp8 is widened to
  // bf16 and keys past n_kv are zeroed on the way.
  u32x4 rg[TG];
  float sc_pend = 1.0f;      // fp8 scale of the staged tile
  auto load_k = [&](int t) {
    const int64_t k0 = (int64_t)t * BN;
    if (!SMALLPAGE && k0 + BN <= a.n_kv) {
      const int64_t page = a.page_table[k0 >> ps_log2];
      const uint8_t* kb = kpages + ((((page * H + h) << ps_log2) | (k0 & psm)) * D) * EB;
#pragma unroll
      for (int i = 0; i < TG; ++i) {
        const int c = gt + i * GT;
        rg[i] = ld16(kb + (c / KPR) * D * EB + (c % KPR) * 16);
      }
      if constexpr (FP8) sc_pend = a.k_scales[page * H + h];
      return;
    }
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = gt + i * GT;
      const int64_t key = k0 + c / KPR;
      rg[i] = u32x4{0, 0, 0, 0};
      if (key < a.n_kv) {
        const int64_t page = a.page_table[key >> ps_log2];
        rg[i] = ld16(kpages + ((((page * H + h) << ps_log2) | (key & psm)) * D) * EB + (c % KPR) * 16);
      }
    }
    if constexpr (FP8) sc_pend = a.k_scales[a.page_table[k0 >> ps_log2] * H + h];
  };
  auto load_v = [&](int t) {
    const int64_t k0 = (int64_t)t * BN;
    constexpr int per = 16 / EB;             // keys per 16 bytes
    if (!SMALLPAGE && k0 + BN <= a.n_kv) {
      const int64_t page = a.page_table[k0 >> ps_log2];
      const uint8_t* vb = vpages + ((((page * H + h) * D) << ps_log2) + (k0 & psm)) * EB;
#pragma unroll
      for (int i = 0; i < TG; ++i) {
        const int c = gt + i * GT;
        rg[i] = ld16(vb + (((int64_t)(c / VPR)) << ps_log2) * EB + (c % VPR) * 16);
      }
      if constexpr (FP8) sc_pend = a.v_scales[page * H + h];
      return;
    }
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = gt + i * GT;
      const int d = c / VPR, cc = c % VPR;
      const int64_t key = k0 + cc * per;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (key < a.n_kv) {
        const int64_t page = a.page_table[key >> ps_log2];
        v = ld16(vpages + ((((page * H + h) * D + d) << ps_log2) + (key & psm)) * EB);
        if (key + per > a.n_kv) {
          // zero the values of keys past n_kv (they could hold anything)
          constexpr int kpw = 4 / EB;        // keys per 32-bit word
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int e = 0; e < kpw; ++e)
              if (key + w * kpw + e >= a.n_kv) v[w] &= ~(((1u << (8 * EB)) - 1) << (8 * EB * e));
        }
      }
      rg[i] = v;
    }
    if constexpr (FP8) sc_pend = a.v_scales[a.page_table[k0 >> ps_log2] * H + h];
  };
  auto store_k = [&](uint16_t* kl) {
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = gt + i * GT;
      const int row = c / KPR, cc = c % KPR;
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(kl + (row * RK + (cc ^ swz<RK>(row))) * 8) = rg[i];
      } else {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint2 lo = fp8x4_to_bf16x4(rg[i][2 * part]);
          const uint2 hi = fp8x4_to_bf16x4(rg[i][2 * part + 1]);
          const int ch = 2 * cc + part;
          *reinterpret_cast<u32x4*>(kl + (row * RK + (ch ^ swz<RK>(row))) * 8) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
  };
  auto store_v = [&](uint16_t* vl) {
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = gt + i * GT;
      const int d = c / VPR, cc = c % VPR;
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(vl + (d * 8 + (cc ^ swz<8>(d))) * 8) = rg[i];
      } else {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint2 lo = fp8x4_to_bf16x4(rg[i][2 * part]);
          const uint2 hi = fp8x4_to_bf16x4(rg[i][2 * part + 1]);
          const int ch = 2 * cc + part;
          *reinterpret_cast<u32x4*>(vl + (d * 8 + (ch ^ swz<8>(d))) * 8) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
  };
  // fp8 scales by ring slot (written to a small LDS table by the group that
  // stages the tile, read by every wave)
  __shared__ float kscale[2], vscale[3];

  // ------------------------------------------------------------ main loop
  if (t_begin < t_end) {
    const int t0 = t_begin;
    // prologue (synchronous): K(t0) by group A; V(t0), V(t0+1) by group B
    if (!group_b) {
      load_k(t0); store_k(lk);
      if (gt == 0) kscale[0] = sc_pend;
    } else {
      load_v(t0); store_v(lv);
      if (gt == 0) vscale[0] = sc_pend;
      if (t0 + 1 < t_end) {
        load_v(t0 + 1); store_v(lv + D * BN);
        if (gt == 0) vscale[1] = sc_pend;
      }
    }
    // first staged loads of the loop: K(t0+1) by A, V(t0+2) by B
    if (!group_b) { if (t0 + 1 < t_end) load_k(t0 + 1); }
    else { if (t0 + 2 < t_end) load_v(t0 + 2); }
    lds_barrier();
    if (group_b) lds_barrier();            // group B runs one phase behind

    bf16x8 pp[4];                          // P(t-1)
    int kslot = 0, vslot = 0;              // ring slots of tile t
    for (int t = t0; t < t_end; ++t) {
      const int vprev = vslot == 0 ? 2 : vslot - 1;
      // ---------------- matrix phase: S(t), then O += V(t-1)^T P(t-1)^T
      f32x16 s[2];
      {
        const uint16_t* kl = lk + kslot * (BN * D);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          bf16x8 kf[2];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) kf[mb] = __builtin_bit_cast(bf16x8, ld16(kl + koff[kk] + mb * 32 * D));
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mb], qf[kk], kk == 0 ? f32x16{} : s[mb], 0, 0, 0);
        }
        // keep four LDS reads in flight ahead of the MFMAs that consume them
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * KK - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      if (t > t0) {
        const uint16_t* vl = lv + vprev * (D * BN);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8 vf[DB];
#pragma unroll
          for (int db = 0; db < DB; ++db) vf[db] = __builtin_bit_cast(bf16x8, ld16(vl + voff[c] + db * 32 * BN));
#pragma unroll
          for (int db = 0; db < DB; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pp[c], o[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4 * DB - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      const float ks = FP8 ? kscale[kslot] : 1.0f;
      const float vs = FP8 ? vscale[vslot] : 1.0f;
      lds_barrier();

      // ---------------- vector phase: softmax of tile t -> P(t)
      {
        const int64_t k0 = (int64_t)t * BN;
        if (k0 + BN > lim_first) {
          const int lrel = (int)min(lim - k0, (int64_t)BN);   // keys of this tile the row sees
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = 32 * mb + 16 * (r >> 3) + 8 * half + (r & 7);
              if (key >= lrel) s[mb][r] = -INFINITY;
            }
        }
        const float sl = FP8 ? a.scale_log2 * ks : a.scale_log2;
        if (t == t0) {
          // first tile: the row maximum becomes the fixed reference
          float mx = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
          m_run = pair_max(mx) * sl;
        }
        const float mneg = -m_run;
        float part[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int mb = c >> 1, rb = 8 * (c & 1);
          float acc = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][rb + e], sl, mneg));
            acc += p;
            if constexpr (FP8) p *= vs;
            pp[c][e] = (__bf16)p;
          }
          part[c] = acc;
        }
        const float tsum = (part[0] + part[1]) + (part[2] + part[3]);
        overflow |= !(tsum <= kSlowSum);
        l_run += tsum;
      }
      // staging: group A writes K(t+1) (slot kslot^1, which held K(t-1)) and
      // loads K(t+2); group B writes V(t+2) (slot of V(t-1)) and loads V(t+3)
      if (!group_b) {
        if (t + 1 < t_end) {
          store_k(lk + (kslot ^ 1) * (BN * D));
          if (gt == 0) kscale[kslot ^ 1] = sc_pend;
          if (t + 2 < t_end) load_k(t + 2);
        }
      } else {
        if (t + 2 < t_end) {
          store_v(lv + vprev * (D * BN));
          if (gt == 0) vscale[vprev] = sc_pend;
          if (t + 3 < t_end) load_v(t + 3);
        }
      }
      lds_barrier();
      kslot ^= 1;
      vslot = vslot == 2 ? 0 : vslot + 1;
    }
    // O += V(last)^T P(last)^T
    {
      const int vlast = vslot == 0 ? 2 : vslot - 1;
      const uint16_t* vl = lv + vlast * (D * BN);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x8 vf[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[db] = __builtin_bit_cast(bf16x8, ld16(vl + voff[c] + db * 32 * BN));
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pp[c], o[db], 0, 0, 0);
      }
    }
    if (!group_b) lds_barrier();           // balance group B's extra barrier
  }

  // one flag per (query tile, split, wave), written unconditionally
  const bool wave_overflow = __builtin_amdgcn_ballot_w64(overflow) != 0;
  if (lane == 0) a.flags_out[((int64_t)(h * nqt + qt) * a.nsplit + split) * NW + wave] = wave_overflow;
  if (wave_overflow) {
    // the exact kernel rewrites this query tile; keep the partials finite
    m_run = 0.0f;
    l_run = 1.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  }

  // ---------------- epilogue: lane owns query `col` and head dims
  // 32*db + 8*half + [0,8) (regs 0..7) and +16 (regs 8..15).
  const float l_tot = pair_sum(l_run);
  if (qrow >= a.n_q) return;
  if (a.nsplit == 1) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const int d = 32 * db + 16 * run + 8 * half;
        const int64_t off = (qrow * H + h) * D + d;
        if (a.out_f32) {
          float* op = static_cast<float*>(a.out) + off;
          f32x4 x0, x1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0[e] = o[db][8 * run + e] * inv;
            x1[e] = o[db][8 * run + 4 + e] * inv;
          }
          *reinterpret_cast<f32x4*>(op) = x0;
          *reinterpret_cast<f32x4*>(op + 4) = x1;
        } else {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)(o[db][8 * run + e] * inv);
          *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(a.out) + off) = v;
        }
      }
    }
  } else {
    const int64_t prow = (int64_t)split * a.n_q + qrow;
    float* op = a.ws_o + (prow * H + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const int d = 32 * db + 16 * run + 8 * half;
        f32x4 x0, x1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x0[e] = o[db][8 * run + e];
          x1[e] = o[db][8 * run + 4 + e];
        }
        *reinterpret_cast<f32x4*>(op + d) = x0;
        *reinterpret_cast<f32x4*>(op + d + 4) = x1;
      }
    if (half == 0) {
      float* ml = a.ws_ml + (prow * H + h) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

// Merge the nsplit partials of every (row, head) in split order:
// M = max m_s, O = sum 2^(m_s - M) O_s / sum 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (row, head)
  const int lane = threadIdx.x & 63;
  const int H = a.n_heads;
  if (item >= a.n_q * H) return;
  const int64_t stride = a.n_q * H;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_ml[(s * stride + item) * 2]);
  constexpr int PER = D / 64;
  float acc[PER > 0 ? PER : 1] = {};
  float L = 0.0f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = a.ws_ml[(s * stride + item) * 2];
    const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
    L += w * a.ws_ml[(s * stride + item) * 2 + 1];
    const float* op = a.ws_o + (s * stride + item) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += w * op[lane * PER + e];
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int64_t off = item * D + lane * PER + e;
    if (a.out_f32) static_cast<float*>(a.out)[off] = acc[e] * inv;
    else reinterpret_cast<__bf16*>(a.out)[off] = (__bf16)(acc[e] * inv);
  }
}

namespace {
template <int D, bool FP8, bool SMALL>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const int64_t nqt = (a.n_q + BM - 1) / BM;
  const int64_t total = nqt * a.n_heads * a.nsplit;
  const unsigned grid = (unsigned)((total + 7) / 8 * 8);
  attn_fwd_kernel<D, FP8, SMALL><<<grid, NT, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const unsigned cgrid = (unsigned)((a.n_q * a.n_heads + 3) / 4);
  attn_combine_kernel<D><<<cgrid, 256, 0, s>>>(a);
  return hipGetLastError();
}
}  // namespace

int attn_mfma_rows_per_wg() { return BM; }

hipError_t launch_attn_mfma(const AttnArgs& a, bool kv_fp8, hipStream_t s) {
  const bool small = a.ps_log2 < 6;
  if (kv_fp8) {
    if (a.head_dim != 128 || small) return hipErrorInvalidValue;
    return launch_t<128, true, false>(a, s);
  }
  switch (a.head_dim) {
    case 64: return small ? launch_t<64, false, true>(a, s) : launch_t<64, false, false>(a, s);
    case 128: return small ? launch_t<128, false, true>(a, s) : launch_t<128, false, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bca
