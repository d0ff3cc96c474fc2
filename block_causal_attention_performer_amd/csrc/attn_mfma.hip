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

#include "attn_common.h"

namespace bca {
namespace {

using namespace attn;

constexpr int BN = kKeyTile;      // keys per tile
constexpr int QW = 32;            // query rows per wave
constexpr int NW = 8;             // waves per workgroup (two groups of four)
constexpr int NT = NW * 64;
constexpr int GT = NT / 2;        // threads per group
constexpr int BM = NW * QW;       // query rows per workgroup
constexpr int NIF = 6;            // LDS reads kept in flight ahead of the MFMAs
static_assert(NW == kAttnFlagWaves, "one overflow flag per wave");

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

  // per-lane LDS read addresses (bytes): chunk j of the lane's row sits at
  // row_base + ((16 j) ^ x) with x = 16 (swizzle(row) ^ half) -- the lane's
  // half is the low bit of j.  A slot offset (a multiple of the 16 KB slot
  // size, above every in-slot bit) is folded into x by XOR once per tile;
  // +32 rows per MFMA row block is an immediate offset.
  const int kr = sigma32(col);
  const uint32_t krow = (uint32_t)(kr * D * 2), kx = (uint32_t)((swz<RK>(kr) ^ half) * 16);
  const uint32_t vrow = (uint32_t)(kr * BN * 2), vx = (uint32_t)((swz<8>(kr) ^ half) * 16);

  const int ps_log2 = a.ps_log2;
  const int psm = (1 << ps_log2) - 1;
  const uint8_t* kpages = static_cast<const uint8_t*>(a.k_pages);
  const uint8_t* vpages = static_cast<const uint8_t*>(a.v_pages);

  // ------------------------------------------------------------ tile staging
  // HBM -> registers -> LDS by one group (256 threads): group A stages K
  // tiles, group B V^T tiles.  Every tile is loaded by one sequence of
  // unconditional 16-byte loads (keys past n_kv read whatever their page
  // holds, or a clamped key on small pages) so the staging registers have a
  // single definition in the loop; the LDS store widens fp8 to bf16.
  u32x4 rg[TG];
  float sc_pend = 1.0f;      // fp8 scale of the staged tile
  int64_t k0_pend = 0;       // first key of the staged tile
  // per-lane byte offset of load 0 inside a tile; load i adds a uniform step
  static_assert(GT % KPR == 0 && GT % VPR == 0, "loads step by whole rows");
  const uint32_t goff = group_b ? (uint32_t)(((gt / VPR) << ps_log2) * EB + (gt % VPR) * 16)
                                : (uint32_t)((gt / KPR) * D * EB + (gt % KPR) * 16);
  const int64_t gstep = group_b ? ((int64_t)(GT / VPR) << ps_log2) * EB : (int64_t)(GT / KPR) * D * EB;
  const uint8_t* gpages = group_b ? vpages : kpages;
  const float* gscales = group_b ? a.v_scales : a.k_scales;
  auto load_tile = [&](int t) {
    const int64_t k0 = (int64_t)t * BN;
    k0_pend = k0;
    const int64_t page = page_of(a.page_table, k0 >> ps_log2);
    if constexpr (FP8) sc_pend = gscales[page * H + h];
    if constexpr (!SMALLPAGE) {
      // a whole tile lies in one page: uniform base, per-lane offsets
      const int64_t ph = page * H + h;
      const uint8_t* base = gpages + (group_b ? (((ph * D) << ps_log2) + (k0 & psm)) * EB
                                              : (((ph << ps_log2) | (k0 & psm)) * D) * EB);
#pragma unroll
      for (int i = 0; i < TG; ++i) rg[i] = ld16(base + i * gstep + goff);
    } else {
      // pages shorter than a tile: page per key (clamped to the last key)
#pragma unroll
      for (int i = 0; i < TG; ++i) {
        const int c = gt + i * GT;
        const int64_t key0 = group_b ? k0 + (c % VPR) * (16 / EB) : k0 + c / KPR;
        const int64_t key = key0 < a.n_kv ? key0 : a.n_kv - 1;
        const int64_t pg = a.page_table[key >> ps_log2];
        const int64_t off = group_b
            ? ((((pg * H + h) * D + c / VPR) << ps_log2) + (key & psm)) * EB
            : ((((pg * H + h) << ps_log2) | (key & psm)) * D) * EB + (c % KPR) * 16;
        rg[i] = ld16(gpages + off);
      }
    }
  };
  // K rows past n_kv are stored as loaded: their scores are replaced by
  // -inf in the softmax, whatever the row holds.  V values past n_kv are
  // zeroed (a zero weight times a non-finite value would not be zero).
  auto store_k = [&](uint16_t* kl) {
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = gt + i * GT;
      const int row = c / KPR, cc = c % KPR;
      const u32x4 v = rg[i];
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(kl + (row * RK + (cc ^ swz<RK>(row))) * 8) = v;
      } else {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint2 lo = fp8x4_to_bf16x4(v[2 * part]);
          const uint2 hi = fp8x4_to_bf16x4(v[2 * part + 1]);
          const int ch = 2 * cc + part;
          *reinterpret_cast<u32x4*>(kl + (row * RK + (ch ^ swz<RK>(row))) * 8) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
  };
  auto store_v = [&](uint16_t* vl) {
    const bool tail = k0_pend + BN > a.n_kv;
    constexpr int per = 16 / EB;             // keys per 16 bytes
    constexpr int kpw = 4 / EB;              // keys per 32-bit word
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = gt + i * GT;
      const int d = c / VPR, cc = c % VPR;
      u32x4 v = rg[i];
      if (tail) {
        const int64_t key = k0_pend + cc * per;
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int e = 0; e < kpw; ++e)
            if (key + w * kpw + e >= a.n_kv) v[w] &= ~(((1u << (8 * EB)) - 1) << (8 * EB * e));
      }
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(vl + (d * 8 + (cc ^ swz<8>(d))) * 8) = v;
      } else {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint2 lo = fp8x4_to_bf16x4(v[2 * part]);
          const uint2 hi = fp8x4_to_bf16x4(v[2 * part + 1]);
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
      load_tile(t0); store_k(lk);
      if (gt == 0) kscale[0] = sc_pend;
    } else {
      load_tile(t0); store_v(lv);
      // slot 2 stands for V(t0-1): zeros, so the first tile's PV step
      // (with P(t0-1) = 0) adds exact zeros whatever LDS held before
      if (gt == 0) vscale[0] = sc_pend;
#pragma unroll
      for (int i = 0; i < TG; ++i) rg[i] = u32x4{0, 0, 0, 0};
      store_v(lv + 2 * D * BN);
      load_tile(min(t0 + 1, t_end - 1)); store_v(lv + D * BN);
      if (gt == 0) vscale[1] = sc_pend;
    }
    // first staged loads of the loop: K(t0+1) by A, V(t0+2) by B.  Tile
    // indexes past the range are clamped to the last tile: the loop then
    // stages harmless duplicates into free slots instead of branching.
    const int tl = t_end - 1;
    load_tile(min(t0 + 1 + (int)group_b, tl));
    lds_barrier();
    if (group_b) lds_barrier();            // group B runs one phase behind

    bf16x8 pp[4];                          // P(t-1); P(t0-1) = 0
#pragma unroll
    for (int c = 0; c < 4; ++c) pp[c] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    int kslot = 0, vslot = 0;              // ring slots of tile t
    for (int t = t0; t < t_end; ++t) {
      const int vprev = vslot == 0 ? 2 : vslot - 1;
      // ---------------- matrix phase: S(t), then O += V(t-1)^T P(t-1)^T,
      // written as one software-pipelined stream: read j feeds MFMA j, and
      // read j + NIF is issued right after MFMA j; scheduling barriers keep
      // that order (the compiler would otherwise regroup the MFMAs and wait
      // for every outstanding read).
      f32x16 s[2];
      // priority to the wave in its matrix phase (the issue arbiter favours
      // older waves, which would put group B's MFMAs behind group A's softmax)
      __builtin_amdgcn_s_setprio(2);
      {
        uint32_t xk = kx ^ (uint32_t)(kslot * (BN * D * 2));
        uint32_t xv = vx ^ (uint32_t)(vprev * (D * BN * 2));
        asm volatile("" : "+v"(xk), "+v"(xv));   // per-tile values: keep the address math in the loop
        const char* kbase = reinterpret_cast<const char*>(lk) + krow;
        const char* vbase = reinterpret_cast<const char*>(lv) + vrow;
        constexpr int NK = 2 * KK;               // K reads / S MFMAs
        constexpr int NR = NK + 4 * DB;          // all reads (= MFMAs) of the phase
        auto rd = [&](int j) -> bf16x8 {
          if (j < NK) {
            const int kk = j >> 1, mb = j & 1;
            return __builtin_bit_cast(bf16x8, ld16(kbase + (((uint32_t)(32 * kk)) ^ xk) + mb * 32 * D * 2));
          }
          const int c = (j - NK) / DB, db = (j - NK) % DB;
          return __builtin_bit_cast(bf16x8, ld16(vbase + (((uint32_t)(32 * c)) ^ xv) + db * 32 * BN * 2));
        };
        bf16x8 fr[NR];
#pragma unroll
        for (int j = 0; j < NIF; ++j) fr[j] = rd(j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          if (j < NK) {
            const int kk = j >> 1, mb = j & 1;
            s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], qf[kk], kk == 0 ? f32x16{} : s[mb], 0, 0, 0);
          } else {
            const int c = (j - NK) / DB, db = (j - NK) % DB;
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], pp[c], o[db], 0, 0, 0);
          }
          if (j + NIF < NR) fr[j + NIF] = rd(j + NIF);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      const float ks = FP8 ? kscale[kslot] : 1.0f;
      const float vs = FP8 ? vscale[vslot] : 1.0f;
      lds_barrier();

      // ---------------- vector phase
      // staging first, so the LDS writes and the next loads overlap the
      // softmax: group A writes K(t+1) (slot kslot^1, which held K(t-1):
      // both groups read it before this phase) and loads K(t+2); group B
      // writes V(t+2) (slot of V(t-1)) and loads V(t+3)
      if (!group_b) {
        store_k(lk + (kslot ^ 1) * (BN * D));
        if (gt == 0) kscale[kslot ^ 1] = sc_pend;
      } else {
        store_v(lv + vprev * (D * BN));
        if (gt == 0) vscale[vprev] = sc_pend;
      }
      load_tile(min(t + 2 + (int)group_b, tl));
      // softmax of tile t -> P(t)
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
          // fp32 adds (v_dot2 would share the matrix pipe with the other
          // group's MFMAs)
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
      lds_barrier();
      kslot ^= 1;
      vslot = vslot == 2 ? 0 : vslot + 1;
    }
    // O += V(last)^T P(last)^T
    {
      const int vlast = vslot == 0 ? 2 : vslot - 1;
      const uint32_t xv = vx ^ (uint32_t)(vlast * (D * BN * 2));
      const char* vbase = reinterpret_cast<const char*>(lv) + vrow;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x8 vf[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
          vf[db] = __builtin_bit_cast(bf16x8, ld16(vbase + (((uint32_t)(32 * c)) ^ xv) + db * 32 * BN * 2));
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
    // the split's output normalised by its own row sum, in bf16; an empty
    // split stores zeros
    const int64_t prow = (int64_t)split * a.n_q + qrow;
    uint16_t* op = a.ws_o + (prow * H + h) * D;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const int d = 32 * db + 16 * run + 8 * half;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)(o[db][8 * run + e] * inv);
        *reinterpret_cast<bf16x8*>(op + d) = v;
      }
    if (half == 0) {
      float* ml = a.ws_ml + (prow * H + h) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

// Merge the NS partials of every (row, head) in split order:
// M = max m_s, O = sum 2^(m_s - M) O_s / sum 2^(m_s - M) l_s.
// 32 lanes per (row, head), D / 32 consecutive values each; the split count
// is a template argument, so every split's (m, l) and partial row are
// loaded at once.
template <int D, int NS>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int PER = D / 32;
  static_assert(PER == 2 || PER == 4, "head dim 64 or 128");
  using vec = float __attribute__((ext_vector_type(PER)));
  const int64_t item = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);   // (row, head)
  const int lane = threadIdx.x & 31;
  const int H = a.n_heads;
  if (item >= a.n_q * H) return;
  const int64_t stride = a.n_q * H;
  float2 ml[NS];
  vec os[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    ml[s] = *reinterpret_cast<const float2*>(a.ws_ml + (s * stride + item) * 2);
    const uint16_t* src = a.ws_o + (s * stride + item) * D + lane * PER;
    if constexpr (PER == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(src);
      os[s] = vec{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
    } else {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(src);
      os[s] = vec{__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u)};
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) M = fmaxf(M, ml[s].x);
  vec acc = {};
  float L = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    // partial s holds its output normalised by its row sum l: its weight
    // is l * 2^(m - M)
    const float w = ml[s].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[s].x - M) * ml[s].y;
    L += w;
    acc += w * os[s];
  }
  const float inv = 1.0f / L;
  const int64_t off = item * D + lane * PER;
  if (a.out_f32) {
    *reinterpret_cast<vec*>(static_cast<float*>(a.out) + off) = acc * inv;
  } else if constexpr (PER == 4) {
    uint2 u;
    u.x = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)});
    u.y = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(acc[2] * inv), (__bf16)(acc[3] * inv)});
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) = u;
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + off) =
        __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)});
  }
}


namespace {
template <int D, int NS>
hipError_t combine_ns(const AttnArgs& a, hipStream_t s) {
  if constexpr (NS > kMaxAttnSplit) {
    return hipErrorInvalidValue;
  } else {
    if (a.nsplit != NS) return combine_ns<D, NS + 1>(a, s);
    const unsigned cgrid = (unsigned)((a.n_q * a.n_heads + 7) / 8);
    attn_combine_kernel<D, NS><<<cgrid, 256, 0, s>>>(a);
    return hipGetLastError();
  }
}
}  // namespace

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s) {
  if (a.nsplit < 2 || a.nsplit > kMaxAttnSplit) return hipErrorInvalidValue;
  switch (a.head_dim) {
    case 64: return combine_ns<64, 2>(a, s);
    case 128: return combine_ns<128, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

namespace {
template <int D, bool FP8, bool SMALL>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const int64_t nqt = (a.n_q + BM - 1) / BM;
  const int64_t total = nqt * a.n_heads * a.nsplit;
  const unsigned grid = (unsigned)((total + 7) / 8 * 8);
  attn_fwd_kernel<D, FP8, SMALL><<<grid, NT, 0, s>>>(a);
  return hipGetLastError();
}
}  // namespace

int attn_mfma_rows_per_wg() { return BM; }

hipError_t launch_attn_mfma(const AttnArgs& a, bool kv_fp8, hipEvent_t main_done, hipStream_t s) {
  const bool small = a.ps_log2 < 6;
  hipError_t e;
  if (a.head_dim == 128 && !small && a.ps_log2 <= 20) {
    // direct HBM -> LDS tile loads (same query tiles, flags and partials)
    e = launch_attn_dma(a, kv_fp8, s);
  } else if (kv_fp8) {
    if (a.head_dim != 128 || small) return hipErrorInvalidValue;
    e = launch_t<128, true, false>(a, s);
  } else {
    switch (a.head_dim) {
      case 64: e = small ? launch_t<64, false, true>(a, s) : launch_t<64, false, false>(a, s); break;
      case 128: e = small ? launch_t<128, false, true>(a, s) : launch_t<128, false, false>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e == hipSuccess && main_done) e = hipEventRecord(main_done, s);
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_attn_combine(a, s);
}

}  // namespace bca
