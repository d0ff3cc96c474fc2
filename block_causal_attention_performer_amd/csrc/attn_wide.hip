// Block-causal attention over the paged KV cache: bf16 / fp8 MFMA kernel
// with 64 query rows per wave (gfx950, head dim 128, pages of >= 64 keys).
//
// Visibility (explainer "wan-streamer-realtime-av", listening-while-speaking
// section and its figure caption; youleyou.com article section 3.1): query
// at global position p sees key j iff j / B <= p / B.
//
// Kernel shape: one workgroup = 4 waves (one per SIMD) x 64 query rows of
// one head; 64-key tiles; v_mfma_f32_32x32x16_bf16 throughout.
//   S^T = K Q^T: keys on the MFMA rows (permuted by sigma32), the wave's 64
//   queries on two 32-column blocks, Q held in registers for the whole
//   kernel.  Every K fragment read from LDS feeds two MFMAs (both query
//   blocks), and so does every V^T fragment of O^T += V^T P^T: half the LDS
//   bytes per MFMA of a 32-row wave.
//   With one wave per SIMD the matrix cores are kept busy from inside the
//   wave: the MFMAs of S(t+1) are interleaved with the softmax of tile t
//   (exp/convert/sum on the vector ALUs), then O += V(t)^T P(t)^T.
//
// Pipeline, one barrier per key tile.  LDS holds two K slots and two V^T
// slots.  Iteration t (all four waves alike):
//   1. store the staged K(t+2) into K(t)'s slot and V(t+1) into V(t-1)'s
//      slot (both free: read before the previous barrier);
//   2. load K(t+3), V(t+2) from HBM into the staging registers;
//   3. S(t+1) = K(t+1) Q^T interleaved with softmax(S(t)) -> P(t);
//   4. O += V(t)^T P(t)^T;  barrier.
// Tile indexes past the range are clamped to the last tile (duplicate
// stores into free slots instead of branches).
//
// Softmax in base 2 against a fixed per-row reference m (the exact maximum
// of the row over the first key tile); later tiles use p = 2^(s*c - m)
// without a running maximum.  O / l does not depend on m, so this is exact
// unless something overflows: a tile row sum above 2^40 (or not finite)
// raises the query tile's flag and the exact-rescaling kernel recomputes
// every flagged query tile afterwards.  Row sums add the bf16 weights the
// PV product uses (v_dot2_f32_bf16).
//
// Optional split of the key range (nsplit workgroups per query tile) writes
// unnormalised partials merged by the fixed-order log-sum-exp combine.
#include <math.h>

#include "attn_common.h"

namespace bca {
namespace {

using namespace attn;

constexpr int BN = kKeyTile;      // keys per tile
constexpr int QW = 64;            // query rows per wave
constexpr int NB = QW / 32;       // 32-column MFMA blocks per wave
constexpr int NW = 4;             // waves per workgroup, one per SIMD
constexpr int NT = NW * 64;
constexpr int BM = NW * QW;       // query rows per workgroup
static_assert(NW * NB == kAttnFlagWaves, "flag slots per (query tile, split)");

}  // namespace

template <int D, bool FP8>
__global__ __launch_bounds__(NT, 1) void attn_wide_kernel(AttnArgs a) {
  constexpr int KK = D / 16;                 // k-steps of S^T
  constexpr int DB = D / 32;                 // head-dim blocks of O^T
  constexpr int RK = D / 8;                  // bf16 16-byte chunks per LDS K row
  constexpr int EB = FP8 ? 1 : 2;            // bytes per element in HBM
  constexpr int TG = BN * D * EB / 16 / NT;  // 16-byte loads per thread per tile (K or V)
  constexpr int KPR = D * EB / 16;           // loads per K row
  constexpr int VPR = BN * EB / 16;          // loads per V^T row
  static_assert(TG >= 1 && NT % KPR == 0 && NT % VPR == 0, "tile staging shape");

  __shared__ __attribute__((aligned(16))) uint16_t lk[2 * BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t lv[2 * D * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware mapping (consecutive block ids go to the 8 XCDs in turn; each
  // XCD gets a contiguous run of (head, split, q-tile) ids).
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

  int64_t qrow[NB], lim[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    qrow[nb] = r0 + wave * QW + nb * 32 + col;
    lim[nb] = min(a.n_kv, ((a.q_pos0 + qrow[nb]) / B + 1) * B);
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds query column `col` of
  // block nb, head-dim elements 16*kk + 8*half .. +7.
  bf16x8 qf[NB][KK];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow[nb] * H + h) * D + 8 * half;
    const bool ok = qrow[nb] < a.n_q;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[nb][kk] = __builtin_bit_cast(bf16x8, ok ? ld16(qp + 16 * kk) : u32x4{0, 0, 0, 0});
  }

  f32x16 o[NB][DB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[nb][db] = f32x16{};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { m_run[nb] = -INFINITY; l_run[nb] = 0.0f; }
  bool overflow = false;

  // per-lane LDS read addresses (bytes): chunk j of the lane's row is at
  // row + ((16 j) ^ x); a slot offset (a multiple of the 16 KB slot) is
  // folded into x by XOR; +32 rows per MFMA row block is an immediate.
  const int kr = sigma32(col);
  const uint32_t krow = (uint32_t)(kr * D * 2), kx = (uint32_t)((swz<RK>(kr) ^ half) * 16);
  const uint32_t vrow = (uint32_t)(kr * BN * 2), vx = (uint32_t)((swz<8>(kr) ^ half) * 16);
  const char* lkb = reinterpret_cast<const char*>(lk) + krow;
  const char* lvb = reinterpret_cast<const char*>(lv) + vrow;
  constexpr uint32_t SLOT = BN * D * 2;      // bytes per K or V^T slot

  const int ps_log2 = a.ps_log2;
  const int psm = (1 << ps_log2) - 1;
  const uint8_t* kpages = static_cast<const uint8_t*>(a.k_pages);
  const uint8_t* vpages = static_cast<const uint8_t*>(a.v_pages);

  // ------------------------------------------------------------ staging
  // Every thread moves TG 16-byte chunks of a K tile and TG of a V^T tile;
  // a whole tile lies in one page, so load i is base + i * step + goff.
  u32x4 rk[TG], rv[TG];
  float ksc_pend = 1.0f, vsc_pend = 1.0f;
  int64_t vk0_pend = 0;
  const uint32_t kgoff = (uint32_t)((tid / KPR) * D * EB + (tid % KPR) * 16);
  const uint32_t vgoff = (uint32_t)(((tid / VPR) << ps_log2) * EB + (tid % VPR) * 16);
  const int64_t kstep = (int64_t)(NT / KPR) * D * EB;
  const int64_t vstep = ((int64_t)(NT / VPR) << ps_log2) * EB;
  auto load_k = [&](int t) {
    const int64_t k0 = (int64_t)t * BN;
    const int64_t page = page_of(a.page_table, k0 >> ps_log2);
    if constexpr (FP8) ksc_pend = a.k_scales[page * H + h];
    const uint8_t* base = kpages + ((((page * H + h) << ps_log2) | (k0 & psm)) * D) * EB;
#pragma unroll
    for (int i = 0; i < TG; ++i) rk[i] = ld16(base + i * kstep + kgoff);
  };
  auto load_v = [&](int t) {
    const int64_t k0 = (int64_t)t * BN;
    vk0_pend = k0;
    const int64_t page = page_of(a.page_table, k0 >> ps_log2);
    if constexpr (FP8) vsc_pend = a.v_scales[page * H + h];
    const uint8_t* base = vpages + ((((page * H + h) * D) << ps_log2) + (k0 & psm)) * EB;
#pragma unroll
    for (int i = 0; i < TG; ++i) rv[i] = ld16(base + i * vstep + vgoff);
  };
  // K rows past n_kv are stored as loaded (their scores become -inf); V
  // values past n_kv are zeroed (a zero weight times a non-finite value is
  // not zero).
  auto store_k = [&](int slot) {
    uint16_t* kl = lk + slot * (BN * D);
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = tid + i * NT;
      const int row = c / KPR, cc = c % KPR;
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(kl + (row * RK + (cc ^ swz<RK>(row))) * 8) = rk[i];
      } else {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint2 lo = fp8x4_to_bf16x4(rk[i][2 * part]);
          const uint2 hi = fp8x4_to_bf16x4(rk[i][2 * part + 1]);
          const int ch = 2 * cc + part;
          *reinterpret_cast<u32x4*>(kl + (row * RK + (ch ^ swz<RK>(row))) * 8) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
  };
  auto store_v = [&](int slot) {
    uint16_t* vl = lv + slot * (D * BN);
    const bool tail = vk0_pend + BN > a.n_kv;
    constexpr int per = 16 / EB;             // keys per 16 bytes
    constexpr int kpw = 4 / EB;              // keys per 32-bit word
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int c = tid + i * NT;
      const int d = c / VPR, cc = c % VPR;
      u32x4 v = rv[i];
      if (tail) {
        const int64_t key = vk0_pend + cc * per;
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

  // ------------------------------------------------------------ compute pieces
  // K fragment kk, row block mb of the K tile in slot ks
  auto rd_k = [&](uint32_t xk, int kk, int mb) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, ld16(lkb + (((uint32_t)(32 * kk)) ^ xk) + mb * 32 * D * 2));
  };
  auto rd_v = [&](uint32_t xv, int c, int db) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, ld16(lvb + (((uint32_t)(32 * c)) ^ xv) + db * 32 * BN * 2));
  };
  // mask the keys of tile t that a row does not see (uniform test first)
  auto mask = [&](f32x16 (&s)[2][NB], int t) {
    const int64_t k0 = (int64_t)t * BN;
    if (k0 + BN > lim_first) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lrel = (int)min(lim[nb] - k0, (int64_t)BN);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * mb + 16 * (r >> 3) + 8 * half + (r & 7);
            if (key >= lrel) s[mb][nb][r] = -INFINITY;
          }
      }
    }
  };
  // ------------------------------------------------------------ main loop
  if (t_begin < t_end) {
    const int t0 = t_begin, tl = t_end - 1;
    // prologue: K(t0) into K slot 0; V slot 1 stands for V(t0-1) and holds
    // zeros, P(t0-1) = 0, so the first PV step adds exact zeros; then the
    // loads the first iteration stores (K(t0+1), V(t0))
    load_k(t0);
    store_k(0);
    float ks_cur = ksc_pend;                 // scale of K(t0) (fp8)
#pragma unroll
    for (int i = 0; i < TG; ++i) rv[i] = u32x4{0, 0, 0, 0};
    vk0_pend = 0;
    store_v(1);
    load_k(min(t0 + 1, tl));
    load_v(t0);
    lds_barrier();

    bf16x8 pa[NB][4], pb[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < 4; ++c) pa[nb][c] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});

    // iteration t: S(t); softmax(S(t)) -> p_cur interleaved with
    // O += V(t-1)^T p_prev^T
    auto iter = [&](int t, bf16x8 (&p_prev)[NB][4], bf16x8 (&p_cur)[NB][4]) {
      const int kslot = (t - t0) & 1;        // K(t) and (after step 1) V(t) slot
      // 1. staged K(t+1) -> K(t-1)'s slot, V(t) -> V(t-2)'s slot; their fp8
      //    scales stay in registers (every thread loaded them)
      store_k(kslot ^ 1);
      store_v(kslot);
      const float ks_next = ksc_pend;        // K(t+1)
      const float vs_t = vsc_pend;           // V(t), folded into P(t)
      // 2. next loads
      load_k(min(t + 2, tl));
      load_v(min(t + 1, tl));
      const float ks = ks_cur;
      // 3. S(t) = K(t) Q^T, reads NIF ahead of the MFMAs
      f32x16 s[2][NB];
      {
        uint32_t xk = kx ^ (uint32_t)(kslot * SLOT);
        asm volatile("" : "+v"(xk));
        constexpr int NR = 2 * KK;
        constexpr int NIF = 6;
        bf16x8 fr[NR];
#pragma unroll
        for (int j = 0; j < NIF; ++j) fr[j] = rd_k(xk, j >> 1, j & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          const int kk = j >> 1, mb = j & 1;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], qf[nb][kk], kk == 0 ? f32x16{} : s[mb][nb], 0, 0, 0);
          if (j + NIF < NR) fr[j + NIF] = rd_k(xk, (j + NIF) >> 1, (j + NIF) & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      mask(s, t);
      const float sl = a.scale_log2 * ks;
      if (t == t0) {
        // first tile: the row maximum becomes the fixed reference
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float mx = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][nb][r]);
          m_run[nb] = pair_max(mx) * sl;
        }
      }
      // 4. softmax(S(t)) -> p_cur, interleaved with O += V(t-1)^T p_prev^T
      float part[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float mneg = -m_run[nb];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int mb = c >> 1, rb = 8 * (c & 1);
          float acc = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][nb][rb + e], sl, mneg));
            if constexpr (FP8) {
              acc += p;
              p *= vs_t;
            }
            p_cur[nb][c][e] = (__bf16)p;
          }
          if constexpr (!FP8) {
            const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const bf16x2 pr = {p_cur[nb][c][e], p_cur[nb][c][e + 1]};
              acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
            }
          }
          part[nb][c] = acc;
        }
      }
      {
        uint32_t xv = vx ^ (uint32_t)((kslot ^ 1) * SLOT);
        asm volatile("" : "+v"(xv));
        bf16x8 vf[4][DB];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int db = 0; db < DB; ++db) vf[c][db] = rd_v(xv, c, db);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              o[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c][db], p_prev[nb][c], o[nb][db], 0, 0, 0);
        // schedule: 3 V reads ahead; per MFMA a share of the softmax
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int j = 0; j < 4 * DB; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
          if (j + 3 < 4 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float tsum = (part[nb][0] + part[nb][1]) + (part[nb][2] + part[nb][3]);
        overflow |= !(tsum <= kSlowSum);
        l_run[nb] += tsum;
      }
      ks_cur = ks_next;
      lds_barrier();
    };

    int t = t0;
    for (; t + 1 <= tl; t += 2) {
      iter(t, pa, pb);
      iter(t + 1, pb, pa);
    }
    if (t <= tl) iter(t, pa, pb);
    // O += V(tl)^T P(tl)^T (V(tl) was stored in the last iteration)
    {
      const bool in_pb = ((tl - t0) & 1) == 0; // an odd number of iterations ends writing pb
      const int vslot = (tl - t0) & 1;
      uint32_t xv = vx ^ (uint32_t)(vslot * SLOT);
      asm volatile("" : "+v"(xv));
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vf = rd_v(xv, c, db);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            o[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, in_pb ? pb[nb][c] : pa[nb][c], o[nb][db], 0, 0, 0);
        }
    }
  }

  // flags: the wave's slot pair of its (query tile, split), written unconditionally
  const bool wave_overflow = __builtin_amdgcn_ballot_w64(overflow) != 0;
  if (lane < NB)
    a.flags_out[((int64_t)(h * nqt + qt) * a.nsplit + split) * kAttnFlagWaves + wave * NB + lane] = wave_overflow;
  if (wave_overflow) {
    // the exact kernel rewrites this query tile; keep the partials finite
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = 0.0f;
      l_run[nb] = 1.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[nb][db] = f32x16{};
    }
  }

  // ---------------- epilogue: lane owns query `col` of each block and head
  // dims 32*db + 8*half + [0,8) (regs 0..7) and +16 (regs 8..15).
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l_tot = pair_sum(l_run[nb]);
    if (qrow[nb] >= a.n_q) continue;
    if (a.nsplit == 1) {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          const int d = 32 * db + 16 * run + 8 * half;
          const int64_t off = (qrow[nb] * H + h) * D + d;
          if (a.out_f32) {
            float* op = static_cast<float*>(a.out) + off;
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x0[e] = o[nb][db][8 * run + e] * inv;
              x1[e] = o[nb][db][8 * run + 4 + e] * inv;
            }
            *reinterpret_cast<f32x4*>(op) = x0;
            *reinterpret_cast<f32x4*>(op + 4) = x1;
          } else {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)(o[nb][db][8 * run + e] * inv);
            *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(a.out) + off) = v;
          }
        }
    } else {
      const int64_t prow = (int64_t)split * a.n_q + qrow[nb];
      float* op = a.ws_o + (prow * H + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          const int d = 32 * db + 16 * run + 8 * half;
          f32x4 x0, x1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0[e] = o[nb][db][8 * run + e];
            x1[e] = o[nb][db][8 * run + 4 + e];
          }
          *reinterpret_cast<f32x4*>(op + d) = x0;
          *reinterpret_cast<f32x4*>(op + d + 4) = x1;
        }
      if (half == 0) {
        float* ml = a.ws_ml + (prow * H + h) * 2;
        ml[0] = m_run[nb];
        ml[1] = l_tot;
      }
    }
  }
}

hipError_t launch_attn_wide(const AttnArgs& a, bool kv_fp8, hipStream_t s) {
  if (a.head_dim != 128 || a.ps_log2 < 6) return hipErrorInvalidValue;
  const int64_t nqt = (a.n_q + BM - 1) / BM;
  const int64_t total = nqt * a.n_heads * a.nsplit;
  const unsigned grid = (unsigned)((total + 7) / 8 * 8);
  if (kv_fp8) attn_wide_kernel<128, true><<<grid, NT, 0, s>>>(a);
  else attn_wide_kernel<128, false><<<grid, NT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bca
