// Block-causal attention, exact-rescaling variant of the bf16 MFMA path.
//
// Same math and layouts as the fast kernel (attn_mfma.hip); the softmax keeps
// a per-row running maximum that is refreshed (with O and l rescaled)
// whenever a tile's maximum exceeds it by more than 2^8, so it handles any
// logit range.  It runs when no workspace is given, and after the fast
// kernel for the query tiles the fast kernel flagged (a later key tile
// exceeding the first tile's maximum by more than 2^40).
//
// Visibility (explainer "wan-streamer-realtime-av", listening-while-speaking
// section and its figure caption; youleyou.com article section 3.1): query
// at global position p sees key j iff j / B <= p / B.  For a query tile the
// key range splits into tiles that every row sees (no mask work), tiles that
// straddle the diagonal block or the n_kv tail (masked per element) and
// tiles no row sees (never visited).
//
// Kernel shape (one workgroup = NW waves = NW*QW query rows of one head):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys on the MFMA rows, queries
//   on its columns, so a lane owns one query column and the row softmax
//   needs only one swap between the two 32-lane halves (v_permlane32_swap).
//   O^T += V^T P^T with the same MFMA: P^T is the S^T accumulator converted
//   to bf16 in place, because the key order on the MFMA rows is permuted
//   (sigma32) so that each lane half holds 8 consecutive keys per 16-key
//   chunk -- exactly the B-operand layout of the next MFMA.
//   K tiles are staged in LDS token-major, V tiles d-major (the cache stores
//   V d-major), both XOR-swizzled by row so 16-byte reads are conflict free.
//   Online softmax in base 2 with lazy rescaling: the running max is only
//   moved when a tile's max exceeds it by more than 2^8, so O and l are
//   rescaled rarely; the final O / l is exact either way.
//   Optional split of the key range (nsplit workgroups per query tile)
//   writes unnormalised partials merged by a fixed-order log-sum-exp
//   combine.
#include <math.h>

#include "attn_common.h"

namespace bca {
namespace {

using namespace attn;

constexpr int BN = kKeyTile;
constexpr float kRescaleLog2 = 8.0f;

template <int D, int NT, bool FP8>
struct TileLoader {
  // bf16 pages: K tile = BN rows x D (16-byte chunks), V^T tile = D rows x BN.
  // fp8 pages: same tiles at one byte per element, widened to bf16 on store.
  static constexpr int EB = FP8 ? 1 : 2;                 // bytes per element in HBM
  static constexpr int KCH = BN * D * EB / 16 / NT;      // 16-byte loads per thread, K
  static constexpr int VCH = D * BN * EB / 16 / NT;      // 16-byte loads per thread, V
  static constexpr int KPR = D * EB / 16;                // loads per K row
  static constexpr int VPR = BN * EB / 16;               // loads per V^T row
  u32x4 k[KCH];
  u32x4 v[VCH];
};

}  // namespace

template <int D, int QW, int NW, bool FP8, bool SMALLPAGE>
__global__ __launch_bounds__(NW * 64, 1) void attn_exact_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * QW;
  constexpr int NB = QW / 32;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int RK = D / 8;                  // bf16 16-byte chunks per LDS K row
  using TL = TileLoader<D, NT, FP8>;
  static_assert(TL::KCH >= 1 && TL::VCH >= 1, "tile too small for the workgroup");

  __shared__ __attribute__((aligned(16))) uint16_t lk[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t lv[2][D * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;

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
  if (a.flags) {
    // rerun only the query tiles the fast kernel flagged (its tiles have the
    // same rows: 256 per workgroup); at most kMaxAttnSplit x kAttnFlagWaves
    // = 64 flags, one per lane, so every wave reaches the same verdict
    static_assert(kMaxAttnSplit * kAttnFlagWaves <= 64, "one flag per lane");
    const int32_t* f = a.flags + (int64_t)(h * nqt + qt) * a.flag_splits * kAttnFlagWaves;
    const int fl = lane < a.flag_splits * kAttnFlagWaves ? f[lane] : 0;
    if (__builtin_amdgcn_ballot_w64(fl != 0) == 0) return;
  }

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

  // Q fragments (B operand of S^T = K Q^T): lane holds query column `col`,
  // head-dim elements 16*kk + 8*half .. +7.
  bf16x8 qf[NB][KK];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bool ok = qrow[nb] < a.n_q;
      const uint16_t* qp = q + (qrow[nb] * H + h) * D + 8 * half;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4 v = ok ? ld16(qp + 16 * kk) : u32x4{0, 0, 0, 0};
        qf[nb][kk] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  f32x16 o[DB][NB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][nb][r] = 0.0f;
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { m_run[nb] = -INFINITY; l_run[nb] = 0.0f; }

  const int ps_log2 = a.ps_log2;
  const int psm = (1 << ps_log2) - 1;
  const uint8_t* kpages = static_cast<const uint8_t*>(a.k_pages);
  const uint8_t* vpages = static_cast<const uint8_t*>(a.v_pages);
  TL pre;
  float ks_next = 1.0f, vs_next = 1.0f;

  // ---- global -> registers for key tile t
  auto load_tile = [&](int t) {
    const int64_t k0 = (int64_t)t * BN;
    const bool tail = k0 + BN > a.n_kv;
    if constexpr (!SMALLPAGE) {
      const int64_t page = a.page_table[k0 >> ps_log2];
      const int64_t slot0 = k0 & psm;
      const uint8_t* kb = kpages + ((((page * H + h) << ps_log2) | slot0) * D) * TL::EB;
      const uint8_t* vb = vpages + ((((page * H + h) * D) << ps_log2) + slot0) * TL::EB;
      if constexpr (FP8) {
        ks_next = a.k_scales[page * H + h];
        vs_next = a.v_scales[page * H + h];
      }
#pragma unroll
      for (int i = 0; i < TL::KCH; ++i) {
        const int c = tid + i * NT;
        const int row = c / TL::KPR, cc = c % TL::KPR;
        pre.k[i] = (!tail || k0 + row < a.n_kv) ? ld16(kb + (row * D * TL::EB) + cc * 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < TL::VCH; ++i) {
        const int c = tid + i * NT;
        const int d = c / TL::VPR, cc = c % TL::VPR;
        u32x4 v = ld16(vb + ((int64_t)d << ps_log2) * TL::EB + cc * 16);
        if (tail) {
          // zero the values of keys past n_kv (they could hold anything)
          const int per = 16 / TL::EB;                 // keys per 16 bytes
          const int64_t kfirst = k0 + cc * per;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t word = v[w];
            const int kpw = 4 / TL::EB;                // keys per word
#pragma unroll
            for (int e = 0; e < kpw; ++e)
              if (kfirst + w * kpw + e >= a.n_kv) word &= ~(((1u << (8 * TL::EB)) - 1) << (8 * TL::EB * e));
            v[w] = word;
          }
        }
        pre.v[i] = v;
      }
    } else {
      // pages shorter than a tile (bf16 only): look the page up per row / run
#pragma unroll
      for (int i = 0; i < TL::KCH; ++i) {
        const int c = tid + i * NT;
        const int row = c / TL::KPR, cc = c % TL::KPR;
        const int64_t key = k0 + row;
        if (key < a.n_kv) {
          const int64_t page = a.page_table[key >> ps_log2];
          pre.k[i] = ld16(kpages + ((((page * H + h) << ps_log2) | (key & psm)) * D) * 2 + cc * 16);
        } else {
          pre.k[i] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int i = 0; i < TL::VCH; ++i) {
        const int c = tid + i * NT;
        const int d = c / TL::VPR, cc = c % TL::VPR;
        const int64_t key = k0 + cc * 8;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (key < a.n_kv) {
          const int64_t page = a.page_table[key >> ps_log2];
          v = ld16(vpages + ((((page * H + h) * D + d) << ps_log2) + (key & psm)) * 2);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if (key + 2 * w >= a.n_kv) v[w] = 0;
            else if (key + 2 * w + 1 >= a.n_kv) v[w] &= 0xFFFFu;
          }
        }
        pre.v[i] = v;
      }
    }
  };

  // ---- registers -> LDS buffer (bf16, swizzled)
  auto store_tile = [&](int buf) {
    uint16_t* kl = lk[buf];
    uint16_t* vl = lv[buf];
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < TL::KCH; ++i) {
        const int c = tid + i * NT;
        const int row = c / RK, cc = c % RK;
        *reinterpret_cast<u32x4*>(kl + (row * RK + (cc ^ swz<RK>(row))) * 8) = pre.k[i];
      }
#pragma unroll
      for (int i = 0; i < TL::VCH; ++i) {
        const int c = tid + i * NT;
        const int d = c / 8, cc = c % 8;
        *reinterpret_cast<u32x4*>(vl + (d * 8 + (cc ^ swz<8>(d))) * 8) = pre.v[i];
      }
    } else {
      // one 16-byte fp8 load = 16 elements = two bf16 chunks
#pragma unroll
      for (int i = 0; i < TL::KCH; ++i) {
        const int c = tid + i * NT;
        const int row = c / TL::KPR, cc = c % TL::KPR;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint2 lo = fp8x4_to_bf16x4(pre.k[i][2 * part]);
          const uint2 hi = fp8x4_to_bf16x4(pre.k[i][2 * part + 1]);
          const int ch = 2 * cc + part;
          *reinterpret_cast<u32x4*>(kl + (row * RK + (ch ^ swz<RK>(row))) * 8) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
#pragma unroll
      for (int i = 0; i < TL::VCH; ++i) {
        const int c = tid + i * NT;
        const int d = c / TL::VPR, cc = c % TL::VPR;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const uint2 lo = fp8x4_to_bf16x4(pre.v[i][2 * part]);
          const uint2 hi = fp8x4_to_bf16x4(pre.v[i][2 * part + 1]);
          const int ch = 2 * cc + part;
          *reinterpret_cast<u32x4*>(vl + (d * 8 + (ch ^ swz<8>(d))) * 8) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
  };

  float ks_cur = 1.0f, vs_cur = 1.0f;
  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
    ks_cur = ks_next;
    vs_cur = vs_next;
    __syncthreads();
  }

  const int krow0 = sigma32(col);            // MFMA row -> tile row (keys / head dims)

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) load_tile(t + 1);

    // ---------------- S^T = K Q^T  (rows: 64 keys in two 32-row blocks)
    f32x16 s[2][NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][nb][r] = 0.0f;
    const uint16_t* kl = lk[buf];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 kf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * mb + krow0;
        const int ch = 2 * kk + half;
        kf[mb] = __builtin_bit_cast(bf16x8, ld16(kl + (row * RK + (ch ^ swz<RK>(row))) * 8));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mb], qf[nb][kk], s[mb][nb], 0, 0, 0);
    }

    // ---------------- mask (diagonal block / n_kv tail only)
    const int64_t k0 = (int64_t)t * BN;
    if (k0 + BN > lim_first) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lrel = (int)min(lim[nb] - k0, (int64_t)BN);   // keys of this tile the row sees
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * mb + 16 * (r >> 3) + 8 * half + (r & 7);
            if (key >= lrel) s[mb][nb][r] = -INFINITY;
          }
      }
    }

    // ---------------- online softmax (base 2, lazy rescale)
    const float sl = FP8 ? a.scale_log2 * ks_cur : a.scale_log2;
    float mt[NB];
    bool grow = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][nb][r]);
      mt[nb] = pair_max(mx) * sl;
      grow |= mt[nb] > m_run[nb] + kRescaleLog2;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float mn = fmaxf(m_run[nb], mt[nb]);
        const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[nb] - mn);
        m_run[nb] = mn;
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][nb][r] *= alpha;
      }
    }
    bf16x8 pb[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float mu = m_run[nb] == -INFINITY ? 0.0f : m_run[nb];
      float lsum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][nb][8 * c2 + e], sl, -mu));
            lsum += p[e];
            if constexpr (FP8) p[e] *= vs_cur;
          }
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)p[e];
          pb[nb][2 * mb + c2] = v;
        }
      }
      l_run[nb] += lsum;
    }

    // ---------------- O^T += V^T P^T  (rows: head dims in 32-row blocks)
    const uint16_t* vl = lv[buf];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 vf[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + krow0;
        const int ch = 2 * c + half;
        vf[db] = __builtin_bit_cast(bf16x8, ld16(vl + (d * 8 + (ch ^ swz<8>(d))) * 8));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pb[nb][c], o[db][nb], 0, 0, 0);
    }

    if (more) {
      store_tile(buf ^ 1);
      ks_cur = ks_next;
      vs_cur = vs_next;
    }
    __syncthreads();
  }

  // ---------------- epilogue: lane owns query `col` of each 32-block and
  // head dims 32*db + 8*half + [0,8) (regs 0..7) and +16 (regs 8..15).
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l_tot = pair_sum(l_run[nb]);
    if (qrow[nb] >= a.n_q) continue;
    if (a.nsplit == 1) {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          const int d = 32 * db + 16 * run + 8 * half;
          const int64_t off = (qrow[nb] * H + h) * D + d;
          if (a.out_f32) {
            float* op = static_cast<float*>(a.out) + off;
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x0[e] = o[db][nb][8 * run + e] * inv;
              x1[e] = o[db][nb][8 * run + 4 + e] * inv;
            }
            *reinterpret_cast<f32x4*>(op) = x0;
            *reinterpret_cast<f32x4*>(op + 4) = x1;
          } else {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)(o[db][nb][8 * run + e] * inv);
            *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(a.out) + off) = v;
          }
        }
      }
    } else {
      // normalised by the split's row sum, in bf16, as the merge reads it
      const int64_t prow = (int64_t)split * a.n_q + qrow[nb];
      uint16_t* op = a.ws_o + (prow * H + h) * D;
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          const int d = 32 * db + 16 * run + 8 * half;
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)(o[db][nb][8 * run + e] * inv);
          *reinterpret_cast<bf16x8*>(op + d) = v;
        }
      if (half == 0) {
        float* ml = a.ws_ml + (prow * H + h) * 2;
        ml[0] = m_run[nb];
        ml[1] = l_tot;
      }
    }
  }
}

namespace {
constexpr int kExactQW = 32;   // query rows per wave
constexpr int kExactNW = 8;    // waves per workgroup (256 rows, as the fast kernel)

template <int D, bool FP8, bool SMALL>
hipError_t launch_exact_t(const AttnArgs& a, hipStream_t s) {
  constexpr int BM = kExactQW * kExactNW;
  const int64_t nqt = (a.n_q + BM - 1) / BM;
  const int64_t total = nqt * a.n_heads * a.nsplit;
  const unsigned grid = (unsigned)((total + 7) / 8 * 8);
  attn_exact_kernel<D, kExactQW, kExactNW, FP8, SMALL><<<grid, kExactNW * 64, 0, s>>>(a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_exact(const AttnArgs& a, bool kv_fp8, hipStream_t s) {
  const bool small = a.ps_log2 < 6;
  if (kv_fp8) {
    if (a.head_dim != 128 || small) return hipErrorInvalidValue;
    return launch_exact_t<128, true, false>(a, s);
  }
  switch (a.head_dim) {
    case 64: return small ? launch_exact_t<64, false, true>(a, s) : launch_exact_t<64, false, false>(a, s);
    case 128: return small ? launch_exact_t<128, false, true>(a, s) : launch_exact_t<128, false, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bca
