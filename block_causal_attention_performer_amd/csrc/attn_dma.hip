// Block-causal attention over the paged KV cache: MFMA kernel whose K / V^T
// tiles move HBM -> LDS by direct 16-byte LDS loads (gfx950
// buffer_load_dwordx4 ... lds), head dim 128, pages of >= 64 keys; bf16
// pages, or fp8 pages with S on the fp8 MFMA and PV in bf16.
//
// Visibility (explainer "wan-streamer-realtime-av", listening-while-speaking
// section and its figure caption; youleyou.com article section 3.1): query
// at global position p sees key j iff j / B <= p / B.
//
// Compute is that of the register-staged kernel (attn_mfma.hip): one
// workgroup = 8 waves x 32 query rows of one head, two wave groups in
// opposite phases so one group's MFMAs (S(t) = K(t) Q^T, O += V(t-1)^T
// P(t-1)^T) overlap the other's softmax; the fixed-reference base-2 softmax
// with an overflow flag and the exact kernel as fallback; split partials.
//
// Staging: group A streams K tiles, group B V^T tiles, straight into LDS.
// A direct LDS load writes lane i's 16 bytes at (wave-uniform base) + 16 i,
// so each lane fetches the global chunk that the XOR-swizzled LDS layout
// wants at its position.  Each ring slot is a separate LDS array and the
// loop is unrolled by the ring length, so every slot is named at compile
// time: reads of one slot never wait for loads into another.  A group waits
// for its own loads of a tile (vmcnt) before the barrier that publishes it.
// V values of keys past n_kv are zeroed in LDS after they land (tail tile
// only).  bf16 pages: rings of four slots and one barrier per key tile (a
// barrier between the two phases cost more in waiting than the skew it
// removed); fp8 pages: rings of three slots, a barrier after each phase,
// and V^T widened to bf16 in LDS by group B between the MFMAs of its matrix
// phase, where the conversions take issue slots the MFMA chains leave free
// (at the end of the phase they lengthened it by ~7%).
//
// The loads use the buffer (MUBUF) form with a per-tile descriptor, not the
// global (FLAT-encoded) form: the compiler treats a FLAT direct load in
// flight as a possible LDS access of unknown order and then drains every
// LDS read before each use (lgkmcnt(0) every few MFMAs of the matrix
// phase), while a buffer load counts on vmcnt only and the matrix phase
// keeps three reads in flight.
//
// Scheduling: one persistent workgroup per CU takes (query tile, split,
// head) items from per-XCD work queues in the workspace (its own XCD's
// first, then the others), and the key-range splits are cut 2 : ... : 2 : 1
// so short items come last.  With one workgroup per item the launch ended
// when the slowest XCD's share did (XCDs differ by several percent in
// speed under this load) and the last round of items left CUs idle.
#include <math.h>

#include <algorithm>
#include <type_traits>

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
constexpr int NIF = 4;            // LDS reads kept in flight ahead of the MFMAs
// fp8 matrix phase: the step at which group B's V^T widening starts, and
// the steps between its parts (0/2, 1/3, 1/6, 3/2 and 5/4 timed within 1%)
constexpr int kWidenAt = 1;
constexpr int kWidenStep = 3;
static_assert(NW == kAttnFlagWaves, "one overflow flag per wave");

template <int N>
using ic = std::integral_constant<int, N>;

typedef __attribute__((address_space(3))) void* lds_ptr;

// s_waitcnt with only vmcnt = n (lgkmcnt and expcnt left alone)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

}  // namespace

template <int D, bool FP8>
__global__ __launch_bounds__(NT, 1) void attn_dma_kernel(AttnArgs a) {
  constexpr int KK = D / 16;                 // k-steps of S^T
  constexpr int DB = D / 32;                 // head-dim blocks of O^T
  constexpr int RK = D / 8;                  // 16-byte chunks per LDS K row
  constexpr int SLOT = BN * D * 2;           // bytes per K or V^T slot
  constexpr int NL = SLOT / (GT * 16);       // direct loads per thread per tile
  static_assert(NL == 4 && RK == 16, "staging layout assumes D = 128");
  // fp8 cache: tiles of 1-byte codes land in their own rings; K is read
  // from its ring by the fp8 MFMA, V^T is widened into the bf16 slots by
  // group B
  constexpr int SLOT8 = FP8 ? BN * D : 16;   // bytes per fp8 K or V^T slot
  constexpr int NL8 = FP8 ? SLOT8 / (GT * 16) : 1;
  static_assert(!FP8 || NL8 == 2, "the fp8 widening runs in two parts");

  // bf16: four-slot K and V^T rings; fp8: three-slot bf16 V^T ring (K is
  // read from the fp8 ring), so its fourth slots and the bf16 K slots are
  // never referenced and take no LDS
  __shared__ __attribute__((aligned(1024))) char lk0[SLOT], lk1[SLOT], lk2[SLOT], lk3[SLOT];
  __shared__ __attribute__((aligned(1024))) char lv0[SLOT], lv1[SLOT], lv2[SLOT], lv3[SLOT];
  __shared__ __attribute__((aligned(16))) char fk0[SLOT8], fk1[SLOT8], fk2[SLOT8];
  __shared__ __attribute__((aligned(16))) char fv0[SLOT8], fv1[SLOT8], fv2[SLOT8];
  __shared__ float scl[2][3];                // fp8: K and V scale of the tile in each slot
  auto kslot = [&](auto r) -> char* {
    constexpr int i = decltype(r)::value & 3;
    if constexpr (i == 0) return lk0;
    else if constexpr (i == 1) return lk1;
    else if constexpr (i == 2) return lk2;
    else return lk3;
  };
  auto vslot = [&](auto r) -> char* {
    constexpr int i = decltype(r)::value & 3;
    if constexpr (i == 0) return lv0;
    else if constexpr (i == 1) return lv1;
    else if constexpr (i == 2) return lv2;
    else return lv3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= NW / 2;
  const int gw = wave & 3;                   // wave index inside its group
  auto k8slot = [&](auto r) -> char* {       // fp8 K ring (read by both groups)
    constexpr int i = decltype(r)::value % 3;
    if constexpr (i == 0) return fk0;
    else if constexpr (i == 1) return fk1;
    else return fk2;
  };
  auto fslot = [&](auto r) -> char* {        // fp8 ring of this thread's group
    constexpr int i = decltype(r)::value % 3;
    if constexpr (i == 0) return group_b ? fv0 : fk0;
    else if constexpr (i == 1) return group_b ? fv1 : fk1;
    else return group_b ? fv2 : fk2;
  };

  const int H = a.n_heads;
  const int nqt = (int)((a.n_q + BM - 1) / BM);

  // ------------------------------------------------------------ work queues
  // One queue per XCD holds the items of its share of the heads, every first
  // split before every second split and so on (query tiles of one head and
  // split next to each other, so they stream the same K/V through that
  // XCD's L2 together).  A persistent workgroup takes items from the queue
  // of the XCD it runs on and, once that is empty, from the others: the
  // launch ends when the last item does, whatever speed each XCD runs at.
  // Thread 0 (group A) claims the next item as soon as its own part of the
  // current one is done, while group B still runs its last phase; claiming
  // any earlier would hold items back from CUs that fall idle at the end.
  auto heads_lo = [&](int x) { return (x * H + kAttnQueues - 1) / kAttnQueues; };
  auto qlen = [&](int x) { return (heads_lo(x + 1) - heads_lo(x)) * nqt * a.nsplit; };
  __shared__ int item_sh[2];
  int cur_q = (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (31 << 11)) & (kAttnQueues - 1));
  uint32_t dead = 0;                         // thread 0: queues found empty
  // item from claim pv of queue cur_q, else from the other queues; -1 when all are empty
  auto settle = [&](int pv) -> int {
    if (pv < qlen(cur_q)) return (cur_q << 24) | pv;
    dead |= 1u << cur_q;
    for (int k = 1; k < kAttnQueues; ++k) {
      const int x = (cur_q + k) & (kAttnQueues - 1);
      if ((dead >> x) & 1) continue;
      const int n = qlen(x);
      const int v = n > 0 ? atomicAdd(a.sched + x, 1) : 0;
      if (v < n) {
        cur_q = x;
        return (x << 24) | v;
      }
      dead |= 1u << x;
    }
    return -1;
  };

  // one (query tile, key-range split, head) item; thread 0 leaves the next
  // item in item_sh[nxt]
  auto work = [&](const int qt, const int split, const int h, const int nxt) {
  const int64_t B = a.block_size;
  const int64_t r0 = (int64_t)qt * BM;
  const int64_t rlast = (r0 + BM < a.n_q ? r0 + BM : a.n_q) - 1;
  const int64_t lim_first = min(a.n_kv, ((a.q_pos0 + r0) / B + 1) * B);
  const int64_t lim_last = min(a.n_kv, ((a.q_pos0 + rlast) / B + 1) * B);
  const int ntile = (int)((lim_last + BN - 1) / BN);
  // splits in the ratio 2 : 2 : ... : 2 : 1: the last split's items are
  // half as long and fill the end of the launch (2 : 1 measured best
  // among 1 : 1, 3 : 2, 2 : 1, 5 : 2, 3 : 1, 4 : 1 and 8 : 1)
  const int wsum = 2 * (a.nsplit - 1) + 1;
  const int t_begin = (int)((int64_t)ntile * (2 * split) / wsum);
  const int t_end = split + 1 == a.nsplit ? ntile : (int)((int64_t)ntile * (2 * split + 2) / wsum);

  const int64_t qrow = r0 + wave * QW + col;
  const int64_t lim = min(a.n_kv, ((a.q_pos0 + qrow) / B + 1) * B);
  // a wave whose rows all lie past n_q (the ragged last query tile) keeps
  // staging its share of the tiles and meeting the barriers but computes
  // nothing: its SIMD partner then runs its phases uncontended
  const bool idle = r0 + wave * QW >= a.n_q;

  bf16x8 qf[KK];
  // fp8 cache: S = K Q^T runs on the fp8 MFMA with the K codes as they lie
  // in LDS and Q as two E4M3 terms on one scale per query row,
  // Q = qs (hi + lo) with hi = E4M3(Q/qs), lo = E4M3(Q/qs - hi), qs =
  // amax/448: as accurate as the bf16 Q itself.  Lane (half, col) holds
  // dims 64 kk + 32 half + [0, 32) of query col, the B operand of
  // v_mfma_scale_f32_32x32x64_f8f6f4 (its K fragments cover the same dims
  // in the same byte order).
  i32x8 qh[2], ql[2];
  float qs = 1.0f;
  if constexpr (!FP8) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow * H + h) * D + 8 * half;
    const bool ok = qrow < a.n_q;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(qp + 16 * kk) : u32x4{0, 0, 0, 0});
  } else {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow * H + h) * D + 32 * half;
    const bool ok = qrow < a.n_q;
    u32x4 qv[2][4];
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        qv[kk][p] = ok ? ld16(qp + 64 * kk + 8 * p) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < 4; ++w)
          amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(qv[kk][p][w] << 16)),
                                   fabsf(__uint_as_float(qv[kk][p][w] & 0xFFFF0000u))));
      }
    amax = pair_max(amax);
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    qs = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {     // 4 dims per code word
          const uint32_t u0 = qv[kk][p][2 * w2], u1 = qv[kk][p][2 * w2 + 1];
          const float y0 = __uint_as_float(u0 << 16) * inv, y1 = __uint_as_float(u0 & 0xFFFF0000u) * inv;
          const float y2 = __uint_as_float(u1 << 16) * inv, y3 = __uint_as_float(u1 & 0xFFFF0000u) * inv;
          int hw = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
          hw = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, hw, true);
          const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
          const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
          int lw = __builtin_amdgcn_cvt_pk_fp8_f32(y0 - d01[0], y1 - d01[1], 0, false);
          lw = __builtin_amdgcn_cvt_pk_fp8_f32(y2 - d23[0], y3 - d23[1], lw, true);
          qh[kk][2 * p + w2] = hw;
          ql[kk][2 * p + w2] = lw;
        }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  bool overflow = false;
  // bf16: running row sums of the lane's keys, one per 16-key chunk of a
  // tile, added up once at the end of the item
  float lc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  // per-lane LDS read addresses: chunk j of the lane's row at row + ((16 j) ^ x)
  const int kr = sigma32(col);
  const uint32_t krow = (uint32_t)(kr * D * 2), kx = (uint32_t)((swz<RK>(kr) ^ half) * 16);
  const uint32_t vrow = (uint32_t)(kr * BN * 2), vx = (uint32_t)((swz<8>(kr) ^ half) * 16);
  // fp8 K rows of 128 bytes: lane reads chunks 4 kk + 2 half (+1) of row kr
  const uint32_t krow8 = (uint32_t)(kr * 128), kx8 = (uint32_t)(((2 * half) ^ swz<8>(kr)) * 16);

  const int ps_log2 = a.ps_log2;
  const int psm = (1 << ps_log2) - 1;
  const char* kpages = static_cast<const char*>(a.k_pages);
  const char* vpages = static_cast<const char*>(a.v_pages);

  // ------------------------------------------------------------ staging
  // Direct load i of wave gw writes LDS bytes [i*4096 + gw*1024, +1024) of
  // the slot.  K: 4 rows of 256 bytes, lane -> row 16i + 4gw + lane/16,
  // position lane%16, global chunk position ^ swz16(row).  V^T: 8 rows of
  // 128 bytes, lane -> head dim 32i + 8gw + lane/8, position lane%8, global
  // chunk position ^ swz8(d).  The swizzles depend on the row's low 4 bits
  // only, so load i is the lane offset of load 0 plus a uniform step.
  uint32_t goff;
  int64_t gstep;
  if (!group_b) {
    const int row = 4 * gw + (lane >> 4);
    goff = (uint32_t)(row * 256 + (((lane & 15) ^ swz<16>(row)) * 16));
    gstep = 16 * 256;
  } else {
    const int d = 8 * gw + (lane >> 3);
    goff = (uint32_t)(((int64_t)d << ps_log2) * 2 + (((lane & 7) ^ swz<8>(d)) * 16));
    gstep = (int64_t)32 << ps_log2 << 1;
  }
  // issue the direct loads of tile t (K for group A, V^T for group B) into
  // `dst`.  K and V^T pages have the same size; a tile of K starts 2 D bytes
  // per key into its page, a tile of V^T 2 bytes per key.
  const int64_t pstride = ((int64_t)H * D << ps_log2) * 2;
  const char* gbase = (group_b ? vpages : kpages) + (((int64_t)h * D) << ps_log2) * 2;
  const int kshift = group_b ? 1 : 8;
  auto stage = [&](int t, char* dst) {
    const int64_t k0 = (int64_t)t * BN;
    const int64_t page = page_of(a.page_table, k0 >> ps_log2);
    const char* base = gbase + page * pstride + ((k0 & psm) << kshift);
    char* l = dst + gw * 1024;
    // raw descriptor over the tile: stride 0, no range limit, gfx9 default
    // data format; lane offsets stay below 2^31 for pages up to 2^20 keys
    // (the dispatcher's bound for this kernel)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000);
#pragma unroll
    for (int i = 0; i < NL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(l + i * 4096), 16, (int)(i * gstep + goff), 0, 0, 0);
  };
  // group B, tail tile: zero the V^T entries of keys >= n_kv once they
  // landed.  Chunk position c of head-dim row d holds the keys
  // (c ^ swz8(d)) * 8 .. +7; each thread rewrites 4 of the 1024 chunks.
  auto zero_tail = [&](int t, char* vl) {
    const int64_t k0 = (int64_t)t * BN;
    if (k0 + BN <= a.n_kv) return;
    wait_vm<0>();
    const int nvalid = (int)(a.n_kv - k0);   // keys of the tile that exist
    const int gt = tid & (GT - 1);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = i * GT + gt;             // chunk index: row q / 8, position q % 8
      const int d = q >> 3, c = q & 7;
      const int key0 = (c ^ swz<8>(d)) * 8;
      u32x4* p = reinterpret_cast<u32x4*>(vl + q * 16);
      u32x4 v = *p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (key0 + 2 * w >= nvalid) v[w] &= 0xFFFF0000u;
        if (key0 + 2 * w + 1 >= nvalid) v[w] &= 0x0000FFFFu;
      }
      *p = v;
    }
  };

  // fp8: direct load i of wave gw writes fp8-slot bytes [i*4096 + gw*1024,
  // +1024): K as 64 rows of 128 bytes (one run in the page) with their
  // 16-byte chunks swizzled for the fp8 MFMA's reads, V^T as 128 head-dim
  // rows of 64 bytes (row d at d * page size in the page) as they lie.  The tile's scale (one per page and head) is read
  // after the loads, by a vector load so it is counted with them.
  uint32_t goff8 = 0;
  int64_t gstep8 = 0;
  if constexpr (FP8) {
    if (!group_b) {
      // 16-byte chunk c of K row r at position c ^ swz8(r) (the swizzle
      // depends on r's low 4 bits, so load i is rows + 32 i at a uniform step)
      const int row = gw * 8 + (lane >> 3);
      goff8 = (uint32_t)(row * 128 + (((lane & 7) ^ swz<8>(row)) * 16));
      gstep8 = 4096;
    } else {
      const int q0 = gw * 64 + lane;         // chunk q0: row q0 / 4, 16 keys (q0 % 4) * 16 ..
      goff8 = (uint32_t)(((int64_t)(q0 >> 2) << ps_log2) + (q0 & 3) * 16);
      gstep8 = (int64_t)64 << ps_log2;
    }
  }
  auto stage8 = [&](int t, char* dst) -> float {
    const int64_t k0 = (int64_t)t * BN;
    const int64_t page = page_of(a.page_table, k0 >> ps_log2);
    const int64_t ph = page * H + h;
    const char* base = group_b ? vpages + ((ph * D) << ps_log2) + (k0 & psm)
                               : kpages + (((ph << ps_log2) | (k0 & psm)) * D);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000);
#pragma unroll
    for (int i = 0; i < NL8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(dst + gw * 1024 + i * 4096), 16,
                                               (int)(i * gstep8 + goff8), 0, 0, 0);
    int si = (int)ph;
    asm volatile("" : "+v"(si));
    return (group_b ? a.v_scales : a.k_scales)[si];
  };
  // fp8, group B: widen the V^T chunks this thread loaded (fp8 slot `src`)
  // into the swizzled bf16 slot `dst` (exact: E4M3 fits bf16), zeroing the
  // entries of keys >= n_kv, and publish the tile's V scale sc in scl[1][ss].
  // Chunk q = head-dim row q / 4, keys (q % 4) * 16 .. +15 -> bf16 chunks
  // 2 (q % 4) and + 1 of that row.
  auto widen_one = [&](int i, const u32x4 c, int nvalid, char* dst, auto Masked) {
    const int q = i * GT + (tid & (GT - 1));
    {
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        lo[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, false));
        lo[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, true));
        hi[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w + 2], 1.0f, false));
        hi[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w + 2], 1.0f, true));
      }
      const int d = q >> 2, cq = q & 3;
      if (decltype(Masked)::value && nvalid < BN) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int key = 16 * cq + 2 * w;
          if (key >= nvalid) lo[w] &= 0xFFFF0000u;
          if (key + 1 >= nvalid) lo[w] &= 0x0000FFFFu;
          if (key + 8 >= nvalid) hi[w] &= 0xFFFF0000u;
          if (key + 9 >= nvalid) hi[w] &= 0x0000FFFFu;
        }
      }
      char* rp = dst + d * 128;
      *reinterpret_cast<u32x4*>(rp + (((2 * cq) ^ swz<8>(d)) * 16)) = lo;
      *reinterpret_cast<u32x4*>(rp + (((2 * cq + 1) ^ swz<8>(d)) * 16)) = hi;
    }
  };
  auto nvalid_of = [&](int t) { return (int)min((int64_t)BN, a.n_kv - (int64_t)t * BN); };
  auto widen_tile = [&](int t, const char* src, char* dst) {
    const int gt = tid & (GT - 1);
    const int nvalid = nvalid_of(t);
#pragma unroll
    for (int i = 0; i < NL8; ++i) widen_one(i, ld16(src + (i * GT + gt) * 16), nvalid, dst, ic<1>{});
  };
  auto widen = [&](int t, const char* src, char* dst, float sc, int ss) {
    widen_tile(t, src, dst);
    if ((tid & (GT - 1)) == 0) scl[1][ss] = sc;
  };

  // O += V(last)^T P(last)^T, V(last) in V slot rl
  auto final_pv = [&](const bf16x8 (&p)[4], int rl) {
    if (idle) return;
    const char* vl;
    if constexpr (FP8) vl = rl == 0 ? lv0 : (rl == 1 ? lv1 : lv2);
    else vl = rl == 0 ? lv0 : (rl == 1 ? lv1 : (rl == 2 ? lv2 : lv3));
    const char* vbase = vl + vrow;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 vf[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vf[db] = __builtin_bit_cast(bf16x8, ld16(vbase + (((uint32_t)(32 * c)) ^ vx) + db * 32 * BN * 2));
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], p[c], o[db], 0, 0, 0);
    }
  };

  // ------------------------------------------------------------ main loop
  if (t_begin < t_end) {
    const int t0 = t_begin, tl = t_end - 1;
    bf16x8 pp[4];                          // P(t-1); P(t0-1) = 0
#pragma unroll
    for (int c = 0; c < 4; ++c) pp[c] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    // The two waves sharing a SIMD (one per group) are in opposite phases.
    // The issue arbiter favours older waves, so without a raised priority in
    // the matrix phase group B's MFMAs and LDS reads queue behind group A's
    // softmax; with it, whichever wave is in its matrix phase issues first
    // and the softmax fills the gaps.

    if constexpr (FP8) {
      // fp8: three-slot rings, two barriers per tile.  Iteration t with ring
      // position R = (t - t0) % 3: K(t) and V(t) in slot R, V(t-1) in slot
      // R+2 (mod 3), which also receives K(t+2) and V(t+2) during the vector
      // phase; group B runs one phase behind group A.
      // prologue: K(t0), K(t0+1) into the fp8 K ring (group A); V(t0), V(t0+1)
      // into the fp8 V ring, zeros into bf16 V slot 2, which stands for
      // V(t0-1) (group B); P(t0-1) = 0, so the first PV step adds exact zeros.
      float sc[3] = {1.0f, 1.0f, 1.0f};      // scale of the tile staged into each slot
      sc[0] = stage8(t0, fslot(ic<0>{}));
      sc[1] = stage8(min(t0 + 1, tl), fslot(ic<1>{}));
      if (group_b) {
        const int gt = tid & (GT - 1);
#pragma unroll
        for (int i = 0; i < NL; ++i) *reinterpret_cast<u32x4*>(lv2 + (i * GT + gt) * 16) = u32x4{0, 0, 0, 0};
      }
      wait_vm<0>();
      // V: widened (t0 + 1 in matrix phase t0); K: read as fp8, only its scale
      if (group_b) widen(t0, fslot(ic<0>{}), lv0, sc[0], 0);
      else if ((tid & (GT - 1)) == 0) scl[0][0] = sc[0];
      lds_barrier();
      if (group_b) lds_barrier();            // group B runs one phase behind

      // G: the group (0 = A, 1 = B), fixed per loop so that group B's
      // widening steps sit between its MFMAs without a branch
      auto iter = [&](int t, auto R, auto G) {
        constexpr int r = decltype(R)::value;
        constexpr bool GB = decltype(G)::value != 0;
        constexpr int rp = (r + 2) % 3;
        char* kl = k8slot(ic<r>{});
        char* vprev = vslot(ic<rp>{});
        // ---------------- matrix phase: S(t), then O += V(t-1)^T P(t-1)^T
        f32x16 s[2];
        // group B widens V(t+1), staged one phase ago, into the bf16 slot that
        // held V(t-2), between its MFMAs
        const int wt = min(t + 1, tl);
        const char* wsrc = fslot(ic<r + 1>{});
        char* wdst = vslot(ic<(r + 1) % 3>{});
        const int wgt = tid & (GT - 1);
        __builtin_amdgcn_s_setprio(2);
        if (!idle) {
          // opaque per-iteration copies: keep the read addresses from being
          // precomputed for all three slots outside the loop
          uint32_t xk = kx8, xv = vx, kro = krow8, vro = vrow;
          asm volatile("" : "+v"(xk), "+v"(xv), "+v"(kro), "+v"(vro));
          const char* kbase = kl + kro;
          const char* vbase = vprev + vro;
          constexpr int NK = 8;                // (mb, kk, 16-byte part)
          constexpr int NR = NK + 4 * DB;
          auto rd = [&](int j) -> bf16x8 {
            if (j < NK) {
              const int mb = j >> 2, kk = (j >> 1) & 1, part = j & 1;
              return __builtin_bit_cast(bf16x8, ld16(kbase + (((uint32_t)((4 * kk + part) * 16)) ^ xk) + mb * 32 * 128));
            }
            const int c = (j - NK) / DB, db = (j - NK) % DB;
            return __builtin_bit_cast(bf16x8, ld16(vbase + (((uint32_t)(32 * c)) ^ xv) + db * 32 * BN * 2));
          };
          bf16x8 fr[NR];
          u32x4 wc;
#pragma unroll
          for (int j = 0; j < NIF; ++j) fr[j] = rd(j);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < NR; ++j) {
            if (j < NK) {
              if (j & 1) {                     // both halves of the (mb, kk) fragment read
                const int mb = j >> 2, kk = (j >> 1) & 1;
                const i32x8 af = __builtin_bit_cast(
                    i32x8, __builtin_shufflevector(__builtin_bit_cast(u32x4, fr[j - 1]), __builtin_bit_cast(u32x4, fr[j]),
                                                   0, 1, 2, 3, 4, 5, 6, 7));
                s[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, qh[kk], kk == 0 ? f32x16{} : s[mb],
                                                                         0, 0, 0, 127, 0, 127);
                s[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, ql[kk], s[mb], 0, 0, 0, 127, 0, 127);
              }
            } else {
              const int c = (j - NK) / DB, db = (j - NK) % DB;
              o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], pp[c], o[db], 0, 0, 0);
            }
            if (j + NIF < NR) fr[j + NIF] = rd(j + NIF);
            if constexpr (GB) {
              // the conversions fill the issue slots the MFMA chains leave
              // (without the tail mask, which would put a branch among the
              // MFMAs: the one tile that ends past n_kv is widened again,
              // masked, before the last PV step)
              if (j == kWidenAt) {
                wait_vm<0>();
                wc = ld16(wsrc + wgt * 16);
              } else if (j == kWidenAt + kWidenStep) {
                widen_one(0, wc, 0, wdst, ic<0>{});
                wc = ld16(wsrc + (GT + wgt) * 16);
              } else if (j == kWidenAt + 2 * kWidenStep) {
                widen_one(1, wc, 0, wdst, ic<0>{});
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        wait_vm<0>();
        if (group_b) {
          if (idle) widen(wt, wsrc, wdst, sc[(r + 1) % 3], (r + 1) % 3);
          else if (wgt == 0) scl[1][(r + 1) % 3] = sc[(r + 1) % 3];
        } else if (wgt == 0) {
          scl[0][(r + 1) % 3] = sc[(r + 1) % 3];
        }
        lds_barrier();

        // ---------------- vector phase: next tile two ahead into the free
        // slot, then the softmax of tile t -> P(t)
        sc[(r + 2) % 3] = stage8(min(t + 2, tl), fslot(ic<r + 2>{}));
        if (!idle) {
          const int64_t k0 = (int64_t)t * BN;
          if (k0 + BN > lim_first) {
            int thr = (int)min(lim - k0, (int64_t)BN) - 8 * half;
            asm volatile("" : "+v"(thr));
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr)
                if (32 * mb + 16 * (rr >> 3) + (rr & 7) >= thr) s[mb][rr] = -INFINITY;
          }
          // the K scale of tile t multiplies its logits; its V scale
          // multiplies P(t) (folded into the exponent), the row sum is
          // divided by it back
          const float sl = a.scale_log2 * scl[0][r] * qs;
          if (t == t0) {
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[mb][rr]);
            m_run = pair_max(mx) * sl;
          }
          const float mneg = __builtin_amdgcn_logf(scl[1][r]) - m_run;
          float part[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int mb = c >> 1, rb = 8 * (c & 1);
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][rb + e], sl, mneg));
              acc += p;
              pp[c][e] = (__bf16)p;
            }
            part[c] = acc;
          }
          // the tile's own V scale divides its sum back out
          float tsum = (part[0] + part[1]) + (part[2] + part[3]);
          tsum *= __builtin_amdgcn_rcpf(scl[1][r]);
          overflow |= !(tsum <= kSlowSum);
          l_run += tsum;
        }
        lds_barrier();
      };

      auto run = [&](auto G) {
        int t = t0;
        for (; t + 2 <= tl; t += 3) {
          iter(t, ic<0>{}, G);
          iter(t + 1, ic<1>{}, G);
          iter(t + 2, ic<2>{}, G);
        }
        if (t <= tl) iter(t, ic<0>{}, G);
        if (t + 1 <= tl) iter(t + 1, ic<1>{}, G);
      };
      if (group_b) run(ic<1>{});
      else run(ic<0>{});
      if (tl > t0 && nvalid_of(tl) < BN) {
        // the last tile ends past n_kv: group A widens it again from its
        // codes with the tail zeroed (the codes are still in its fp8 slot:
        // the re-stagings of the clamped tiles past tl went to the other two
        // slots) while group B runs its last vector phase, and the barrier
        // publishes it before either group's last PV step
        if (!group_b) {
          const int rl = (tl - t0) % 3;
          if (rl == 0) widen_tile(tl, fv0, lv0);
          else if (rl == 1) widen_tile(tl, fv1, lv1);
          else widen_tile(tl, fv2, lv2);
        }
        lds_barrier();
      }
      final_pv(pp, (tl - t0) % 3);
      if (tid == 0) item_sh[nxt] = settle(atomicAdd(a.sched + cur_q, 1));
      if (!group_b) lds_barrier();           // balance group B's extra barrier

    } else {
      // bf16: four-slot rings, tile t in slot (t - t0) % 4, one barrier per
      // tile.  Between two barriers (window k) group A runs the vector phase
      // of tile k and then the matrix phase of tile k+1, group B the matrix
      // phase of tile k and then the vector phase of tile k, so the groups are
      // in opposite phases without a barrier between the phases.  In window k
      // group A stages K(k+3) and waits for K(k+2), group B stages V(k+2) and
      // waits for V(k+1) (and clears its tail); the barrier ending the window
      // publishes both.  The tiles read in window k are K(k), K(k+1), V(k-1)
      // and V(k), none of them in a slot being staged into.
      // prologue: K(t0..t0+2) into K slots 0..2 (group A); V(t0), V(t0+1) into
      // V slots 0, 1 and zeros into V slot 3, which stands for V(t0-1) (group
      // B); K(t0), K(t0+1) and V(t0) complete before the first barrier.
      if (!group_b) {
        stage(t0, lk0);
        stage(min(t0 + 1, tl), lk1);
        stage(min(t0 + 2, tl), lk2);
        wait_vm<NL>();
      } else {
        stage(t0, lv0);
        stage(min(t0 + 1, tl), lv1);
        const int gt = tid & (GT - 1);
#pragma unroll
        for (int i = 0; i < NL; ++i) *reinterpret_cast<u32x4*>(lv3 + (i * GT + gt) * 16) = u32x4{0, 0, 0, 0};
        wait_vm<NL>();
        zero_tail(t0, lv0);
      }
      lds_barrier();

      f32x16 s[2];
      // matrix phase of tile t (ring position r): S(t) = K(t) Q^T, then
      // O += V(t-1)^T P(t-1)^T
      auto mat = [&](int t, auto R) {
        constexpr int r = decltype(R)::value;
        char* kl = kslot(ic<r>{});
        char* vprev = vslot(ic<(r + 3) & 3>{});
        __builtin_amdgcn_s_setprio(2);
        if (!idle) {
          // opaque per-phase copies: keep the read addresses from being
          // precomputed for all four slots outside the loop
          uint32_t xk = kx, xv = vx, kro = krow, vro = vrow;
          asm volatile("" : "+v"(xk), "+v"(xv), "+v"(kro), "+v"(vro));
          const char* kbase = kl + kro;
          const char* vbase = vprev + vro;
          constexpr int NK = 2 * KK;
          constexpr int NR = NK + 4 * DB;
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
        __builtin_amdgcn_sched_barrier(0);
      };
      // vector phase of tile t (ring position r): stage the group's next tile,
      // the softmax of S(t) -> P(t), then wait for the tile the window
      // publishes
      auto vec = [&](int t, auto R) {
        constexpr int r = decltype(R)::value;
        if (!group_b) stage(min(t + 3, tl), kslot(ic<(r + 3) & 3>{}));
        else stage(min(t + 2, tl), vslot(ic<(r + 2) & 3>{}));
        if (!idle) {
          const int64_t k0 = (int64_t)t * BN;
          if (k0 + BN > lim_first) {
            // key 32 mb + 16 (rr / 8) + 8 half + rr % 8 is masked when it is
            // >= lrel: compare the lane-independent part (an inline constant)
            // with lrel - 8 half, so no per-element key index is held in a
            // register across the loop
            int thr = (int)min(lim - k0, (int64_t)BN) - 8 * half;
            asm volatile("" : "+v"(thr));
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr)
                if (32 * mb + 16 * (rr >> 3) + (rr & 7) >= thr) s[mb][rr] = -INFINITY;
          }
          const float sl = a.scale_log2;
          if (t == t0) {
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[mb][rr]);
            m_run = pair_max(mx) * sl;
          }
          const float mneg = -m_run;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int mb = c >> 1, rb = 8 * (c & 1);
            float acc = lc[c];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][rb + e], sl, mneg));
              acc += p;
              pp[c][e] = (__bf16)p;
            }
            lc[c] = acc;
          }
        }
        wait_vm<NL>();
        if (group_b) zero_tail(min(t + 1, tl), vslot(ic<(r + 1) & 3>{}));
        __builtin_amdgcn_sched_barrier(0);
      };
      // window k at ring position R = (k - t0) % 4; each group runs its own
      // loop, with the same number of barriers
      auto window_a = [&](int k, auto R) {
        constexpr int r = decltype(R)::value;
        vec(k, ic<r>{});
        if (k < tl) mat(k + 1, ic<(r + 1) & 3>{});
        lds_barrier();
      };
      auto window_b = [&](int k, auto R) {
        constexpr int r = decltype(R)::value;
        mat(k, ic<r>{});
        vec(k, ic<r>{});
        lds_barrier();
      };
      int t = t0;
      if (!group_b) {
        mat(t0, ic<0>{});                    // the window before t0: group B waits
        lds_barrier();
        for (; t + 3 <= tl; t += 4) {
          window_a(t, ic<0>{});
          window_a(t + 1, ic<1>{});
          window_a(t + 2, ic<2>{});
          window_a(t + 3, ic<3>{});
        }
        if (t <= tl) window_a(t, ic<0>{});
        if (t + 1 <= tl) window_a(t + 1, ic<1>{});
        if (t + 2 <= tl) window_a(t + 2, ic<2>{});
      } else {
        lds_barrier();
        for (; t + 3 <= tl; t += 4) {
          window_b(t, ic<0>{});
          window_b(t + 1, ic<1>{});
          window_b(t + 2, ic<2>{});
          window_b(t + 3, ic<3>{});
        }
        if (t <= tl) window_b(t, ic<0>{});
        if (t + 1 <= tl) window_b(t + 1, ic<1>{});
        if (t + 2 <= tl) window_b(t + 2, ic<2>{});
      }
      final_pv(pp, (tl - t0) & 3);
      if (tid == 0) item_sh[nxt] = settle(atomicAdd(a.sched + cur_q, 1));
    }
    wait_vm<0>();                          // no direct load outlives the item
  } else if (tid == 0) {
    item_sh[nxt] = settle(atomicAdd(a.sched + cur_q, 1));
  }

  if constexpr (!FP8) {
    // bf16: the whole sum against the bound (any tile's sum above it puts
    // the total above it too)
    l_run = (lc[0] + lc[1]) + (lc[2] + lc[3]);
    overflow |= !(l_run <= kSlowSum);
  }
  // one flag per (query tile, split, wave), written unconditionally
  const bool wave_overflow = __builtin_amdgcn_ballot_w64(overflow) != 0;
  if (lane == 0) a.flags_out[((int64_t)(h * nqt + qt) * a.nsplit + split) * NW + wave] = wave_overflow;
  if (wave_overflow) {
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
    for (int db = 0; db < DB; ++db)
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
  } else {
    // the split's output over its keys, normalised by its own row sum, in
    // bf16 (the merge weighs it by l 2^(m - M)); an empty split stores zeros
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
  };

  // LDS-only barriers between items: the partial stores of an item need
  // not land before the next one starts
  if (tid == 0) item_sh[0] = settle(qlen(cur_q) > 0 ? atomicAdd(a.sched + cur_q, 1) : 0);
  lds_barrier();
  for (int k = 0;; k ^= 1) {
    const int item = item_sh[k];
    if (item < 0) break;
    const int x = item >> 24, v = item & 0xFFFFFF;
    const int hl = heads_lo(x);
    const int per = (heads_lo(x + 1) - hl) * nqt;
    const int split = v / per;
    const int rem = v - split * per;
    work(rem % nqt, split, hl + rem / nqt, k ^ 1);
    lds_barrier();                           // next item visible; LDS rings free
  }
}

__global__ void attn_sched_reset_kernel(int32_t* sched) {
  if (threadIdx.x < kAttnQueues) sched[threadIdx.x] = 0;
}

hipError_t launch_attn_dma(const AttnArgs& a, bool kv_fp8, hipStream_t s) {
  if (a.head_dim != 128 || a.ps_log2 < 6 || !a.sched) return hipErrorInvalidValue;
  if (kv_fp8 && (!a.k_scales || !a.v_scales)) return hipErrorInvalidValue;
  if ((int64_t)a.n_heads * ((a.n_q + BM - 1) / BM) * a.nsplit >= (int64_t{1} << 24))
    return hipErrorInvalidValue;             // item numbers must fit 24 bits
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t nqt = (a.n_q + BM - 1) / BM;
  const int64_t total = nqt * a.n_heads * a.nsplit;
  // one persistent workgroup per CU (the LDS rings allow one per CU)
  const unsigned grid = (unsigned)std::min<int64_t>(total, std::max(ncu, 1));
  attn_sched_reset_kernel<<<1, 64, 0, s>>>(a.sched);
  if (kv_fp8) attn_dma_kernel<128, true><<<grid, NT, 0, s>>>(a);
  else attn_dma_kernel<128, false><<<grid, NT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bca
