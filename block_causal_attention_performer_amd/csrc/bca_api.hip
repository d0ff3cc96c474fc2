// Host side of the C ABI declared in include/bca.h: argument validation,
// work-split heuristics and kernel dispatch.  Nothing here allocates device
// memory; the state kept between calls is a small host-side memo of split
// decisions and, per GPU, the address of the fixed scratch array of
// performer_unit_noalloc.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "bca_internal.h"

using namespace bca;

// Fixed scratch of performer_unit_noalloc, for callers that cannot allocate:
// one copy per GPU the library runs on, in the code object's device data,
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host the name is a stand-in, not a device address): the
// device address of each GPU's copy is looked up once, with that GPU
// current, and kept in noalloc_ptr.
static __device__ __align__(256) char scratch[BCA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[kMaxDevices];

// Device address of the current GPU's scratch array.
bca_status noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BCA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return BCA_EUNSUPPORTED;
  std::lock_guard<std::mutex> g(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return BCA_EHIP;
    }
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return BCA_OK;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) { int l = 0; while ((int64_t{1} << l) < x) ++l; return l; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Validates the cache descriptor (not its device contents).
bca_status check_cache(const bca_kv_cache* c) {
  if (!c || !c->k_pages || !c->v_pages || !c->page_table) return BCA_EINVAL;
  if (c->n_heads <= 0 || c->head_dim <= 0 || c->max_logical_pages <= 0 || c->n_phys_pages <= 0)
    return BCA_EINVAL;
  if (c->n_tokens < 0) return BCA_EINVAL;
  if (!is_pow2(c->page_size) || c->page_size < 16) return BCA_EUNSUPPORTED;
  switch (c->dtype) {
    case BCA_F32:
      if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return BCA_EUNSUPPORTED;
      break;
    case BCA_BF16:
      if (c->head_dim != 64 && c->head_dim != 128) return BCA_EUNSUPPORTED;
      break;
    case BCA_FP8_E4M3:
      if (c->head_dim != 128 || c->page_size < 64 || c->page_size > 256) return BCA_EUNSUPPORTED;
      if (!c->k_scales || !c->v_scales) return BCA_EINVAL;
      break;
    default:
      return BCA_EUNSUPPORTED;
  }
  if (c->n_tokens > (int64_t)c->max_logical_pages * c->page_size) return BCA_ERANGE;
  return BCA_OK;
}

bca_status check_append(const bca_kv_cache* c, const void* k_new, const void* v_new,
                        int64_t n_new, int32_t src_dtype) {
  bca_status st = check_cache(c);
  if (st != BCA_OK) return st;
  if (n_new < 0) return BCA_EINVAL;
  if (n_new > 0 && (!k_new || !v_new)) return BCA_EINVAL;
  const int32_t want = c->dtype == BCA_F32 ? BCA_F32 : BCA_BF16;
  if (src_dtype != want) return BCA_EUNSUPPORTED;
  if (c->n_tokens + n_new > (int64_t)c->max_logical_pages * c->page_size) return BCA_ERANGE;
  return BCA_OK;
}

bca_status enqueue_append(bca_kv_cache* c, const void* k_new, const void* v_new, int64_t n_new,
                          hipStream_t s) {
  if (n_new == 0) return BCA_OK;
  AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pages = c->k_pages;
  a.v_pages = c->v_pages;
  a.k_scales = c->k_scales;
  a.v_scales = c->v_scales;
  a.page_table = c->page_table;
  a.n0 = c->n_tokens;
  a.n_new = n_new;
  a.n_heads = c->n_heads;
  a.head_dim = c->head_dim;
  a.ps_log2 = ilog2(c->page_size);
  hipError_t e = c->dtype == BCA_FP8_E4M3 ? launch_append_fp8(a, s)
                                          : launch_append_copy(a, c->dtype == BCA_F32 ? 4 : 2, s);
  if (e != hipSuccess) return BCA_EHIP;
  c->n_tokens += n_new;
  return BCA_OK;
}

struct AttnPlan {
  int nsplit;
  size_t o_bytes;
};

// Attention workspace: overflow flags, the work-queue counters, then (with a
// split) the partials.
size_t attn_flag_bytes(const bca_kv_cache* c, int64_t n_q, int nsplit) {
  const int64_t BM = attn_mfma_rows_per_wg();
  const int64_t nqt = (n_q + BM - 1) / BM;
  return align256((size_t)nqt * c->n_heads * nsplit * kAttnFlagWaves * 4);
}
size_t attn_split_bytes(const bca_kv_cache* c, int64_t n_q, int nsplit) {
  const size_t per = (size_t)nsplit * n_q * c->n_heads;
  const size_t parts = nsplit > 1 ? align256(per * c->head_dim * 2) + align256(per * 2 * 4) : 0;
  return attn_flag_bytes(c, n_q, nsplit) + kAttnSchedBytes + parts;
}

// Workspace layout: [velocity-projection partials, kEulerChunks x 64 bytes
// per token] [attention: overflow flags, queue counters, split partials].
size_t euler_ws_bytes(int64_t n_tok) { return align256((size_t)kEulerChunks * n_tok * 16 * 4); }

// Calls that run on the persistent direct-load kernel (its dispatch rule).
bool attn_persistent(const bca_kv_cache* c) {
  return c->dtype != BCA_F32 && c->head_dim == 128 && c->page_size >= 64 && c->page_size <= (1 << 20);
}

// Modelled duration (us) of a persistent attention launch with `s` splits
// plus its split combine.  The model follows the kernel's scheduling: one
// workgroup per CU, workgroup i on XCD i % kAttnQueues, kAttnQueues queues
// holding their heads' items split-major, then head, then query tile; a
// workgroup takes the next item of its own queue, else of the first later
// queue with items left.  An item costs its key tiles times the per-tile
// time of a CU under full load (fewer when its query tile has idle waves)
// plus a fixed per-item cost; the combine reads s bf16 partials and writes
// the output at a plain copy's rate.  The constants are measured on MI355X
// (v0.2 launch: 1.63 us per 64-key tile per CU, about 6 us per item).
double persistent_cost_us(const std::vector<int64_t>& qt_tiles, const std::vector<double>& qt_frac,
                          int H, int s, int cus, int64_t n_q, int D) {
  constexpr double kTileUs = 1.63, kItemUs = 6.0, kCopyBytesPerUs = 4.0e6;
  const int64_t wsum = 2 * (s - 1) + 1;
  const int nqt = (int)qt_tiles.size();
  // cost of the item of split sp and query tile t (equal for every head)
  std::vector<double> cost_tab((size_t)s * nqt);
  for (int sp = 0; sp < s; ++sp)
    for (int t = 0; t < nqt; ++t) {
      const int64_t T = qt_tiles[t];
      const int64_t b = T * (2 * sp) / wsum;
      const int64_t e = sp + 1 == s ? T : T * (2 * sp + 2) / wsum;
      cost_tab[(size_t)sp * nqt + t] = kItemUs + (double)(e - b) * qt_frac[t] * kTileUs;
    }
  // queue x holds heads [lo(x), lo(x+1)): item v is split v / per, query
  // tile v % nqt, per = its heads x nqt
  int64_t per[kAttnQueues], len[kAttnQueues], pos[kAttnQueues] = {};
  int64_t total = 0;
  for (int x = 0; x < kAttnQueues; ++x) {
    const int64_t lo = ((int64_t)x * H + kAttnQueues - 1) / kAttnQueues;
    const int64_t hi = ((int64_t)(x + 1) * H + kAttnQueues - 1) / kAttnQueues;
    per[x] = (hi - lo) * nqt;
    len[x] = per[x] * s;
    total += len[x];
  }
  // binary min-heap of (time a workgroup frees, workgroup)
  const int grid = (int)std::min<int64_t>(total, cus);
  std::vector<double> ht((size_t)grid, 0.0);
  std::vector<int> hw((size_t)grid);
  for (int i = 0; i < grid; ++i) hw[i] = i;
  int n = grid;
  double end = 0.0;
  while (n > 0) {
    const double t0 = ht[0];
    const int w = hw[0];
    int y = -1;
    for (int k = 0; k < kAttnQueues && y < 0; ++k) {
      const int x = (w + k) % kAttnQueues;
      if (pos[x] < len[x]) y = x;
    }
    double t_new;
    int w_new;
    if (y < 0) {                      // nothing left: the workgroup ends
      end = std::max(end, t0);
      --n;
      if (n == 0) break;
      t_new = ht[n];
      w_new = hw[n];
    } else {
      const int64_t v = pos[y]++;
      t_new = t0 + cost_tab[(size_t)(v / per[y]) * nqt + (size_t)(v % nqt)];
      w_new = w;
    }
    // sift the new root down
    int i = 0;
    for (;;) {
      int c = 2 * i + 1;
      if (c >= n) break;
      if (c + 1 < n && ht[c + 1] < ht[c]) ++c;
      if (ht[c] >= t_new) break;
      ht[i] = ht[c];
      hw[i] = hw[c];
      i = c;
    }
    ht[i] = t_new;
    hw[i] = w_new;
  }
  const double comb = s == 1 ? 0.0 : ((double)s * n_q * H * D * 2 + (double)n_q * H * D * 2) / kCopyBytesPerUs;
  return end + comb;
}

// Split count for the persistent kernel: the modelled best; among counts
// within 0.75% of it the largest, since finer items also absorb the spread
// of CU and XCD speeds that the model leaves out.  Decisions are memoised
// per call shape (one evaluation costs about 1 ms at 40 heads x 15 query
// tiles).
int choose_split_persistent(const bca_kv_cache* c, int64_t n_q, int64_t q_pos0, int32_t B, int64_t n_kv,
                            int max_s, int cus) {
  struct Memo { int64_t key[7]; int s; };
  static std::mutex mu;
  static Memo memo[16];
  static int n_memo = 0, next_slot = 0;
  const int64_t key[7] = {c->n_heads, n_q, q_pos0, B, n_kv, max_s, cus};
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < n_memo; ++i)
      if (!memcmp(memo[i].key, key, sizeof key)) return memo[i].s;
  }
  const int64_t BM = attn_mfma_rows_per_wg();
  const int64_t nqt = (n_q + BM - 1) / BM;
  std::vector<int64_t> tiles((size_t)nqt);
  std::vector<double> frac((size_t)nqt);
  for (int64_t qt = 0; qt < nqt; ++qt) {
    const int64_t rows = std::min(BM, n_q - qt * BM);
    const int64_t lim = std::min(n_kv, ((q_pos0 + qt * BM + rows - 1) / B + 1) * (int64_t)B);
    tiles[qt] = (lim + kKeyTile - 1) / kKeyTile;
    // a query tile with idle waves: measured 0.87 of a full tile's time
    // with half of its 8 waves idle
    frac[qt] = 0.74 + 0.26 * (double)((rows + 31) / 32) / 8.0;
  }
  // as for the register-staged kernels: at least 4 key tiles per split on
  // average
  double mean_tiles = 0.0;
  for (int64_t t : tiles) mean_tiles += (double)t;
  mean_tiles /= (double)nqt;
  while (max_s > 1 && mean_tiles / max_s < 4.0) --max_s;
  std::vector<double> cost((size_t)max_s + 1);
  double best = 1e300;
  for (int s = 1; s <= max_s; ++s) {
    cost[s] = persistent_cost_us(tiles, frac, c->n_heads, s, cus, n_q, c->head_dim);
    best = std::min(best, cost[s]);
  }
  int pick = 1;
  for (int s = 1; s <= max_s; ++s)
    if (cost[s] <= 1.0075 * best) pick = s;
  std::lock_guard<std::mutex> g(mu);
  Memo& m = memo[next_slot];
  memcpy(m.key, key, sizeof key);
  m.s = pick;
  next_slot = (next_slot + 1) % 16;
  n_memo = std::min(n_memo + 1, 16);
  return pick;
}

// Pick the number of key-range splits.  Persistent kernel with at most 4
// (query tile, head) pairs per CU: from the model above, where the end of
// the launch (a few items per CU) decides.  Otherwise (more pairs, or the
// register-staged kernels with one workgroup per item): enough workgroups
// to fill every CU for the last wave without making the partial round
// trips dominate; with many items per CU the two agree (both pick 4 splits
// for 8 v0.2 units of queries at once).
int choose_attn_split(const bca_kv_cache* c, int64_t n_q, int64_t q_pos0, int32_t B, int64_t n_kv,
                      size_t room) {
  if (c->dtype == BCA_F32) return 1;
  const int cus = cu_count();
  if (attn_persistent(c) &&
      ((n_q + attn_mfma_rows_per_wg() - 1) / attn_mfma_rows_per_wg()) * c->n_heads <= 4 * (int64_t)cus) {
    int max_s = 1;
    while (max_s < kMaxAttnSplit && attn_split_bytes(c, n_q, max_s + 1) <= room) ++max_s;
    return choose_split_persistent(c, n_q, q_pos0, B, n_kv, max_s, cus);
  }
  const int64_t BM = attn_mfma_rows_per_wg();
  const int64_t nqt = (n_q + BM - 1) / BM;
  double tiles = 0.0;
  for (int64_t qt = 0; qt < nqt; ++qt) {
    const int64_t rl = (qt * BM + BM < n_q ? qt * BM + BM : n_q) - 1;
    const int64_t lim = std::min(n_kv, ((q_pos0 + rl) / B + 1) * (int64_t)B);
    tiles += (double)((lim + kKeyTile - 1) / kKeyTile);
  }
  tiles /= (double)nqt;
  const double wgs = (double)nqt * c->n_heads;
  int best = 1;
  double best_cost = 1e300;
  for (int s = 1; s <= kMaxAttnSplit; ++s) {
    if (attn_split_bytes(c, n_q, s) > room) break;
    if (tiles / s < 4.0 && s > 1) break;
    const double rounds = ceil(wgs * s / cus);
    const double cost = rounds * (tiles / s + 6.0) + (s > 1 ? 2.0 + 0.5 * s : 0.0);
    if (cost < best_cost - 1e-9) { best_cost = cost; best = s; }
  }
  return best;
}

bca_status check_attn(const void* q, int64_t n_q, int64_t q_pos0, int32_t block_size,
                      const bca_kv_cache* c, int64_t n_kv, void* out, int32_t q_dtype,
                      int32_t out_dtype, float softmax_scale) {
  bca_status st = check_cache(c);
  if (st != BCA_OK) return st;
  if (!q || !out) return BCA_EINVAL;
  if (n_q <= 0 || n_kv <= 0 || block_size <= 0 || q_pos0 < 0) return BCA_EINVAL;
  if (q_pos0 + n_q > n_kv) return BCA_EINVAL;
  if (n_kv > c->n_tokens) return BCA_ERANGE;
  if (!isfinite(softmax_scale)) return BCA_EINVAL;
  if (c->dtype == BCA_F32) {
    if (q_dtype != BCA_F32 || out_dtype != BCA_F32) return BCA_EUNSUPPORTED;
  } else {
    if (q_dtype != BCA_BF16) return BCA_EUNSUPPORTED;
    if (out_dtype != BCA_BF16 && out_dtype != BCA_F32) return BCA_EUNSUPPORTED;
  }
  return BCA_OK;
}

bca_status enqueue_attn(const void* q, int64_t n_q, int64_t q_pos0, int32_t block_size,
                        const bca_kv_cache* c, int64_t n_kv, void* out, int32_t out_dtype,
                        float softmax_scale, void* workspace, size_t workspace_bytes,
                        hipEvent_t main_done, hipStream_t s) {
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)c->head_dim);
  AttnArgs a{};
  a.q = q;
  a.out = out;
  a.k_pages = c->k_pages;
  a.v_pages = c->v_pages;
  a.k_scales = c->k_scales;
  a.v_scales = c->v_scales;
  a.page_table = c->page_table;
  a.n_q = n_q;
  a.q_pos0 = q_pos0;
  a.n_kv = n_kv;
  a.block_size = block_size;
  a.n_heads = c->n_heads;
  a.head_dim = c->head_dim;
  a.ps_log2 = ilog2(c->page_size);
  a.out_f32 = out_dtype == BCA_F32;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  const size_t room = workspace ? workspace_bytes : 0;
  const bool fp8 = c->dtype == BCA_FP8_E4M3;
  hipError_t e;
  if (c->dtype == BCA_F32) {
    a.nsplit = 1;
    e = launch_attn_f32(a, s);
    if (e == hipSuccess && main_done) e = hipEventRecord(main_done, s);
  } else if (room >= attn_split_bytes(c, n_q, 1)) {
    // fast kernel (+ combine), then the exact kernel for flagged query tiles
    a.nsplit = choose_attn_split(c, n_q, q_pos0, block_size, n_kv, room);
    char* ws = static_cast<char*>(workspace);
    a.flags_out = reinterpret_cast<int32_t*>(ws);
    ws += attn_flag_bytes(c, n_q, a.nsplit);
    a.sched = reinterpret_cast<int32_t*>(ws);
    ws += kAttnSchedBytes;
    if (a.nsplit > 1) {
      const size_t per = (size_t)a.nsplit * n_q * c->n_heads;
      a.ws_o = reinterpret_cast<uint16_t*>(ws);
      a.ws_ml = reinterpret_cast<float*>(ws + align256(per * c->head_dim * 2));
    }
    e = launch_attn_mfma(a, fp8, main_done, s);
    if (e == hipSuccess) {
      AttnArgs x = a;
      x.flags = a.flags_out;
      x.flag_splits = a.nsplit;
      x.flags_out = nullptr;
      x.nsplit = 1;
      e = launch_attn_exact(x, fp8, s);
    }
  } else {
    a.nsplit = 1;
    e = launch_attn_exact(a, fp8, s);
    if (e == hipSuccess && main_done) e = hipEventRecord(main_done, s);
  }
  return e == hipSuccess ? BCA_OK : BCA_EHIP;
}

bca_status check_euler(float* z, const void* x, const float* w, int64_t n_tok, int32_t k,
                       int32_t n_ch, float dtau, int32_t x_dtype) {
  if (n_tok < 0 || n_ch <= 0 || !isfinite(dtau)) return BCA_EINVAL;
  if (n_tok > 0 && (!z || !x)) return BCA_EINVAL;   // zero tokens touch nothing
  if (n_ch > 64) return BCA_EUNSUPPORTED;
  if (w) {
    if (k <= 0) return BCA_EINVAL;
    if (x_dtype != BCA_BF16 && x_dtype != BCA_F32) return BCA_EUNSUPPORTED;
  } else {
    if (x_dtype != BCA_F32) return BCA_EUNSUPPORTED;
  }
  return BCA_OK;
}

bool euler_mfma_ok(const float* w, int32_t k, int32_t n_ch, int32_t x_dtype) {
  return w && x_dtype == BCA_BF16 && n_ch == 16 && k % (32 * kEulerChunks) == 0 && k <= kEulerMaxK;
}

bca_status enqueue_euler(float* z, const void* x, const float* w, int64_t n_tok, int32_t k,
                         int32_t n_ch, float dtau, int32_t x_dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t s) {
  if (n_tok == 0) return BCA_OK;
  EulerArgs a{};
  a.z = z;
  a.x = x;
  a.w = w;
  a.n_tok = n_tok;
  a.k = k;
  a.n_ch = n_ch;
  a.dtau = dtau;
  hipError_t e;
  if (!w) {
    e = launch_euler_plain(a, s);
  } else if (euler_mfma_ok(w, k, n_ch, x_dtype) && workspace &&
             workspace_bytes >= euler_ws_bytes(n_tok)) {
    a.part = static_cast<float*>(workspace);
    e = launch_euler_proj(a, s);
  } else {
    e = launch_euler_generic(a, x_dtype == BCA_F32, s);
  }
  return e == hipSuccess ? BCA_OK : BCA_EHIP;
}

// performer_unit in two passes, so a caller that must change state between
// validation and launch (the streaming session) can validate first.
bca_status check_performer(const bca_kv_cache* c, const void* k_new, const void* v_new,
                           const void* q, int64_t n_q, const float* w, float* z, int32_t n_ch,
                           int32_t n_steps, void* o_scratch) {
  if (!c || !q || !w || !z || !o_scratch || n_q <= 0 || n_steps <= 0) return BCA_EINVAL;
  const int32_t io = c->dtype == BCA_F32 ? BCA_F32 : BCA_BF16;
  bca_status st = check_append(c, k_new, v_new, n_q, io);
  if (st != BCA_OK) return st;
  const int64_t n_kv = c->n_tokens + n_q;
  if (n_kv > INT32_MAX) return BCA_EINVAL;    // the unit's block size is n_kv (int32)
  bca_kv_cache after = *c;
  after.n_tokens = n_kv;
  st = check_attn(q, n_q, n_kv - n_q, (int32_t)n_kv, &after, n_kv, o_scratch, io, io, 0.0f);
  if (st != BCA_OK) return st;
  const int32_t kdim = c->n_heads * c->head_dim;
  st = check_euler(z, o_scratch, w, n_q, kdim, n_ch, 1.0f / (float)n_steps, io);
  if (st != BCA_OK) return st;
  if (n_q > INT32_MAX) return BCA_EINVAL;
  return BCA_OK;
}

bca_status enqueue_performer(bca_kv_cache* c, const void* k_new, const void* v_new, const void* q,
                             int64_t n_q, const float* w, float* z, int32_t n_ch, int32_t n_steps,
                             void* o_scratch, void* workspace, size_t workspace_bytes,
                             hipEvent_t* attn_events, hipStream_t s) {
  const int32_t io = c->dtype == BCA_F32 ? BCA_F32 : BCA_BF16;
  const int64_t n_kv = c->n_tokens + n_q;
  const int32_t kdim = c->n_heads * c->head_dim;
  const float dtau = 1.0f / (float)n_steps;
  bca_status st = enqueue_append(c, k_new, v_new, n_q, s);
  if (st != BCA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  size_t room = workspace ? workspace_bytes : 0;
  const size_t eu_bytes = euler_ws_bytes(n_q);
  const bool eu = room >= eu_bytes;
  char* attn_ws = room > eu_bytes ? ws + eu_bytes : nullptr;
  const size_t attn_room = room > eu_bytes ? room - eu_bytes : 0;
  for (int32_t step = 0; step < n_steps; ++step) {
    hipEvent_t* ev = attn_events ? attn_events + 3 * step : nullptr;
    if (ev && hipEventRecord(ev[0], s) != hipSuccess) return BCA_EHIP;
    // the unit is one block: its queries see every cached key, their own
    // slice included, whatever the history length (block size n_kv)
    st = enqueue_attn(q, n_q, n_kv - n_q, (int32_t)n_kv, c, n_kv, o_scratch, io, 0.0f, attn_ws,
                      attn_room, ev ? ev[1] : nullptr, s);
    if (st != BCA_OK) return st;
    if (ev && hipEventRecord(ev[2], s) != hipSuccess) return BCA_EHIP;
    st = enqueue_euler(z, o_scratch, w, n_q, kdim, n_ch, dtau, io, eu ? ws : nullptr,
                       eu ? eu_bytes : 0, s);
    if (st != BCA_OK) return st;
  }
  return BCA_OK;
}

// Streaming session: page-table entries for newly mapped logical pages are
// written by a kernel on the stream (values in the kernel arguments, so a
// captured graph carries them), before the unit's append reads them.
constexpr int kPtBatch = 32;
struct PtUpdate {
  int32_t lp0, count;
  int32_t phys[kPtBatch];
};
__global__ void pt_set_kernel(int32_t* pt, PtUpdate u) {
  const int i = (int)threadIdx.x;
  if (i < u.count) pt[u.lp0 + i] = u.phys[i];
}

}  // namespace

// Graph units alternate between two instantiated graphs.  A graph is
// updated (or destroyed) only once its previous launch, two units back, has
// finished (its event): rewriting the kernel arguments of an instantiated
// graph whose launch may still be queued on the stream is not something
// the runtime promises to keep from that launch.
struct bca_session {
  bca_kv_cache* cache;
  std::vector<int32_t> free_pages;   // handed out in this order
  size_t next_free;
  int64_t mapped;                    // logical pages [0, mapped) have physical pages
  hipGraphExec_t exec[2];            // unit graphs, used in turn (updated in place)
  hipEvent_t done[2];                // recorded on the stream after each one's launch
  int next_exec;                     // slot of the next graph unit
  hipStream_t cap;                   // capture-only stream (nothing executes on it)
};

extern "C" {

const char* bca_status_string(int32_t st) {
  switch (st) {
    case BCA_OK: return "ok";
    case BCA_EINVAL: return "invalid argument";
    case BCA_ERANGE: return "out of range";
    case BCA_EUNSUPPORTED: return "unsupported combination";
    case BCA_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t bca_workspace_bytes(const bca_kv_cache* c, int64_t n_q, int64_t n_kv, int32_t n_ch) {
  if (!c || n_q <= 0 || n_kv <= 0 || c->n_heads <= 0 || c->head_dim <= 0) return 0;
  (void)n_ch;
  return euler_ws_bytes(n_q) + attn_split_bytes(c, n_q, kMaxAttnSplit);
}

bca_status kv_append(bca_kv_cache* c, const void* k_new, const void* v_new, int64_t n_new,
                     int32_t src_dtype, hipStream_t s) {
  bca_status st = check_append(c, k_new, v_new, n_new, src_dtype);
  if (st != BCA_OK) return st;
  return enqueue_append(c, k_new, v_new, n_new, s);
}

bca_status block_causal_attn(const void* q, int64_t n_q, int64_t q_pos0, int32_t block_size,
                             const bca_kv_cache* c, int64_t n_kv, void* out, int32_t q_dtype,
                             int32_t out_dtype, float softmax_scale, void* workspace,
                             size_t workspace_bytes, hipStream_t s) {
  bca_status st = check_attn(q, n_q, q_pos0, block_size, c, n_kv, out, q_dtype, out_dtype,
                             softmax_scale);
  if (st != BCA_OK) return st;
  // the attention region follows the velocity projection's partial sums
  char* ws = static_cast<char*>(workspace);
  size_t room = workspace_bytes;
  if (ws) {
    const size_t skip = euler_ws_bytes(n_q);
    if (room > skip) { ws += skip; room -= skip; } else { ws = nullptr; room = 0; }
  }
  return enqueue_attn(q, n_q, q_pos0, block_size, c, n_kv, out, out_dtype, softmax_scale, ws,
                      room, nullptr, s);
}

bca_status fm_euler_step(float* z, const void* x, const float* w, int64_t n_tok, int32_t k,
                         int32_t n_ch, float dtau, int32_t x_dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t s) {
  bca_status st = check_euler(z, x, w, n_tok, k, n_ch, dtau, x_dtype);
  if (st != BCA_OK) return st;
  return enqueue_euler(z, x, w, n_tok, k, n_ch, dtau, x_dtype, workspace, workspace_bytes, s);
}

bca_status performer_unit(bca_kv_cache* c, const void* k_new, const void* v_new, const void* q,
                          int64_t n_q, const float* w, float* z, int32_t n_ch, int32_t n_steps,
                          void* o_scratch, void* workspace, size_t workspace_bytes,
                          hipEvent_t* attn_events, hipStream_t s) {
  // validate every phase before the first launch
  bca_status st = check_performer(c, k_new, v_new, q, n_q, w, z, n_ch, n_steps, o_scratch);
  if (st != BCA_OK) return st;
  return enqueue_performer(c, k_new, v_new, q, n_q, w, z, n_ch, n_steps, o_scratch, workspace,
                           workspace_bytes, attn_events, s);
}

bca_status performer_unit_noalloc(bca_kv_cache* c, const void* k_new, const void* v_new,
                                  const void* q, int64_t n_q, const float* w, float* z,
                                  int32_t n_ch, int32_t n_steps, void* o_scratch, hipStream_t s) {
  bca_status st = check_performer(c, k_new, v_new, q, n_q, w, z, n_ch, n_steps, o_scratch);
  if (st != BCA_OK) return st;
  // the fast path's least need: the velocity partials and the attention
  // flags and queue counters of an unsplit call
  if (euler_ws_bytes(n_q) + attn_split_bytes(c, n_q, 1) > BCA_NOALLOC_SCRATCH_BYTES) return BCA_ERANGE;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != BCA_OK) return st;
  return enqueue_performer(c, k_new, v_new, q, n_q, w, z, n_ch, n_steps, o_scratch, ws,
                           BCA_NOALLOC_SCRATCH_BYTES, nullptr, s);
}

bca_status bca_session_create(bca_kv_cache* c, const int32_t* free_pages, int32_t n_free,
                              bca_session** out) {
  if (!out) return BCA_EINVAL;
  *out = nullptr;
  bca_status st = check_cache(c);
  if (st != BCA_OK) return st;
  if (n_free < 0 || (n_free > 0 && !free_pages)) return BCA_EINVAL;
  std::vector<bool> seen((size_t)c->n_phys_pages, false);
  for (int32_t i = 0; i < n_free; ++i) {
    const int32_t p = free_pages[i];
    if (p < 0 || p >= c->n_phys_pages || seen[(size_t)p]) return BCA_EINVAL;
    seen[(size_t)p] = true;
  }
  bca_session* ss = new (std::nothrow) bca_session;
  if (!ss) return BCA_EINVAL;
  ss->cache = c;
  ss->free_pages.assign(free_pages, free_pages + n_free);
  ss->next_free = 0;
  ss->mapped = (c->n_tokens + c->page_size - 1) / c->page_size;
  ss->exec[0] = ss->exec[1] = nullptr;
  ss->done[0] = ss->done[1] = nullptr;
  ss->next_exec = 0;
  ss->cap = nullptr;
  *out = ss;
  return BCA_OK;
}

bca_status bca_session_unit(bca_session* ss, const void* k_new, const void* v_new, const void* q,
                            int64_t n_q, const float* w, float* z, int32_t n_ch, int32_t n_steps,
                            void* o_scratch, void* workspace, size_t workspace_bytes,
                            int32_t use_graph, hipStream_t s) {
  if (!ss) return BCA_EINVAL;
  bca_kv_cache* c = ss->cache;
  bca_status st = check_performer(c, k_new, v_new, q, n_q, w, z, n_ch, n_steps, o_scratch);
  if (st != BCA_OK) return st;
  const int64_t need = (c->n_tokens + n_q + c->page_size - 1) / c->page_size;
  const int64_t fresh = need > ss->mapped ? need - ss->mapped : 0;
  if (fresh > (int64_t)(ss->free_pages.size() - ss->next_free)) return BCA_ERANGE;

  // Graphs are captured on the session's own stream (the caller's may be the
  // null stream, which cannot be captured) and launched on s.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return BCA_EHIP;
  const bool graph = use_graph && cap == hipStreamCaptureStatusNone;
  if (graph && !ss->cap && hipStreamCreateWithFlags(&ss->cap, hipStreamNonBlocking) != hipSuccess) {
    ss->cap = nullptr;
    return BCA_EHIP;
  }
  const hipStream_t ls = graph ? ss->cap : s;   // where the unit's launches are issued
  const int64_t n_tokens0 = c->n_tokens;
  hipGraph_t g = nullptr;
  if (graph && hipStreamBeginCapture(ls, hipStreamCaptureModeRelaxed) != hipSuccess) return BCA_EHIP;
  hipError_t e = hipSuccess;
  for (int64_t i = 0; i < fresh && e == hipSuccess; i += kPtBatch) {
    PtUpdate u{};
    u.lp0 = (int32_t)(ss->mapped + i);
    u.count = (int32_t)std::min<int64_t>(kPtBatch, fresh - i);
    for (int j = 0; j < u.count; ++j) u.phys[j] = ss->free_pages[ss->next_free + (size_t)(i + j)];
    pt_set_kernel<<<1, kPtBatch, 0, ls>>>(const_cast<int32_t*>(c->page_table), u);
    e = hipGetLastError();
  }
  st = e == hipSuccess ? enqueue_performer(c, k_new, v_new, q, n_q, w, z, n_ch, n_steps, o_scratch,
                                           workspace, workspace_bytes, nullptr, ls)
                       : BCA_EHIP;
  if (graph) {
    const hipError_t ec = hipStreamEndCapture(ls, &g);
    if (st == BCA_OK && ec != hipSuccess) st = BCA_EHIP;
    const int slot = ss->next_exec;
    hipGraphExec_t& ex = ss->exec[slot];
    if (st == BCA_OK && !ss->done[slot] &&
        hipEventCreateWithFlags(&ss->done[slot], hipEventDisableTiming) != hipSuccess) {
      ss->done[slot] = nullptr;
      st = BCA_EHIP;
    }
    // this slot's previous launch (two units back) must be over before its
    // graph is rewritten
    if (st == BCA_OK && ex && hipEventSynchronize(ss->done[slot]) != hipSuccess) st = BCA_EHIP;
    if (st == BCA_OK) {
      if (ex) {
        hipGraphNode_t bad = nullptr;
        hipGraphExecUpdateResult res;
        if (hipGraphExecUpdate(ex, g, &bad, &res) != hipSuccess || res != hipGraphExecUpdateSuccess) {
          // a different shape (new page entries or not, another split
          // count): instantiate afresh, and clear the refused update from
          // the thread's last-error state
          (void)hipGetLastError();
          (void)hipGraphExecDestroy(ex);
          ex = nullptr;
        }
      }
      if (!ex && hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) != hipSuccess) {
        ex = nullptr;
        st = BCA_EHIP;
      }
      if (st == BCA_OK && hipGraphLaunch(ex, s) != hipSuccess) st = BCA_EHIP;
      if (st == BCA_OK && hipEventRecord(ss->done[slot], s) != hipSuccess) st = BCA_EHIP;
      if (st == BCA_OK) ss->next_exec = slot ^ 1;
    }
    if (g) (void)hipGraphDestroy(g);
  }
  if (st != BCA_OK) {
    c->n_tokens = n_tokens0;                 // nothing of this unit is committed
    return st;
  }
  ss->mapped += fresh;
  ss->next_free += (size_t)fresh;
  return BCA_OK;
}

int64_t bca_session_free_pages(const bca_session* ss) {
  return ss ? (int64_t)(ss->free_pages.size() - ss->next_free) : -1;
}

void bca_session_destroy(bca_session* ss) {
  if (!ss) return;
  for (int i = 0; i < 2; ++i) {
    if (ss->done[i]) (void)hipEventSynchronize(ss->done[i]);   // no launch of it still queued
    if (ss->exec[i]) (void)hipGraphExecDestroy(ss->exec[i]);
    if (ss->done[i]) (void)hipEventDestroy(ss->done[i]);
  }
  if (ss->cap) (void)hipStreamDestroy(ss->cap);
  delete ss;
}

}  // extern "C"
