// Host side of the C ABI declared in include/bca.h: argument validation,
// work-split heuristics and kernel dispatch.  Nothing here allocates device
// memory or keeps state between calls.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "bca_internal.h"

using namespace bca;

namespace {

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
  if (c->dtype == BCA_FP8_E4M3 && n_new > 0 && c->n_tokens % c->page_size != 0) return BCA_EUNSUPPORTED;
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
  const size_t parts = nsplit > 1 ? align256(per * c->head_dim * 4) + align256(per * 2 * 4) : 0;
  return attn_flag_bytes(c, n_q, nsplit) + kAttnSchedBytes + parts;
}

// Workspace layout: [velocity-projection partials, kEulerChunks x 64 bytes
// per token] [attention: overflow flags, queue counters, split partials].
size_t euler_ws_bytes(int64_t n_tok) { return align256((size_t)kEulerChunks * n_tok * 16 * 4); }

// Pick the number of key-range splits: enough workgroups to fill every CU
// for the last wave without making the partial round trips dominate.
int choose_attn_split(const bca_kv_cache* c, int64_t n_q, int64_t q_pos0, int32_t B, int64_t n_kv,
                      size_t room) {
  if (c->dtype == BCA_F32) return 1;
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
  const int cus = cu_count();
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
      a.ws_o = reinterpret_cast<float*>(ws);
      a.ws_ml = reinterpret_cast<float*>(ws + align256(per * c->head_dim * 4));
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
  if (!z || !x) return BCA_EINVAL;
  if (n_tok < 0 || n_ch <= 0 || !isfinite(dtau)) return BCA_EINVAL;
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

}  // namespace

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
  // the attention region follows the Euler region (W's transposed halves)
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
  if (!c || !q || !w || !z || !o_scratch || n_q <= 0 || n_steps <= 0) return BCA_EINVAL;
  const int32_t io = c->dtype == BCA_F32 ? BCA_F32 : BCA_BF16;
  bca_status st = check_append(c, k_new, v_new, n_q, io);
  if (st != BCA_OK) return st;
  const int64_t n_kv = c->n_tokens + n_q;
  bca_kv_cache after = *c;
  after.n_tokens = n_kv;
  st = check_attn(q, n_q, n_kv - n_q, (int32_t)n_q, &after, n_kv, o_scratch, io, io, 0.0f);
  if (st != BCA_OK) return st;
  const int32_t kdim = c->n_heads * c->head_dim;
  const float dtau = 1.0f / (float)n_steps;
  st = check_euler(z, o_scratch, w, n_q, kdim, n_ch, dtau, io);
  if (st != BCA_OK) return st;
  if (n_q > INT32_MAX) return BCA_EINVAL;

  st = enqueue_append(c, k_new, v_new, n_q, s);
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
    st = enqueue_attn(q, n_q, n_kv - n_q, (int32_t)n_q, c, n_kv, o_scratch, io, 0.0f, attn_ws,
                      attn_room, ev ? ev[1] : nullptr, s);
    if (st != BCA_OK) return st;
    if (ev && hipEventRecord(ev[2], s) != hipSuccess) return BCA_EHIP;
    st = enqueue_euler(z, o_scratch, w, n_q, kdim, n_ch, dtau, io, eu ? ws : nullptr,
                       eu ? eu_bytes : 0, s);
    if (st != BCA_OK) return st;
  }
  return BCA_OK;
}

}  // extern "C"
