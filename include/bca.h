/*
 * bca.h -- C ABI of the block-causal performer step on MI355X (gfx950).
 *
 * The performer step of Wan-Streamer, one streaming unit at a time:
 *   1. kv_append          append the unit's K/V slice to the full-history cache
 *   2. block_causal_attn  attention of the unit's queries over the cache under
 *                         the block-causal visibility rule
 *   3. fm_euler_step      one explicit Euler step of the flow-matching ODE,
 *                         z <- z - dtau * v, with v the attention output
 *                         projected by a fixed matrix W (stand-in for the
 *                         velocity network)
 *   4. performer_unit     1 once, then n_steps x (2, 3)
 *
 * Sources, cited by page title and section:
 *   - xiaohu-jiedu.pages.dev explainer "wan-streamer-realtime-av": section on
 *     listening while speaking and its block-causal figure caption (tokens of
 *     a block see each other both ways, a block sees only earlier blocks);
 *     deployment section (performer runs only the flow-matching solver over
 *     the shared full-history KV context).
 *   - alwayszhang.cn deep read "全双工语音模型精读⑫：Wan-Streamer":
 *     section 3.2 (z_tau = (1-tau) z0 + tau eps, dz/dtau = eps - z0) and
 *     section 4, step 3 (the performer appends the received KV slice to its
 *     own full-history cache and runs the flow solver for the next unit).
 *   - wiki note "Wan-Streamer v0.1: End-to-end Real-time Interactive
 *     Foundation Models", contribution 3 table (performer: receive KV slice
 *     -> flow-matching solver -> return clean latents).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates no device buffers.  Its only state across calls is
 *     host-side: a 16-entry memo of the attention split count per call
 *     shape (behind a mutex, so calls from several threads are safe; it
 *     changes no result, only which split count a shape gets without
 *     re-running the model that picks it); performer_unit_noalloc alone
 *     adds a fixed per-GPU device array and its looked-up address (see its
 *     declaration).  The streaming session
 *     (bca_session_*) is the one object the library creates: host
 *     bookkeeping plus the HIP graphs it replays, owned by the caller
 *     through the session handle.
 *   - Work is enqueued asynchronously on the caller's stream `s`; calls
 *     return after enqueue.  Two calls that share a cache or a workspace
 *     must be ordered by the caller (same stream or events).
 *   - Arguments are validated on the host before anything is launched; on
 *     error nothing is enqueued and no host field changes.  No C++
 *     exception crosses this boundary.
 *   - Shapes are row-major, innermost index last.
 */
#ifndef BCA_H
#define BCA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifndef BCA_API
#define BCA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BCA_OK = 0,
  BCA_EINVAL = -1,       /* null pointer, bad size, inconsistent arguments   */
  BCA_ERANGE = -2,       /* append past the mapped pages, n_kv > n_tokens    */
  BCA_EUNSUPPORTED = -3, /* head_dim / dtype / page-size combination not built */
  BCA_EHIP = -4          /* the HIP runtime reported a launch error           */
} bca_status;

typedef enum {
  BCA_F32 = 0,
  BCA_BF16 = 1,
  BCA_FP8_E4M3 = 2       /* OCP E4M3FN codes, cache storage only             */
} bca_dtype;

/*
 * Paged full-history KV cache (the performer's copy of the shared context).
 *
 * Logical token t lives in physical page page_table[t / page_size], slot
 * t % page_size.  Per physical page p and head h:
 *   K: k_pages[p][h][slot][d]        (row per token)
 *   V: v_pages[p][h][d][slot]        (d-major: a run of tokens is contiguous)
 * Element type: float (BCA_F32), bf16 (BCA_BF16) or uint8 E4M3FN codes
 * (BCA_FP8_E4M3).  For fp8, the value of a code is decode(code) * scale with
 * one fp32 scale per (physical page, head) for K (k_scales[p][h]) and for V
 * (v_scales[p][h]); k_scales/v_scales are NULL otherwise.
 *
 * Supported: page_size a power of two >= 16 (>= 64 for fp8); head_dim 32, 64
 * or 128 for BCA_F32, 64 or 128 for BCA_BF16, 128 for BCA_FP8_E4M3.
 * page_table (device int32, max_logical_pages entries) must hold distinct
 * physical indices < n_phys_pages; this is not checked on the device.
 * Slots past n_tokens are never read as values that reach an output.
 * n_tokens is HOST state: the number of valid tokens, advanced by kv_append.
 */
typedef struct {
  void* k_pages;
  void* v_pages;
  float* k_scales;
  float* v_scales;
  const int32_t* page_table;
  int32_t max_logical_pages;
  int32_t n_phys_pages;
  int32_t page_size;
  int32_t n_heads;
  int32_t head_dim;
  int32_t dtype;          /* bca_dtype */
  int64_t n_tokens;
} bca_kv_cache;

/*
 * kv_append -- copy a unit's K/V slice into the cache at logical positions
 * [n_tokens, n_tokens + n_new), then n_tokens += n_new (on the host, at
 * enqueue).  (deep read section 4 step 3; wiki contribution 3 table.)
 *
 * k_new, v_new: [n_new][n_heads][head_dim], src_dtype BCA_F32 for an f32
 * cache, BCA_BF16 for bf16 and fp8 caches.  bf16/f32 caches receive a bit
 * copy.  An fp8 cache quantises each touched (page, head) block of K and of
 * V: amax over its valid rows, scale = amax/448, code = RNE-saturate to
 * E4M3FN of (x * (448/amax)) in fp32; amax = 0 gives scale 1 and codes 0;
 * slots past the valid rows get code 0.  An fp8 append that starts inside a
 * partly filled page re-quantises that page: the rows it already holds
 * enter its block as the values they hold, fp32(decode(code) * scale), so
 * they may move by one rounding onto the new scale's grid.
 * n_new == 0 is a no-op.  BCA_ERANGE if the append would pass
 * max_logical_pages * page_size.
 */
BCA_API bca_status kv_append(bca_kv_cache* c, const void* k_new, const void* v_new,
                     int64_t n_new, int32_t src_dtype, hipStream_t s);

/*
 * block_causal_attn -- O[i] = sum_j softmax_j(scale * q_i . k_j) v_j over the
 * keys j < n_kv that query i may see: j / block_size <= (q_pos0 + i) /
 * block_size (tokens of one block see each other both ways and every earlier
 * block, never a later one; explainer figure caption).  Heads are
 * independent; query head h reads KV head h.
 *
 *   q:   [n_q][n_heads][head_dim], q_dtype (BCA_F32 with an f32 cache,
 *        BCA_BF16 with bf16 and fp8 caches)
 *   out: [n_q][n_heads][head_dim], out_dtype BCA_BF16 or BCA_F32 (f32 only
 *        with an f32 cache)
 *   q_pos0: global position of query row 0; requires 0 <= q_pos0 and
 *        q_pos0 + n_q <= n_kv <= c->n_tokens.
 *        Streaming call: q_pos0 = n_kv - n_q, block_size = n_kv: every key
 *        below n_kv is visible to every query, whatever n_kv - n_q is.
 *        (block_size = n_q gives the same only when n_kv - n_q is a
 *        multiple of n_q; otherwise the grid j / n_q cuts the queries'
 *        block in two.)
 *        Full sequence:  q_pos0 = 0, n_q = n_kv.  block_size = 1 is causal.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).
 *   workspace: optional device scratch (may be NULL) of workspace_bytes.
 *        Without it a single kernel with an exact running-maximum softmax
 *        runs.  With it (layout: 512*n_q bytes, rounded up to a multiple of
 *        256, reserved for fm_euler_step's partial sums, then this call's
 *        region: overflow flags, 256 bytes of work-queue counters that the
 *        call zeroes itself, the split partials: per split, its output
 *        normalised by its row sum in bf16 and its (m, l) in fp32) a
 *        faster kernel runs
 *        that keeps the first key tile's row maximum as its softmax
 *        reference and flags any query tile in which a row's weights
 *        relative to that reference add up past 2^40 or to a non-finite
 *        value; flagged tiles are recomputed exactly.  The key range may also
 *        be split across workgroups and merged by a fixed-order log-sum-exp
 *        combine.  Results never depend on timing.  bca_workspace_bytes()
 *        gives the size that enables every path.
 */
BCA_API bca_status block_causal_attn(const void* q, int64_t n_q, int64_t q_pos0,
                             int32_t block_size, const bca_kv_cache* c,
                             int64_t n_kv, void* out, int32_t q_dtype,
                             int32_t out_dtype, float softmax_scale,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t s);

/*
 * fm_euler_step -- one explicit Euler step toward tau = 0 of the
 * flow-matching ODE whose velocity is dz/dtau (deep read section 3.2):
 *   z[i][c] <- z[i][c] - dtau * v[i][c]
 * w != NULL: v[i][c] = sum_k x[i][k] * w[k][c], x [n_tok][k] (x_dtype BCA_BF16
 *            or BCA_F32), w [k][n_ch] fp32.
 * w == NULL: v = x, x [n_tok][n_ch] fp32 (k ignored).
 * z [n_tok][n_ch] fp32, updated in place.  n_ch <= 64.  n_tok == 0 is a
 * no-op (z and x may then be NULL).
 * workspace (may be NULL): with bf16 x, n_ch = 16, k a multiple of 256 and
 * at most 8192, and at least 512*n_tok bytes, the product runs on the
 * matrix cores (W split into bf16 high/low halves, W = hi + lo to ~2^-16;
 * eight partial sums per token written to the workspace, then added in
 * order by a second launch); otherwise a slower fp32 vector path runs.
 * Results do not depend on timing (fixed summation order).
 */
BCA_API bca_status fm_euler_step(float* z, const void* x, const float* w,
                         int64_t n_tok, int32_t k, int32_t n_ch, float dtau,
                         int32_t x_dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t s);

/*
 * performer_unit -- one streaming unit of the performer (deep read section 4
 * step 3; wiki contribution 3 table): kv_append(k_new, v_new); then for
 * s = 0 .. n_steps-1: block_causal_attn of q over the whole cache
 * (n_kv = n_tokens after the append, q_pos0 = n_kv - n_q, block_size = n_kv)
 * into o_scratch, then fm_euler_step(z, o_scratch, w, dtau = 1/n_steps).
 * The unit is one block: its queries see every cached key, their own slice
 * in both directions (explainer, figure caption of the block-causal mask),
 * also when the history is not a multiple of n_q.  n_tokens + n_q must not
 * exceed INT32_MAX (BCA_EINVAL).
 *
 *   k_new, v_new, q: [n_q][n_heads][head_dim] (f32 for an f32 cache, else
 *                    bf16)
 *   w:  [n_heads*head_dim][n_ch] fp32;  z: [n_q][n_ch] fp32, noise in,
 *       clean latents out
 *   o_scratch: [n_q][n_heads][head_dim] (f32 for an f32 cache, else bf16)
 *   workspace: as for block_causal_attn / fm_euler_step (may be NULL);
 *       bca_workspace_bytes() gives the size for the fastest path
 *   attn_events: NULL, or 3*n_steps events (timing hook): for step s,
 *       event 3s is recorded on the stream just before its attention,
 *       3s+1 right after the main attention kernel (before the split
 *       combine and the exact rerun of flagged tiles) and 3s+2 after the
 *       whole attention call
 * All arguments of all four phases are validated before the first launch.
 */
BCA_API bca_status performer_unit(bca_kv_cache* c, const void* k_new, const void* v_new,
                          const void* q, int64_t n_q, const float* w, float* z,
                          int32_t n_ch, int32_t n_steps, void* o_scratch,
                          void* workspace, size_t workspace_bytes,
                          hipEvent_t* attn_events, hipStream_t s);

/*
 * performer_unit_noalloc -- performer_unit for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  The same unit (same arguments and results as
 * performer_unit without the workspace and the timing hook); it calls no
 * allocator.  Its scratch is a fixed array of BCA_NOALLOC_SCRATCH_BYTES in
 * the library's device data, one per GPU, which each GPU the library runs
 * on holds until the process ends.  The key-range split of the attention
 * may take only as many splits as fit in it (at most 6 at the v0.2 unit,
 * 40 heads x 3712 queries, against up to 8), so results can differ from performer_unit
 * with a larger workspace by rounding; with a workspace of exactly
 * BCA_NOALLOC_SCRATCH_BYTES performer_unit gives the same bits.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (the kernels need no initial contents): calls that overlap on one
 * GPU -- on different streams, or from different threads, without ordering
 * -- race on it and must not be made.
 * Errors: as performer_unit; BCA_ERANGE when the unit's least scratch need
 * (512 bytes per query for the velocity partials plus the attention's flags
 * and counters) passes BCA_NOALLOC_SCRATCH_BYTES (about 500,000 queries).
 */
#define BCA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
BCA_API bca_status performer_unit_noalloc(bca_kv_cache* c, const void* k_new, const void* v_new,
                                  const void* q, int64_t n_q, const float* w, float* z,
                                  int32_t n_ch, int32_t n_steps, void* o_scratch, hipStream_t s);

/*
 * Streaming session -- many consecutive performer units over one growing
 * cache (deep read section 4 step 3: the performer appends every received
 * slice to its own full-history cache and runs the solver for the next
 * unit).  The session hands out physical pages as the cache grows: when a
 * unit's tokens reach logical pages not mapped yet, it takes the next
 * entries of free_pages, writes them into the cache's page_table on the
 * stream (before the unit's append), and commits them.  A unit that starts
 * inside a partly filled page continues that page.
 *
 * bca_session_create: c must stay valid for the session's life; the
 *   logical pages holding c->n_tokens tokens must already be mapped;
 *   free_pages (host array of n_free distinct physical page ids in
 *   [0, n_phys_pages), none of them in use) is copied.  Errors: EINVAL.
 * bca_session_unit: one performer_unit (same arguments and result) after
 *   the page mapping.  use_graph != 0: the unit's launches are captured
 *   into a HIP graph and launched on s.  Graph units alternate between two
 *   instantiated graphs; each is updated in place when the new unit's
 *   shape allows, but only after its previous launch (two graph units
 *   back) has finished, which the call waits for on the host.  So one unit
 *   may be queued ahead of the GPU without blocking the host.  On a stream
 *   that is already being captured the launches simply join that capture.
 *   Errors
 *   as performer_unit, plus ERANGE when free_pages cannot cover the unit;
 *   on error nothing of the unit is committed (n_tokens and the page count
 *   unchanged).
 * bca_session_free_pages: free pages left (-1 for NULL).
 * bca_session_destroy: waits for the session's graph launches to finish,
 *   then releases the graphs and the session (NULL is a no-op).
 * Calls on one session must be ordered by the caller.
 */
typedef struct bca_session bca_session;
BCA_API bca_status bca_session_create(bca_kv_cache* c, const int32_t* free_pages,
                              int32_t n_free, bca_session** out);
BCA_API bca_status bca_session_unit(bca_session* ss, const void* k_new, const void* v_new,
                            const void* q, int64_t n_q, const float* w, float* z,
                            int32_t n_ch, int32_t n_steps, void* o_scratch,
                            void* workspace, size_t workspace_bytes, int32_t use_graph,
                            hipStream_t s);
BCA_API int64_t bca_session_free_pages(const bca_session* ss);
BCA_API void bca_session_destroy(bca_session* ss);

/* Workspace size that lets block_causal_attn (n_q queries over n_kv keys of
 * cache c) and fm_euler_step (n_q tokens, k = n_heads*head_dim, n_ch
 * channels) use their fastest split.  Host-only, never fails (0 on bad
 * input). */
BCA_API size_t bca_workspace_bytes(const bca_kv_cache* c, int64_t n_q, int64_t n_kv,
                           int32_t n_ch);

/* Static string naming a status code. */
BCA_API const char* bca_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* BCA_H */
