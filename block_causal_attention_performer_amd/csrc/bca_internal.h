// Internal declarations shared by the library's translation units (host
// launchers and small device helpers).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bca.h"

namespace bca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kKeyTile = 64;        // keys per attention tile (a tile never straddles a >=64 page)
constexpr int kAttnFlagWaves = 8;   // overflow flags per (query tile, split) of the fast attention kernel
constexpr int kMaxAttnSplit = 8;    // most key-range splits of one attention call
constexpr int kEulerChunks = 8;     // k-range parts of the velocity projection
constexpr int kEulerMaxK = 8192;    // largest k the MFMA projection takes (32 k-steps per part)
constexpr int kAttnQueues = 8;      // work queues of the persistent bf16 attention kernel, one per XCD
constexpr size_t kAttnSchedBytes = 256;   // workspace bytes for their counters

// ---------------------------------------------------------------- launchers

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_pages;
  void* v_pages;
  float* k_scales;
  float* v_scales;
  const int32_t* page_table;
  int64_t n0;        // first logical position written
  int64_t n_new;
  int32_t n_heads;
  int32_t head_dim;
  int32_t ps_log2;
};
hipError_t launch_append_copy(const AppendArgs& a, int elem_bytes, hipStream_t s);
hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;
  void* out;
  const void* k_pages;
  const void* v_pages;
  const float* k_scales;
  const float* v_scales;
  const int32_t* page_table;
  uint16_t* ws_o;    // split partials: [nsplit][n_q][H][D] bf16, each split's output over
                     // its keys normalised by its own row sum
  float* ws_ml;      // [nsplit][n_q][H][2]  (reference max in log2 units, row sum)
  int32_t* flags_out;    // fast kernel: [H][n_qtiles][nsplit][kAttnFlagWaves] overflow flags
  int32_t* sched;        // fast kernel: kAttnQueues work-queue counters (zeroed by its launch)
  const int32_t* flags;  // exact kernel: recompute only query tiles flagged here
  int32_t flag_splits;   // nsplit the flags were written with
  int64_t n_q;
  int64_t q_pos0;
  int64_t n_kv;
  int32_t block_size;
  int32_t n_heads;
  int32_t head_dim;
  int32_t ps_log2;
  int32_t nsplit;
  int32_t out_f32;
  float scale_log2;  // softmax_scale * log2(e)
  float scale;       // softmax_scale
};
// bf16 / fp8 MFMA path.  kv_fp8 selects fp8 pages.  Returns the error of the
// launch; nsplit > 1 also launches the combine.  Needs flags_out.
// main_done (may be null) is recorded on s after the main kernel, before
// the split combine
hipError_t launch_attn_mfma(const AttnArgs& a, bool kv_fp8, hipEvent_t main_done, hipStream_t s);
// The kernel with direct HBM -> LDS tile loads (head dim 128, pages of >= 64
// keys; bf16 or fp8 pages, fp8 widened to bf16 in LDS); same query tiles,
// flags and split partials.
hipError_t launch_attn_dma(const AttnArgs& a, bool kv_fp8, hipStream_t s);
// Merge of the split partials into out.
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s);
// Exact-rescaling MFMA kernel (no split); with flags set it only rewrites
// flagged query tiles.
hipError_t launch_attn_exact(const AttnArgs& a, bool kv_fp8, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);
// Query rows per attention workgroup (the unit of the split heuristic).
int attn_mfma_rows_per_wg();

struct EulerArgs {
  float* z;
  const void* x;
  const float* w;
  float* part;             // projection partials [kEulerChunks][n_tok][16] (workspace)
  int64_t n_tok;
  int32_t k;
  int32_t n_ch;
  float dtau;
};
// v = x W (bf16 x, n_ch 16, k a multiple of 32 * kEulerChunks) and the
// update, through the partials in a.part (two launches).
hipError_t launch_euler_proj(const EulerArgs& a, hipStream_t s);
hipError_t launch_euler_generic(const EulerArgs& a, bool x_f32, hipStream_t s);
hipError_t launch_euler_plain(const EulerArgs& a, hipStream_t s);

}  // namespace bca
