/*
 * One performer unit driven through the C ABI of libbca from plain C (no
 * C++, no Python): reads the unit's inputs from a file, appends the history
 * and runs performer_unit on the GPU with a workspace of
 * bca_workspace_bytes(), and writes the unit's attention output and clean
 * latents to another file.  Used by tests/test_gpu_c_abi.py, which writes
 * the inputs and checks the outputs against the oracle.
 *
 * Usage: performer_unit_c IN OUT
 * IN (little endian):
 *   int64 hdr[8] = {n_heads, head_dim, page_size, n_hist, n_q, n_ch,
 *                   n_steps, n_phys_pages}
 *   int32 page_table[ceil((n_hist + n_q) / page_size)]
 *   uint16 (bf16 bits) k_hist, v_hist [n_hist][H][D]; k_new, v_new, q [n_q][H][D]
 *   float w[H*D][n_ch], z[n_q][n_ch] (the noise the solver starts from)
 * OUT: uint16 (bf16 bits) o[n_q][H][D], then float z[n_q][n_ch].
 * Exit status 0 on success; any failing call is named on stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "bca.h"

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));              \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

#define BCA_OK_(call)                                                         \
  do {                                                                        \
    bca_status s_ = (call);                                                   \
    if (s_ != BCA_OK) {                                                       \
      fprintf(stderr, "%s: %s\n", #call, bca_status_string(s_));              \
      exit(3);                                                                \
    }                                                                         \
  } while (0)

static void* read_exact(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input file\n");
    exit(4);
  }
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
  if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int64_t* hdr = (int64_t*)read_exact(in, 8 * sizeof(int64_t));
  const int64_t H = hdr[0], D = hdr[1], ps = hdr[2], n_hist = hdr[3], n_q = hdr[4];
  const int64_t n_ch = hdr[5], n_steps = hdr[6], n_phys = hdr[7];
  const int64_t n_log = (n_hist + n_q + ps - 1) / ps;
  const size_t row = (size_t)(H * D) * 2;          /* bytes of one token's bf16 K, V or Q */

  int32_t* pt = (int32_t*)read_exact(in, (size_t)n_log * 4);
  void* kh = read_exact(in, (size_t)n_hist * row);
  void* vh = read_exact(in, (size_t)n_hist * row);
  void* kn = read_exact(in, (size_t)n_q * row);
  void* vn = read_exact(in, (size_t)n_q * row);
  void* q = read_exact(in, (size_t)n_q * row);
  float* w = (float*)read_exact(in, (size_t)(H * D * n_ch) * 4);
  float* z = (float*)read_exact(in, (size_t)(n_q * n_ch) * 4);
  fclose(in);

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));

  bca_kv_cache c;
  c.k_pages = NULL;
  c.v_pages = NULL;
  const size_t page_bytes = (size_t)(H * ps * D) * 2;
  HIP_OK(hipMalloc(&c.k_pages, (size_t)n_phys * page_bytes));
  HIP_OK(hipMalloc(&c.v_pages, (size_t)n_phys * page_bytes));
  c.k_scales = NULL;
  c.v_scales = NULL;
  c.page_table = (const int32_t*)to_device(pt, (size_t)n_log * 4);
  c.max_logical_pages = (int32_t)n_log;
  c.n_phys_pages = (int32_t)n_phys;
  c.page_size = (int32_t)ps;
  c.n_heads = (int32_t)H;
  c.head_dim = (int32_t)D;
  c.dtype = BCA_BF16;
  c.n_tokens = 0;

  void* d_kh = to_device(kh, (size_t)n_hist * row);
  void* d_vh = to_device(vh, (size_t)n_hist * row);
  void* d_kn = to_device(kn, (size_t)n_q * row);
  void* d_vn = to_device(vn, (size_t)n_q * row);
  void* d_q = to_device(q, (size_t)n_q * row);
  float* d_w = (float*)to_device(w, (size_t)(H * D * n_ch) * 4);
  float* d_z = (float*)to_device(z, (size_t)(n_q * n_ch) * 4);
  void* d_o = NULL;
  HIP_OK(hipMalloc(&d_o, (size_t)n_q * row));
  const size_t ws_bytes = bca_workspace_bytes(&c, n_q, n_hist + n_q, (int32_t)n_ch);
  void* d_ws = NULL;
  HIP_OK(hipMalloc(&d_ws, ws_bytes));

  if (n_hist > 0) BCA_OK_(kv_append(&c, d_kh, d_vh, n_hist, BCA_BF16, s));
  BCA_OK_(performer_unit(&c, d_kn, d_vn, d_q, n_q, d_w, d_z, (int32_t)n_ch, (int32_t)n_steps,
                         d_o, d_ws, ws_bytes, NULL, s));
  HIP_OK(hipStreamSynchronize(s));
  if (c.n_tokens != n_hist + n_q) {
    fprintf(stderr, "n_tokens %lld, expected %lld\n", (long long)c.n_tokens,
            (long long)(n_hist + n_q));
    return 5;
  }

  void* o = malloc((size_t)n_q * row);
  HIP_OK(hipMemcpy(o, d_o, (size_t)n_q * row, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(z, d_z, (size_t)(n_q * n_ch) * 4, hipMemcpyDeviceToHost));
  FILE* out = fopen(argv[2], "wb");
  if (!out || fwrite(o, 1, (size_t)n_q * row, out) != (size_t)n_q * row ||
      fwrite(z, 4, (size_t)(n_q * n_ch), out) != (size_t)(n_q * n_ch)) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 6;
  }
  fclose(out);

  HIP_OK(hipFree(d_ws));
  HIP_OK(hipFree(d_o));
  HIP_OK(hipFree(d_z));
  HIP_OK(hipFree(d_w));
  HIP_OK(hipFree(d_q));
  HIP_OK(hipFree(d_vn));
  HIP_OK(hipFree(d_kn));
  HIP_OK(hipFree(d_vh));
  HIP_OK(hipFree(d_kh));
  HIP_OK(hipFree((void*)c.page_table));
  HIP_OK(hipFree(c.v_pages));
  HIP_OK(hipFree(c.k_pages));
  HIP_OK(hipStreamDestroy(s));
  free(o);
  free(z);
  free(w);
  free(q);
  free(vn);
  free(kn);
  free(vh);
  free(kh);
  free(pt);
  free(hdr);
  return 0;
}
