// Prints the number of key-range splits block_causal_attn picks for a call
// shape, from the library's own host code (no GPU needed: without one the
// CU count falls back to 256, the MI355X's).  Used by
// tests/test_split_choice.py.
//   split_choice H D page_size dtype(0 f32, 1 bf16, 2 fp8) n_q q_pos0 block_size n_kv
#include <cstdio>
#include <cstdlib>

#include "../../block_causal_attention_performer_amd/csrc/bca_api.hip"

int main(int argc, char** argv) {
  if (argc != 9) {
    std::fprintf(stderr, "usage: %s H D page_size dtype n_q q_pos0 block_size n_kv\n", argv[0]);
    return 1;
  }
  bca_kv_cache c{};
  c.n_heads = std::atoi(argv[1]);
  c.head_dim = std::atoi(argv[2]);
  c.page_size = std::atoi(argv[3]);
  c.dtype = std::atoi(argv[4]);
  const int64_t n_q = std::atoll(argv[5]), q_pos0 = std::atoll(argv[6]), n_kv = std::atoll(argv[8]);
  const int32_t B = std::atoi(argv[7]);
  const int s = choose_attn_split(&c, n_q, q_pos0, B, n_kv, attn_split_bytes(&c, n_q, kMaxAttnSplit));
  std::printf("%d\n", s);
  return 0;
}
