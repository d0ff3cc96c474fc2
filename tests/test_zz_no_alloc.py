"""performer_unit_noalloc, the entry point for callers that cannot allocate,
against performer_unit, through the C ABI.  Two units in a row on one
growing cache, the second smaller and starting off the unit grid (its
history is not a multiple of it).  Each must equal performer_unit:
  * bit for bit when performer_unit gets a workspace of exactly the fixed
    scratch's size (the same key-range split, the same kernels);
  * within the bf16 bars (O: max-abs 2e-2, relative RMS 1e-2; z and the
    move z - eps likewise) when performer_unit gets the full workspace and
    may split further.
The first unit has the v0.2 unit's 40 heads x 3712 queries, whose split
partials (bf16, 38 MB per split, plus 1.2 MB of row maxima and sums) the
fixed 256 MiB hold at most six of, against the eight a full workspace allows."""
import pytest
import torch

import workloads
from _helpers import assert_close, assert_latents, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")


def test_noalloc_matches_performer_unit_twice():
    H, D, ps, S = 40, 128, 256, 4
    n_hist, n1, n2 = 2 * 3712, 3712, 1000
    total = n_hist + n1 + n2
    n_pages = -(-total // ps)
    pt = workloads.page_table(n_pages, n_pages + 2, 99)
    caches = [bca.KVCache(H, D, ps, pt, n_pages + 2, "bf16") for _ in range(3)]
    kh = workloads.qkv(901, n_hist, H, D, 0.5, "bf16", "cuda")
    vh = workloads.qkv(902, n_hist, H, D, 0.5, "bf16", "cuda")
    for g in caches:
        bca.kv_append(g, kh, vh)
    w = workloads.randn((H * D, 16), 903, 1.0, "cuda")
    exact_ws = torch.empty(bca.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    full_ws = bca.alloc_workspace(bca.workspace_bytes(caches[0], n1, total, 16))
    for i, n in enumerate((n1, n2)):
        say(f"noalloc unit {i}: {n} queries after {caches[0].n_tokens} tokens")
        k = workloads.qkv(910 + i, n, H, D, 0.5, "bf16", "cuda")
        v = workloads.qkv(920 + i, n, H, D, 0.5, "bf16", "cuda")
        q = workloads.qkv(930 + i, n, H, D, 0.5, "bf16", "cuda")
        eps = workloads.randn((n, 16), 940 + i, 1.0, "cuda")
        zs = [eps.clone() for _ in range(3)]
        os_ = [torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        bca.performer_unit_noalloc(caches[0], k, v, q, w, zs[0], S, os_[0])
        bca.performer_unit(caches[1], k, v, q, w, zs[1], S, o_scratch=os_[1], workspace=exact_ws)
        bca.performer_unit(caches[2], k, v, q, w, zs[2], S, o_scratch=os_[2], workspace=full_ws)
        torch.cuda.synchronize()
        assert caches[0].n_tokens == caches[1].n_tokens == caches[2].n_tokens
        assert torch.equal(os_[0], os_[1]), f"unit {i}: O differs from the same-size workspace"
        assert torch.equal(zs[0], zs[1]), f"unit {i}: z differs from the same-size workspace"
        assert_close(os_[0].float().cpu().numpy(), os_[2].float().cpu().numpy(), 2e-2, 1e-2,
                     what=f"unit {i} O vs full workspace")
        assert_latents(zs[0].cpu().numpy(), zs[2].cpu().numpy(), eps.cpu().numpy(), 2e-2, 1e-2,
                       what=f"unit {i} vs full workspace")
