"""kv_append parity: the GPU pages equal the oracle's pages bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from _helpers import make_caches, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


def _oracle_bits(pages: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(pages)
    return _bits(t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32))


SIZES = [37, 5, 64, 100, 1, 300, 16]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 32)])
@pytest.mark.parametrize("ps,shuffle", [(256, None), (64, 3), (16, 5), (32, None)])
def test_append_bit_exact(dtype, D, ps, shuffle):
    H = 3
    say(f"append dtype={dtype} D={D} ps={ps} shuffle={shuffle}")
    g, o, _ = make_caches(bca, H, D, ps, dtype, sum(SIZES), shuffle)
    for i, n in enumerate(SIZES):
        k = workloads.qkv(100 + i, n, H, D, 1.0, dtype)
        v = workloads.qkv(200 + i, n, H, D, 1.0, dtype)
        bca.kv_append(g, k.cuda(), v.cuda())
        o.append(k.double().numpy(), v.double().numpy())
        assert g.n_tokens == o.n_tokens
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(g.k_pages), _oracle_bits(o.k_pages, dtype))
    np.testing.assert_array_equal(_bits(g.v_pages), _oracle_bits(o.v_pages, dtype))


def test_append_v02_slice_full_size():
    """The 3712-token v0.2 slice appended after 32 units of history (starts at
    page 464, ends mid-page 478), 40 heads x 128, shuffled physical pages."""
    w = workloads.WORKLOADS["v02_unit"]
    H, D, ps = w.n_heads, w.head_dim, w.page_size
    n0 = w.n_hist
    n_log = -(-(n0 + w.unit_tokens) // ps)
    n_phys = n_log + 1
    pt = workloads.page_table(n_log, n_phys, 17)
    g = bca.KVCache(H, D, ps, pt, n_phys, "bf16")
    g.c.n_tokens = n0                      # history already present (not checked here)
    k = workloads.qkv(workloads.seed_for(w.index, "k_new"), w.unit_tokens, H, D, 0.5, "bf16")
    v = workloads.qkv(workloads.seed_for(w.index, "v_new"), w.unit_tokens, H, D, 0.5, "bf16")
    bca.kv_append(g, k.cuda(), v.cuda())
    assert g.n_tokens == n0 + w.unit_tokens
    torch.cuda.synchronize()
    kb = k.view(torch.int16).numpy()
    vb = v.view(torch.int16).numpy()
    kp = g.k_pages.view(torch.int16).cpu().numpy()
    vp = g.v_pages.view(torch.int16).cpu().numpy()
    ptn = pt.numpy()
    for lp in range(n0 // ps, n_log):
        t0 = lp * ps
        r1 = min(ps, n0 + w.unit_tokens - t0)
        page = ptn[lp]
        np.testing.assert_array_equal(kp[page, :, :r1, :], kb[t0 - n0:t0 - n0 + r1].transpose(1, 0, 2))
        np.testing.assert_array_equal(vp[page, :, :, :r1], vb[t0 - n0:t0 - n0 + r1].transpose(1, 2, 0))
        assert not kp[page, :, r1:, :].any() and not vp[page, :, :, r1:].any()
    # pages before the append were not touched
    untouched = ptn[: n0 // ps]
    assert not kp[untouched].any() and not vp[untouched].any()
