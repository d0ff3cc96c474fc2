"""performer_unit parity: append + n_steps x (attention, Euler) against the
oracle's performer_unit, on small shapes and on the v0.1 unit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, assert_latents, make_caches, np64, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")


def _run(H, D, lq, hist_units, ps, dtype, shuffle, qkv_scale, seed, rows=None, with_ws=True):
    n_hist = hist_units * lq
    cap = n_hist + lq
    g, o, _ = make_caches(bca, H, D, ps, dtype, cap, shuffle)
    q = workloads.qkv(seed, lq, H, D, qkv_scale, dtype)
    kh = workloads.qkv(seed + 1, n_hist, H, D, qkv_scale, dtype)
    vh = workloads.qkv(seed + 2, n_hist, H, D, qkv_scale, dtype)
    kn = workloads.qkv(seed + 3, lq, H, D, qkv_scale, dtype)
    vn = workloads.qkv(seed + 4, lq, H, D, qkv_scale, dtype)
    eps = workloads.randn((lq, 16), seed + 5)
    w = workloads.randn((H * D, 16), seed + 7)
    if n_hist:
        bca.kv_append(g, kh.cuda(), vh.cuda())
        o.append(kh.double().numpy(), vh.double().numpy())
    z = eps.clone().cuda()
    ws = bca.alloc_workspace(bca.workspace_bytes(g, lq, cap)) if with_ws else None
    osc = torch.empty((lq, H, D), dtype=g.compute_dtype, device="cuda")
    bca.performer_unit(g, kn.cuda(), vn.cuda(), q.cuda(), w.cuda(), z, 4, o_scratch=osc,
                       workspace=ws)
    assert g.n_tokens == cap
    zw, ow = oracle.performer_unit(o, kn.double().numpy(), vn.double().numpy(),
                                   q.double().numpy(), w.double().numpy(),
                                   eps.double().numpy(), 4, rows=rows)
    zg, og = np64(z), np64(osc)
    e = eps.double().numpy()
    if rows is not None:
        zg, og, e = zg[rows], og[rows], e[rows]
    return zg, og, zw, ow, e


@pytest.mark.parametrize("dtype,D,tol_o,tol_z", [("bf16", 128, 2e-2, 2e-2), ("f32", 64, 1e-4, 1e-4)])
@pytest.mark.parametrize("ps,shuffle", [(256, None), (16, 6)])
def test_small_unit(dtype, D, tol_o, tol_z, ps, shuffle):
    say(f"performer small dtype={dtype} ps={ps}")
    zg, og, zw, ow, e = _run(4, D, 48, 5, ps, dtype, shuffle, 0.5, 60)
    assert_close(og, ow, tol_o, 1e-2 if dtype == "bf16" else None, what="O")
    assert_latents(zg, zw, e, tol_z, 1e-2 if dtype == "bf16" else 1e-4, what="unit")


def test_v01_unit_sampled_rows():
    """v0.1-shaped unit (24 heads x 128, 1024 tokens, 64 history units,
    256-token pages), rows sampled across the unit."""
    w = workloads.WORKLOADS["v01_unit"]
    rows = np.array([0, 1, 255, 256, 511, 700, 1007, 1023])
    say("performer v0.1 unit")
    zg, og, zw, ow, e = _run(w.n_heads, w.head_dim, w.unit_tokens, w.hist_units, 256, "bf16", 21,
                             w.qkv_scale, 1000, rows=rows)
    assert_close(og, ow, 2e-2, 1e-2, what="O v0.1")
    assert_latents(zg, zw, e, 2e-2, 1e-2, what="v0.1 unit")
