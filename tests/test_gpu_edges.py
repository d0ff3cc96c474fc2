"""Degenerate and boundary calls through the C ABI: one query over one key
(the output is that key's value exactly, whatever the logit), a zero-length
append (no-op), an Euler step over zero tokens, a one-token performer unit on
an empty cache, and key counts that end exactly on a 64-key tile or a page,
with and without a workspace."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, assert_latents, make_caches, np64, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ws", [False, True])
def test_one_query_one_key(dtype, ws):
    H, D = 2, 128 if dtype == "bf16" else 64
    say(f"edge: one query one key {dtype} ws={ws}")
    g, _, _ = make_caches(bca, H, D, 64, dtype, 1)
    k = workloads.qkv(1, 1, H, D, 3.0, dtype)
    v = workloads.qkv(2, 1, H, D, 1.0, dtype)
    q = workloads.qkv(3, 1, H, D, 3.0, dtype)
    bca.kv_append(g, k.cuda(), v.cuda())
    w = bca.alloc_workspace(bca.workspace_bytes(g, 1, 1)) if ws else None
    out = bca.block_causal_attn(q.cuda(), g, workspace=w)
    torch.cuda.synchronize()
    # softmax over one key is 1: the output is v itself (bf16 output of a bf16 v is exact)
    np.testing.assert_array_equal(np64(out), np64(v))


def test_zero_length_append_and_empty_euler():
    say("edge: zero-length append, empty Euler step")
    H, D = 2, 128
    g, _, _ = make_caches(bca, H, D, 64, "bf16", 64)
    e = torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda")
    bca.kv_append(g, e, e)
    assert g.n_tokens == 0
    z = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    bca.fm_euler_step(z, torch.empty((0, 16), dtype=torch.float32, device="cuda"), None, 0.25)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_one_token_unit_on_empty_cache(dtype):
    """The smallest unit: one token appended to an empty cache; its query
    sees only itself, so O equals its value (fp8: its value as stored)."""
    H, D = 2, 128 if dtype != "f32" else 64
    say(f"edge: one-token unit {dtype}")
    g, o, _ = make_caches(bca, H, D, 64, dtype, 1)
    src = "f32" if dtype == "f32" else "bf16"
    k = workloads.qkv(11, 1, H, D, 0.5, src)
    v = workloads.qkv(12, 1, H, D, 0.5, src)
    q = workloads.qkv(13, 1, H, D, 0.5, src)
    w = workloads.randn((H * D, 16), 14)
    eps = workloads.randn((1, 16), 15)
    z = eps.clone().cuda()
    osc = torch.empty((1, H, D), dtype=g.compute_dtype, device="cuda")
    bca.performer_unit(g, k.cuda(), v.cuda(), q.cuda(), w.cuda(), z, 4, o_scratch=osc,
                       workspace=bca.alloc_workspace(bca.workspace_bytes(g, 1, 1)))
    torch.cuda.synchronize()
    zw, ow = oracle.performer_unit(o, k.double().numpy() if dtype != "fp8" else k.float().numpy(),
                                   v.double().numpy() if dtype != "fp8" else v.float().numpy(),
                                   q.double().numpy(), w.double().numpy(), eps.double().numpy(), 4)
    tol = 1e-4 if dtype == "f32" else (3e-2 if dtype == "fp8" else 2e-2)
    assert_close(np64(osc), ow, tol, what=f"one-token O {dtype}")
    assert_latents(np64(z), zw, eps.double().numpy(), tol, 1e-2, what=f"one-token {dtype}")


@pytest.mark.parametrize("n_kv", [64, 256, 320, 4096])
@pytest.mark.parametrize("ws", [False, True])
def test_key_count_on_tile_and_page_edges(n_kv, ws):
    """n_kv a whole number of 64-key tiles and of 64/256-key pages: no tail
    tile, the last tile fully visible."""
    H, D, n_q = 2, 128, min(n_kv, 100)
    say(f"edge: n_kv={n_kv} ws={ws}")
    q = workloads.qkv(21, n_q, H, D, 0.5, "bf16")
    k = workloads.qkv(22, n_kv, H, D, 0.5, "bf16")
    v = workloads.qkv(23, n_kv, H, D, 1.0, "bf16")
    g, _, _ = make_caches(bca, H, D, 64, "bf16", n_kv, 3)
    bca.kv_append(g, k.cuda(), v.cuda())
    w = bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv)) if ws else None
    out = bca.block_causal_attn(q.cuda(), g, workspace=w)
    want = oracle.attention_dense(q.double().numpy(), k.double().numpy(), v.double().numpy())
    assert_close(np64(out), want, 2e-2, 1e-2, what=f"n_kv={n_kv}")
