"""Seeded sweep of block_causal_attn over call shapes drawn at random against
the oracle: 1-3 heads, head dims 64 and 128, page sizes 16-256 with shuffled
page tables, key counts from 1 to 5000 (so every remainder of key tiles per
split and per unrolled loop body turns up), query counts and positions,
block sizes from causal (1) to all-visible, with and without a workspace;
bf16 caches, and fp8 caches (head dim 128, pages of 64+ keys).  The shapes
come from fixed seeds, so every run checks the same cases.  Bars as in the
other attention tests: bf16 max-abs 2e-2 and relative RMS 1e-2, fp8 max-abs
3e-2 and relative RMS 1e-2, against the oracle's dense-mask attention over
the keys as the cache holds them."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, make_caches, np64, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")

N_BF16, N_FP8 = 40, 16


def _shape(i, fp8):
    r = np.random.default_rng(7000 + i + (1000 if fp8 else 0))
    H = int(r.integers(1, 4))
    D = 128 if fp8 else int(r.choice([64, 128]))
    ps = int(r.choice([64, 128, 256] if fp8 else [16, 32, 64, 128, 256]))
    n_kv = int(r.integers(1, 5001))
    n_q = int(r.integers(1, min(n_kv, 300) + 1))
    q_pos0 = int(r.integers(0, n_kv - n_q + 1))
    B = int(r.choice([1, 7, 64, 100, 333, n_kv]))
    ws = bool(r.integers(0, 2))
    shuffle = int(r.integers(1, 1000))
    return H, D, ps, n_kv, n_q, q_pos0, B, ws, shuffle


def _run(i, fp8):
    H, D, ps, n_kv, n_q, q_pos0, B, ws, shuffle = _shape(i, fp8)
    dt = "fp8" if fp8 else "bf16"
    say(f"sweep {dt} case {i}: H={H} D={D} ps={ps} n_kv={n_kv} n_q={n_q} q_pos0={q_pos0} B={B} ws={ws}")
    seed = 9000 + 10 * i + (5000 if fp8 else 0)
    k = workloads.qkv(seed, n_kv, H, D, 0.5, "bf16")
    v = workloads.qkv(seed + 1, n_kv, H, D, 0.5, "bf16")
    q = workloads.qkv(seed + 2, n_q, H, D, 0.5, "bf16")
    g, o, _ = make_caches(bca, H, D, ps, dt, n_kv, shuffle)
    bca.kv_append(g, k.cuda(), v.cuda())
    work = bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv)) if ws else None
    out = bca.block_causal_attn(q.cuda(), g, n_kv=n_kv, q_pos0=q_pos0, block_size=B, workspace=work)
    if fp8:
        o.append(k.float().numpy(), v.float().numpy())
        K, V = o.gather()
    else:
        K, V = k.double().numpy(), v.double().numpy()
    want = oracle.attention_dense(q.double().numpy(), K, V, q_pos0, B)
    tol = 3e-2 if fp8 else 2e-2
    assert_close(np64(out), want, tol, 1e-2, what=f"sweep {dt} case {i}")


@pytest.mark.parametrize("i", range(N_BF16))
def test_sweep_bf16(i):
    _run(i, False)


@pytest.mark.parametrize("i", range(N_FP8))
def test_sweep_fp8(i):
    _run(i, True)
