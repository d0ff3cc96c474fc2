"""Streaming sessions (bca_session_*): many consecutive performer units over
one growing cache, physical pages taken from a free list as the cache
grows, units that start inside a partly filled page, and the unit replayed
as a HIP graph.  Every unit is checked against the oracle's performer unit
on a cache with the same logical contents; graph and eager runs of the same
sequence must agree bit for bit, unit after unit (each graph replay follows
eager work and a synchronisation)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, assert_latents, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")


def _run_small(use_graph):
    H, D, ps, n_unit, n_units, S = 2, 128, 64, 100, 5, 4
    n_phys = 12
    free = torch.randperm(n_phys, generator=torch.Generator().manual_seed(11)).tolist()
    pt = torch.full((n_phys,), -1, dtype=torch.int32)
    g = bca.KVCache(H, D, ps, pt, n_phys, "bf16")
    ss = bca.Session(g, free)
    w = workloads.randn((H * D, 16), 21)
    ws = bca.alloc_workspace(bca.workspace_bytes(g, n_unit, n_units * n_unit, 16))
    outs = []
    for u in range(n_units):
        k = workloads.qkv(100 + u, n_unit, H, D, 0.5, "bf16")
        v = workloads.qkv(200 + u, n_unit, H, D, 0.5, "bf16")
        q = workloads.qkv(300 + u, n_unit, H, D, 0.5, "bf16")
        eps = workloads.randn((n_unit, 16), 400 + u)
        z = eps.clone().cuda()
        osc = torch.empty((n_unit, H, D), dtype=torch.bfloat16, device="cuda")
        ss.unit(k.cuda(), v.cuda(), q.cuda(), w.cuda(), z, S, osc, workspace=ws, use_graph=use_graph)
        torch.cuda.synchronize()
        outs.append((k, v, q, eps, osc.clone(), z.clone()))
    pages_used = -(-n_units * n_unit // ps)
    assert ss.free_pages == n_phys - pages_used
    assert g.page_table[:pages_used].cpu().tolist() == free[:pages_used]
    assert g.n_tokens == n_units * n_unit
    ss.close()
    return free, w, outs


@pytest.mark.parametrize("use_graph", [False, True])
def test_session_small_units_against_oracle(use_graph):
    say(f"session small units graph={use_graph}")
    free, w, outs = _run_small(use_graph)
    H, D, ps, S = 2, 128, 64, 4
    ref = oracle.PagedCache(H, D, ps, free, len(free))
    for u, (k, v, q, eps, osc, z) in enumerate(outs):
        z_want, o_want = oracle.performer_unit(ref, k.double().numpy(), v.double().numpy(),
                                               q.double().numpy(), w.double().numpy(),
                                               eps.double().numpy(), S)
        assert_close(osc.float().cpu().numpy(), o_want, 2e-2, 1e-2, what=f"unit {u} O")
        assert_latents(z.cpu().numpy(), z_want, eps.double().numpy(), 2e-2, 1e-2, what=f"unit {u}")


def test_session_graph_equals_eager():
    say("session graph vs eager, bitwise")
    _, _, eager = _run_small(False)
    _, _, graph = _run_small(True)
    for u, (a, b) in enumerate(zip(eager, graph)):
        assert torch.equal(a[4], b[4]), f"unit {u} O"
        assert torch.equal(a[5], b[5]), f"unit {u} z"


def test_session_v02_units_sampled_rows():
    """Three v0.2 units (3712 tokens = 14.5 pages each, so the second starts
    mid-page) on top of the 32-unit v0.2 history, replayed as graphs; every
    unit's O and z on sampled rows against the oracle over all keys."""
    say("session v0.2 units")
    w_ = workloads.WORKLOADS["v02_unit"]
    H, D, ps, lq, S = w_.n_heads, w_.head_dim, w_.page_size, w_.unit_tokens, w_.n_steps
    n_units = 3
    n_hist_pages = w_.n_hist // ps
    n_log = n_hist_pages + -(-n_units * lq // ps)
    n_phys = n_log + 8
    perm = torch.randperm(n_phys, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    pt = torch.full((n_log,), -1, dtype=torch.int32)
    pt[:n_hist_pages] = perm[:n_hist_pages]
    g = bca.KVCache(H, D, ps, pt, n_phys, "bf16")
    inp = workloads.make_unit_inputs(w_, device="cuda")
    bca.kv_append(g, inp["k_hist"], inp["v_hist"])
    ss = bca.Session(g, perm[n_hist_pages:].tolist())
    ws = bca.alloc_workspace(bca.workspace_bytes(g, lq, w_.n_hist + n_units * lq, w_.n_ch))
    rows = np.array([0, 1, 255, 256, 1855, 3583, 3711])
    k_all = [inp["k_hist"]]
    v_all = [inp["v_hist"]]
    for u in range(n_units):
        k = workloads.qkv(500 + u, lq, H, D, w_.qkv_scale, "bf16", "cuda")
        v = workloads.qkv(600 + u, lq, H, D, w_.qkv_scale, "bf16", "cuda")
        q = workloads.qkv(700 + u, lq, H, D, w_.qkv_scale, "bf16", "cuda")
        z = inp["eps"].clone()
        osc = torch.empty((lq, H, D), dtype=torch.bfloat16, device="cuda")
        ss.unit(k, v, q, inp["w"], z, S, osc, workspace=ws, use_graph=True)
        torch.cuda.synchronize()
        k_all.append(k)
        v_all.append(v)
        K = torch.cat(k_all)
        V = torch.cat(v_all)
        qs = q[rows.tolist()].float().cpu().numpy().astype(np.float64)
        o_want = np.zeros((len(rows), H, D))
        for h in range(H):
            kh = K[:, h].float().cpu().numpy().astype(np.float64)[:, None]
            vh = V[:, h].float().cpu().numpy().astype(np.float64)[:, None]
            o_want[:, h] = oracle.attention_dense(qs[:, None, h], kh, vh)[:, 0]
        vel = oracle.velocity(o_want, inp["w"].double().cpu().numpy())
        eps = inp["eps"][rows.tolist()].double().cpu().numpy()
        z_want = oracle.euler_solve(eps, lambda zz, tau: vel, S)
        assert_close(osc[rows.tolist()].float().cpu().numpy(), o_want, 2e-2, 1e-2, what=f"unit {u} O")
        assert_latents(z[rows.tolist()].cpu().numpy(), z_want, eps, 2e-2, 1e-2, what=f"unit {u}")
    assert g.n_tokens == w_.n_hist + n_units * lq
    assert g.page_table[n_hist_pages:n_log].cpu().tolist() == perm[n_hist_pages:n_log].tolist()
    ss.close()


def test_captured_performer_unit_replays_match_eager():
    """A caller captures one performer_unit (append + 4 x (attention with the
    work queues and split combine, Euler with its partial sums)) into a
    graph on its own stream and replays it three times, with eager work and
    a synchronisation between replays (z reset, the cache rolled back on the
    host); every replay must equal the eager unit bit for bit."""
    say("captured performer_unit replays")
    H, D, ps, n_hist, n_q, S = 4, 128, 64, 700, 300, 4
    k = workloads.qkv(31, n_hist + n_q, H, D, 0.5, "bf16").cuda()
    v = workloads.qkv(32, n_hist + n_q, H, D, 0.5, "bf16").cuda()
    q = workloads.qkv(33, n_q, H, D, 0.5, "bf16").cuda()
    w = workloads.randn((H * D, 16), 34).cuda()
    eps = workloads.randn((n_q, 16), 35).cuda()
    n_pages = -(-(n_hist + n_q) // ps)
    pt = torch.randperm(n_pages, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    g = bca.KVCache(H, D, ps, pt, n_pages, "bf16")
    bca.kv_append(g, k[:n_hist], v[:n_hist])
    ws = bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_hist + n_q, 16))
    osc = torch.empty((n_q, H, D), dtype=torch.bfloat16, device="cuda")
    z = eps.clone()
    bca.performer_unit(g, k[n_hist:], v[n_hist:], q, w, z, S, o_scratch=osc, workspace=ws)
    torch.cuda.synchronize()
    z_eager, o_eager = z.clone(), osc.clone()
    # the 700-token history is not a multiple of the 300-token unit: the
    # unit's queries still see every cached key, their whole slice included
    ref = oracle.PagedCache(H, D, ps, pt.numpy(), n_pages)
    ref.append(k[:n_hist].double().cpu().numpy(), v[:n_hist].double().cpu().numpy())
    z_want, o_want = oracle.performer_unit(ref, k[n_hist:].double().cpu().numpy(),
                                           v[n_hist:].double().cpu().numpy(), q.double().cpu().numpy(),
                                           w.double().cpu().numpy(), eps.double().cpu().numpy(), S)
    assert_close(o_eager.float().cpu().numpy(), o_want, 2e-2, 1e-2, what="eager unit O")
    assert_latents(z_eager.cpu().numpy(), z_want, eps.double().cpu().numpy(), 2e-2, 1e-2,
                   what="eager unit")

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    g.c.n_tokens = n_hist
    z.copy_(eps)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        bca.performer_unit(g, k[n_hist:], v[n_hist:], q, w, z, S, o_scratch=osc, workspace=ws)
    for rep in range(3):
        g.c.n_tokens = n_hist
        z.copy_(eps)
        osc.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(z, z_eager), f"replay {rep} z"
        assert torch.equal(osc, o_eager), f"replay {rep} O"


def test_session_graph_units_back_to_back():
    """Five graph units enqueued without a host synchronisation between them
    (distinct z and O buffers, units of 100 tokens on 64-token pages, so
    most start mid-page and their shapes alternate between mapping a new
    page and not).  A unit's graph is rewritten only after its previous
    launch has finished, so no queued unit runs with a later unit's
    arguments: every unit matches the oracle's unit over the same cache."""
    say("session graph units back to back")
    H, D, ps, n_unit, n_units, S = 2, 128, 64, 100, 5, 4
    n_phys = 12
    free = torch.randperm(n_phys, generator=torch.Generator().manual_seed(13)).tolist()
    pt = torch.full((n_phys,), -1, dtype=torch.int32)
    g = bca.KVCache(H, D, ps, pt, n_phys, "bf16")
    ss = bca.Session(g, free)
    w = workloads.randn((H * D, 16), 23)
    ws = bca.alloc_workspace(bca.workspace_bytes(g, n_unit, n_units * n_unit, 16))
    units = []
    for u in range(n_units):
        k = workloads.qkv(110 + u, n_unit, H, D, 0.5, "bf16")
        v = workloads.qkv(210 + u, n_unit, H, D, 0.5, "bf16")
        q = workloads.qkv(310 + u, n_unit, H, D, 0.5, "bf16")
        eps = workloads.randn((n_unit, 16), 410 + u)
        dev = [t.cuda() for t in (k, v, q)]
        z = eps.clone().cuda()
        osc = torch.empty((n_unit, H, D), dtype=torch.bfloat16, device="cuda")
        ss.unit(dev[0], dev[1], dev[2], w.cuda(), z, S, osc, workspace=ws, use_graph=True)
        units.append((k, v, q, eps, dev, z, osc))
    torch.cuda.synchronize()
    assert g.n_tokens == n_units * n_unit
    assert g.page_table[: -(-n_units * n_unit // ps)].cpu().tolist() == free[: -(-n_units * n_unit // ps)]
    ss.close()
    ref = oracle.PagedCache(H, D, ps, free, len(free))
    for u, (k, v, q, eps, _, z, osc) in enumerate(units):
        z_want, o_want = oracle.performer_unit(ref, k.double().numpy(), v.double().numpy(),
                                               q.double().numpy(), w.double().numpy(),
                                               eps.double().numpy(), S)
        assert_close(osc.float().cpu().numpy(), o_want, 2e-2, 1e-2, what=f"unit {u} O")
        assert_latents(z.cpu().numpy(), z_want, eps.double().numpy(), 2e-2, 1e-2, what=f"unit {u}")
