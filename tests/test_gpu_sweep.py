"""Seeded sweeps against the oracle over shapes drawn at random (fixed
seeds, so every run checks the same cases).

block_causal_attn: 1-3 heads, head dims 64 and 128, page sizes 16-256 with
shuffled page tables, key counts from 1 to 5000 (so every remainder of key
tiles per split and per unrolled loop body turns up), query counts and
positions, block sizes from causal (1) to all-visible, with and without a
workspace; bf16 caches, and fp8 caches (head dim 128, pages of 64+ keys).
Bars as in the other attention tests: bf16 max-abs 2e-2 and relative RMS
1e-2, fp8 max-abs 3e-2 and relative RMS 1e-2, against the oracle's
dense-mask attention over the keys as the cache holds them.

kv_append: random sequences of appends into bf16, fp32 and fp8 caches, bit
for bit.  performer_unit: random unit, history, step and channel counts.
Streaming sessions: random unit lengths, page sizes, dtypes, graph or eager."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, assert_latents, make_caches, np64, say

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


N_APPEND = 24


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


@pytest.mark.parametrize("i", range(N_APPEND))
def test_sweep_append(i):
    """Random sequences of 1-6 appends (1-600 tokens each, any start within a
    page) into bf16, fp32 and fp8 caches with shuffled page tables: after
    each append every page equals the oracle's bit for bit (fp8: the codes
    and scales of every page written so far, partly filled pages being
    re-quantised by later appends; the values' scale changes from append to
    append so the scales grow and shrink)."""
    r = np.random.default_rng(8000 + i)
    dt = str(r.choice(["bf16", "f32", "fp8"]))
    H = int(r.integers(1, 5))
    D = 128 if dt == "fp8" else int(r.choice([64, 128] if dt == "bf16" else [32, 64]))
    ps = int(r.choice([64, 128, 256] if dt == "fp8" else [16, 32, 64, 256]))
    sizes = [int(x) for x in r.integers(1, 601, size=int(r.integers(1, 7)))]
    shuffle = int(r.integers(1, 1000))
    say(f"sweep append case {i}: {dt} H={H} D={D} ps={ps} sizes={sizes}")
    g, o, _ = make_caches(bca, H, D, ps, dt, sum(sizes), shuffle)
    for j, n in enumerate(sizes):
        sc = float(r.choice([0.05, 0.5, 3.0]))
        src = "f32" if dt == "f32" else "bf16"
        k = workloads.qkv(20000 + 100 * i + j, n, H, D, sc, src)
        v = workloads.qkv(30000 + 100 * i + j, n, H, D, sc, src)
        bca.kv_append(g, k.cuda(), v.cuda())
        o.append(k.double().numpy() if dt != "fp8" else k.float().numpy(),
                 v.double().numpy() if dt != "fp8" else v.float().numpy())
        assert g.n_tokens == o.n_tokens
        torch.cuda.synchronize()
        if dt == "fp8":
            pages = g.page_table.cpu().numpy()[: -(-o.n_tokens // ps)]
            np.testing.assert_array_equal(g.k_pages.cpu().numpy()[pages], o.k_codes[pages])
            np.testing.assert_array_equal(g.v_pages.cpu().numpy()[pages], o.v_codes[pages])
            np.testing.assert_array_equal(g.k_scales.cpu().numpy()[pages], o.k_scales[pages])
            np.testing.assert_array_equal(g.v_scales.cpu().numpy()[pages], o.v_scales[pages])
        else:
            want_k = torch.from_numpy(o.k_pages).to(torch.bfloat16 if dt == "bf16" else torch.float32)
            want_v = torch.from_numpy(o.v_pages).to(torch.bfloat16 if dt == "bf16" else torch.float32)
            np.testing.assert_array_equal(_bits(g.k_pages), _bits(want_k))
            np.testing.assert_array_equal(_bits(g.v_pages), _bits(want_v))


N_UNIT = 16


@pytest.mark.parametrize("i", range(N_UNIT))
def test_sweep_performer_unit(i):
    """performer_unit on random shapes: 1-4 heads, unit lengths 1-200, a
    history of 0-3000 tokens (rarely a multiple of the unit), 1-6 solver
    steps, 3-16 latent channels, page sizes 16-256, with and without a
    workspace; bf16, fp32 and fp8 caches.  O and z (and the solver's move
    z - eps) against the oracle's performer unit on all rows."""
    r = np.random.default_rng(8500 + i)
    dt = str(r.choice(["bf16", "f32", "fp8"]))
    H = int(r.integers(1, 5))
    D = 128 if dt == "fp8" else int(r.choice([64, 128]))
    ps = int(r.choice([64, 256] if dt == "fp8" else [16, 64, 256]))
    lq = int(r.integers(1, 201))
    n_hist = int(r.integers(0, 3001))
    S = int(r.integers(1, 7))
    C = int(r.choice([3, 8, 16]))
    with_ws = bool(r.integers(0, 2))
    shuffle = int(r.integers(1, 1000))
    say(f"sweep unit case {i}: {dt} H={H} D={D} ps={ps} lq={lq} hist={n_hist} S={S} C={C} ws={with_ws}")
    cap = n_hist + lq
    g, o, _ = make_caches(bca, H, D, ps, dt, cap, shuffle)
    src = "f32" if dt == "f32" else "bf16"
    seed = 40000 + 10 * i
    q = workloads.qkv(seed, lq, H, D, 0.5, src)
    kh = workloads.qkv(seed + 1, n_hist, H, D, 0.5, src)
    vh = workloads.qkv(seed + 2, n_hist, H, D, 0.5, src)
    kn = workloads.qkv(seed + 3, lq, H, D, 0.5, src)
    vn = workloads.qkv(seed + 4, lq, H, D, 0.5, src)
    eps = workloads.randn((lq, C), seed + 5)
    w = workloads.randn((H * D, C), seed + 6)
    if n_hist:
        bca.kv_append(g, kh.cuda(), vh.cuda())
        o.append(kh.double().numpy(), vh.double().numpy())
    z = eps.clone().cuda()
    ws = bca.alloc_workspace(bca.workspace_bytes(g, lq, cap, C)) if with_ws else None
    osc = torch.empty((lq, H, D), dtype=g.compute_dtype, device="cuda")
    bca.performer_unit(g, kn.cuda(), vn.cuda(), q.cuda(), w.cuda(), z, S, o_scratch=osc, workspace=ws)
    zw, ow = oracle.performer_unit(o, kn.double().numpy(), vn.double().numpy(), q.double().numpy(),
                                   w.double().numpy(), eps.double().numpy(), S)
    e = eps.double().numpy()
    if dt == "f32":
        assert_close(np64(osc), ow, 1e-4, what=f"unit case {i} O")
        assert_latents(np64(z), zw, e, 1e-4, 1e-4, what=f"unit case {i}")
    else:
        tol = 3e-2 if dt == "fp8" else 2e-2
        assert_close(np64(osc), ow, tol, 1e-2, what=f"unit case {i} O")
        assert_latents(np64(z), zw, e, tol, 1e-2, what=f"unit case {i}")


N_SESSION = 8


@pytest.mark.parametrize("i", range(N_SESSION))
def test_sweep_session(i):
    """Streaming sessions on random shapes: 3-6 units of random and varying
    lengths (1-300 tokens, so units start anywhere inside pages), pages of
    16-256 tokens taken from a shuffled free list, bf16 or fp8 caches, 1-4
    solver steps, eager or replayed as HIP graphs.  Each unit's O and z
    against the oracle's performer unit over a cache with the same logical
    contents; the free-page count and the page table at the end."""
    r = np.random.default_rng(8800 + i)
    dt = str(r.choice(["bf16", "fp8"]))
    H = int(r.integers(1, 4))
    D = 128
    ps = int(r.choice([64, 256] if dt == "fp8" else [16, 64, 256]))
    lens = [int(x) for x in r.integers(1, 301, size=int(r.integers(3, 7)))]
    S = int(r.integers(1, 5))
    C = int(r.choice([8, 16]))
    use_graph = bool(r.integers(0, 2))
    total = sum(lens)
    n_phys = -(-total // ps) + 2
    free = [int(x) for x in r.permutation(n_phys)]
    say(f"sweep session case {i}: {dt} H={H} ps={ps} lens={lens} S={S} C={C} graph={use_graph}")
    pt = torch.full((n_phys,), -1, dtype=torch.int32)
    g = bca.KVCache(H, D, ps, pt, n_phys, dt)
    ss = bca.Session(g, free)
    ref = (oracle.PagedCacheFP8 if dt == "fp8" else oracle.PagedCache)(H, D, ps, free, n_phys)
    w = workloads.randn((H * D, C), 50000 + i)
    ws = bca.alloc_workspace(bca.workspace_bytes(g, max(lens), total, C))
    tol = 3e-2 if dt == "fp8" else 2e-2
    for u, n in enumerate(lens):
        seed = 51000 + 100 * i + 10 * u
        k = workloads.qkv(seed, n, H, D, 0.5, "bf16")
        v = workloads.qkv(seed + 1, n, H, D, 0.5, "bf16")
        q = workloads.qkv(seed + 2, n, H, D, 0.5, "bf16")
        eps = workloads.randn((n, C), seed + 3)
        z = eps.clone().cuda()
        osc = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
        ss.unit(k.cuda(), v.cuda(), q.cuda(), w.cuda(), z, S, osc, workspace=ws, use_graph=use_graph)
        torch.cuda.synchronize()
        z_want, o_want = oracle.performer_unit(ref, k.double().numpy(), v.double().numpy(),
                                               q.double().numpy(), w.double().numpy(),
                                               eps.double().numpy(), S)
        assert_close(np64(osc), o_want, tol, 1e-2, what=f"session case {i} unit {u} O")
        assert_latents(np64(z), z_want, eps.double().numpy(), tol, 1e-2, what=f"session case {i} unit {u}")
    used = -(-total // ps)
    assert ss.free_pages == n_phys - used
    assert g.page_table[:used].cpu().tolist() == free[:used]
    assert g.n_tokens == total
    ss.close()
