"""fp8 (E4M3FN) KV cache parity: the quantiser bit for bit (codes and
scales) against the oracle's, and attention over the fp8 cache against the
oracle's attention on the K/V that the oracle itself quantised and
dequantised (max-abs 3e-2, relative RMS 1e-2)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import fp8c
from _helpers import assert_close, assert_latents, make_caches, np64, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")

FP8_TOL = 3e-2
FP8_REL = 1e-2


def _crafted_page(ps, H, D, seed):
    """bf16 values on purpose: amax 448 (inv = 1 exactly), round-half-even
    ties between E4M3 neighbours (1.0625, 17, 2^-10, 3*2^-10, 232), values
    that round up into the next binade (1.9375 -> 2), negatives and zeros."""
    rng = np.random.default_rng(seed)
    ties = np.array([1.0625, 17.0, 2.0 ** -10, 3 * 2.0 ** -10, 232.0, 1.9375, 0.0, 448.0,
                     -1.0625, -17.0, -(2.0 ** -10), -232.0, 2.0 ** -12, 300.0, -448.0, 0.5])
    x = rng.choice(ties, size=(ps, H, D))
    x[0, :, 0] = 448.0
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def _bits_equal(g: bca.KVCache, o, n_tok, ps):
    """Codes of every page the appends touched, and their scales."""
    pt = g.page_table.cpu().numpy()
    pages = pt[: -(-n_tok // ps)]
    kg = g.k_pages.cpu().numpy()[pages]
    vg = g.v_pages.cpu().numpy()[pages]
    np.testing.assert_array_equal(kg, o.k_codes[pages])
    np.testing.assert_array_equal(vg, o.v_codes[pages])
    np.testing.assert_array_equal(g.k_scales.cpu().numpy()[pages], o.k_scales[pages])
    np.testing.assert_array_equal(g.v_scales.cpu().numpy()[pages], o.v_scales[pages])


@pytest.mark.parametrize("ps,shuffle", [(256, None), (64, 5), (128, 3)])
def test_fp8_append_bit_exact(ps, shuffle):
    """Page-aligned appends (several whole pages, then one ending mid-page)
    of random bf16 K/V plus a crafted page of ties, zeros and the 448
    bound: codes and per-(page, head) scales equal the oracle's."""
    H, D = 3, 128
    say(f"fp8 append ps={ps} shuffle={shuffle}")
    sizes = [3 * ps, ps, ps + 37]
    g, o, _ = make_caches(bca, H, D, ps, "fp8", sum(sizes), shuffle)
    for i, n in enumerate(sizes):
        k = workloads.qkv(300 + i, n, H, D, 0.5, "bf16")
        v = workloads.qkv(400 + i, n, H, D, 0.5, "bf16")
        if i == 1:
            k = _crafted_page(ps, H, D, 1)
            v = _crafted_page(ps, H, D, 2)
            v[:, 1, :] = 0                      # an all-zero (page, head): scale 1, codes 0
        bca.kv_append(g, k.cuda(), v.cuda())
        o.append(k.float().numpy(), v.float().numpy())
        assert g.n_tokens == o.n_tokens
    torch.cuda.synchronize()
    _bits_equal(g, o, sum(sizes), ps)


def test_fp8_append_zero_blocks():
    """A (page, head) block of zeros, negative zeros among them, gets scale 1
    and codes 0, as the oracle's quantiser defines for amax = 0; a block of
    only -0 beside a normal one in the same page."""
    H, D, ps = 2, 128, 64
    x = torch.zeros((ps, H, D), dtype=torch.bfloat16)
    x[::3, 0] = -0.0                           # head 0: zeros and negative zeros
    x[:, 1] = workloads.qkv(71, ps, 1, D, 0.5, "bf16")[:, 0]
    y = torch.full((ps, H, D), -0.0, dtype=torch.bfloat16)
    g, o, _ = make_caches(bca, H, D, ps, "fp8", ps, None)
    bca.kv_append(g, x.cuda(), y.cuda())
    o.append(x.float().numpy(), y.float().numpy())
    torch.cuda.synchronize()
    _bits_equal(g, o, ps, ps)
    assert g.k_scales[0, 0].item() == 1.0 and g.v_scales[0, 0].item() == 1.0


@pytest.mark.parametrize("ps,shuffle,sizes,grow", [
    (64, None, [10, 5, 100, 49], [1.0, 4.0, 0.25, 1.0]),
    (128, 3, [200, 1, 127, 300], [1.0, 0.5, 8.0, 1.0]),
    (256, 7, [37, 219, 256, 3], [1.0, 2.0, 1.0, 16.0]),
])
def test_fp8_append_inside_a_page_requantises(ps, shuffle, sizes, grow):
    """Appends that start inside a partly filled page: the page is quantised
    afresh over its held rows (their values as held) and the new ones, as
    the oracle defines; codes and scales of every touched page equal the
    oracle's bit for bit after each append, whether the new rows are larger
    (the scale grows and the held rows move onto a coarser grid) or smaller
    than the held ones.  Then attention over the cache against the oracle's
    over its own dequantised K/V."""
    H, D = 3, 128
    say(f"fp8 mid-page appends ps={ps} sizes={sizes}")
    g, o, _ = make_caches(bca, H, D, ps, "fp8", sum(sizes), shuffle)
    for i, (n, f) in enumerate(zip(sizes, grow)):
        k = workloads.qkv(500 + i, n, H, D, 0.5 * f, "bf16")
        v = workloads.qkv(600 + i, n, H, D, 0.5 / f, "bf16")
        bca.kv_append(g, k.cuda(), v.cuda())
        o.append(k.float().numpy(), v.float().numpy())
        assert g.n_tokens == o.n_tokens
        torch.cuda.synchronize()
        _bits_equal(g, o, o.n_tokens, ps)
    n_kv, n_q = o.n_tokens, 64
    q = workloads.qkv(700, n_q, H, D, 0.5, "bf16")
    out = bca.block_causal_attn(q.cuda(), g, workspace=bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv)))
    K, V = o.gather()
    want = oracle.attention_dense(q.double().numpy(), K, V)
    assert_close(np64(out), want, FP8_TOL, FP8_REL, what="fp8 attention after mid-page appends")


def test_fp8_session_units_start_inside_pages():
    """A streaming session over an fp8 cache with 100-token units on 64-token
    pages: most units start inside a page, so the page they share with the
    previous unit is re-quantised.  Each unit's O and z against the oracle's
    performer unit over its own fp8 cache (fed the same appends), and every
    touched page bit for bit after the last unit."""
    H, D, ps, n_unit, n_units, S = 2, 128, 64, 100, 5, 4
    say("fp8 session, units inside pages")
    n_phys = 10
    free = torch.randperm(n_phys, generator=torch.Generator().manual_seed(17)).tolist()
    pt = torch.full((n_phys,), -1, dtype=torch.int32)
    g = bca.KVCache(H, D, ps, pt, n_phys, "fp8")
    ss = bca.Session(g, free)
    ref = oracle.PagedCacheFP8(H, D, ps, free, n_phys)
    w = workloads.randn((H * D, 16), 31)
    ws = bca.alloc_workspace(bca.workspace_bytes(g, n_unit, n_units * n_unit, 16))
    for u in range(n_units):
        k = workloads.qkv(120 + u, n_unit, H, D, 0.5 * (1 + u % 3), "bf16")
        v = workloads.qkv(220 + u, n_unit, H, D, 0.5, "bf16")
        q = workloads.qkv(320 + u, n_unit, H, D, 0.5, "bf16")
        eps = workloads.randn((n_unit, 16), 420 + u)
        z = eps.clone().cuda()
        osc = torch.empty((n_unit, H, D), dtype=torch.bfloat16, device="cuda")
        ss.unit(k.cuda(), v.cuda(), q.cuda(), w.cuda(), z, S, osc, workspace=ws, use_graph=u % 2 == 1)
        torch.cuda.synchronize()
        ref.append(k.float().numpy(), v.float().numpy())
        K, V = ref.gather()
        o_want = oracle.attention_dense(q.double().numpy(), K, V)
        vel = oracle.velocity(o_want, w.double().numpy())
        z_want = oracle.euler_solve(eps.double().numpy(), lambda zz, tau: vel, S)
        assert_close(np64(osc), o_want, FP8_TOL, FP8_REL, what=f"unit {u} O")
        assert_latents(np64(z), z_want, eps.double().numpy(), FP8_TOL, 1e-2, what=f"unit {u}")
    ss.close()
    _bits_equal(g, ref, n_units * n_unit, ps)


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("n_kv,n_q,ps", [(3000, 200, 256), (1000, 300, 64), (640, 640, 128)])
def test_fp8_attention(ws, n_kv, n_q, ps):
    """Streaming attention over an fp8 cache (bf16 queries); the last
    append ends mid-page."""
    H, D = 2, 128
    say(f"fp8 attention n_kv={n_kv} n_q={n_q} ps={ps} ws={ws}")
    q = workloads.qkv(51, n_q, H, D, 0.5, "bf16")
    k = workloads.qkv(52, n_kv, H, D, 0.5, "bf16")
    v = workloads.qkv(53, n_kv, H, D, 0.5, "bf16")
    g, o, _ = make_caches(bca, H, D, ps, "fp8", n_kv, 4)
    bca.kv_append(g, k.cuda(), v.cuda())
    o.append(k.float().numpy(), v.float().numpy())
    wsb = bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv)) if ws else None
    out = bca.block_causal_attn(q.cuda(), g, workspace=wsb)
    K, V = o.gather()
    want = oracle.attention_dense(q.double().numpy(), K, V)     # every cached key visible
    assert_close(np64(out), want, FP8_TOL, FP8_REL, what="fp8 attention")


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("n_kv,n_q", [(2000, 333), (4000, 700), (130, 64)])
def test_fp8_nan_codes_past_n_kv(ws, n_kv, n_q):
    """Codes past n_kv in the last page set to 0x7F (an E4M3 NaN) change no
    output bit: the tile that ends past n_kv has its tail zeroed before any
    PV step reads it (0 * NaN would be NaN)."""
    H, D, ps = 3, 128, 256
    say(f"fp8 NaN codes past n_kv={n_kv} n_q={n_q} ws={ws}")
    q = workloads.qkv(71, n_q, H, D, 0.5, "bf16").cuda()
    k = workloads.qkv(72, n_kv, H, D, 0.5, "bf16").cuda()
    v = workloads.qkv(73, n_kv, H, D, 0.5, "bf16").cuda()
    outs = []
    for poison in (False, True):
        g, _, pt = make_caches(bca, H, D, ps, "fp8", n_kv, 6)
        bca.kv_append(g, k, v)
        if poison:
            last = int(pt[(n_kv - 1) // ps])
            off = n_kv % ps
            assert off > 0
            g.k_pages[last, :, off:, :] = 0x7F
            g.v_pages[last, :, :, off:] = 0x7F
        wsb = bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv)) if ws else None
        outs.append(bca.block_causal_attn(q, g, workspace=wsb))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("n_kv,n_q,ps", [(3000, 200, 256), (1000, 300, 64)])
def test_fp8_attention_sharp_softmax(n_kv, n_q, ps):
    """Logits x4 (Q and K drawn at 2.0, logit std ~4) on the fast path, where
    S runs on the fp8 MFMA with Q as two E4M3 terms: a single E4M3 Q term
    would miss the relative-RMS bar several times over here."""
    H, D = 2, 128
    say(f"fp8 attention sharp n_kv={n_kv} n_q={n_q} ps={ps}")
    q = workloads.qkv(61, n_q, H, D, 2.0, "bf16")
    k = workloads.qkv(62, n_kv, H, D, 2.0, "bf16")
    v = workloads.qkv(63, n_kv, H, D, 0.5, "bf16")
    g, o, _ = make_caches(bca, H, D, ps, "fp8", n_kv, 4)
    bca.kv_append(g, k.cuda(), v.cuda())
    o.append(k.float().numpy(), v.float().numpy())
    out = bca.block_causal_attn(q.cuda(), g, workspace=bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv)))
    K, V = o.gather()
    want = oracle.attention_dense(q.double().numpy(), K, V)
    assert_close(np64(out), want, FP8_TOL, FP8_REL, what="fp8 attention, sharp softmax")


@pytest.mark.timeout(1500)
def test_fp8_c4_whole_unit():
    """The long-history fp8 workload as one whole performer unit: 750 units of
    history (2,784,000 tokens, 10,875 pages of 256) appended chunk by chunk,
    then performer_unit (append of the 3712-token slice, 4 x (attention
    over all 2,787,712 keys + Euler)), 40 heads x 128, in the bench's launch
    configuration.

    The oracle quantises the same seeded bf16 sources itself, with its C
    quantiser (oracle/fp8c.py, pinned to the numpy oracle and torch's
    float8 cast), into its own pages in logical order.  Checked: the codes
    and scales of every page (all heads, K and V) bit for bit; the unit's O
    and its latents z (and the move z - eps) on sampled rows over all 40
    heads, against the oracle's attention over its own dequantised cache,
    its velocity and its Euler solver."""
    w = workloads.WORKLOADS["v02_long_fp8"]
    H, D, ps, lq = w.n_heads, w.head_dim, w.page_size, w.unit_tokens
    CH = workloads.hist_chunk_tokens(w)
    n_chunks = workloads.n_hist_chunks(w)
    assert CH % ps == 0 and n_chunks * CH == w.n_hist and w.n_hist % ps == 0
    n_log = -(-w.n_kv // ps)
    pt = workloads.page_table(n_log, n_log + 1, 4321)
    g = bca.KVCache(H, D, ps, pt, n_log + 1, "fp8")
    ok = np.empty((n_log, H, ps, D), np.uint8)
    ov = np.empty((n_log, H, D, ps), np.uint8)
    oks = np.empty((n_log, H), np.float32)
    ovs = np.empty((n_log, H), np.float32)
    ppc = CH // ps
    say(f"C4: appending {n_chunks} chunks of {CH} tokens (GPU) and quantising them (oracle)")
    for c in range(n_chunks):
        kc = workloads.hist_chunk(w, "k_hist", c, "cuda")
        vc = workloads.hist_chunk(w, "v_hist", c, "cuda")
        bca.kv_append(g, kc, vc)
        p0 = c * ppc
        fp8c.quantize_pages(kc.view(torch.int16).cpu().numpy(), ps, False, ok[p0:p0 + ppc], oks[p0:p0 + ppc])
        fp8c.quantize_pages(vc.view(torch.int16).cpu().numpy(), ps, True, ov[p0:p0 + ppc], ovs[p0:p0 + ppc])
    seed = lambda slot: workloads.seed_for(w.index, slot)
    q = workloads.qkv(seed("q"), lq, H, D, w.qkv_scale, "bf16", "cuda")
    k_new = workloads.qkv(seed("k_new"), lq, H, D, w.qkv_scale, "bf16", "cuda")
    v_new = workloads.qkv(seed("v_new"), lq, H, D, w.qkv_scale, "bf16", "cuda")
    eps = workloads.randn((lq, w.n_ch), seed("eps"), 1.0, "cuda")
    W = workloads.randn((H * D, w.n_ch), seed("w"), 1.0, "cuda")
    p0 = w.n_hist // ps
    fp8c.quantize_pages(k_new.view(torch.int16).cpu().numpy(), ps, False, ok[p0:], oks[p0:])
    fp8c.quantize_pages(v_new.view(torch.int16).cpu().numpy(), ps, True, ov[p0:], ovs[p0:])

    say("C4: performer unit on the GPU")
    z = eps.clone()
    osc = torch.empty((lq, H, D), dtype=torch.bfloat16, device="cuda")
    ws = bca.alloc_workspace(bca.workspace_bytes(g, lq, w.n_kv, w.n_ch))
    bca.performer_unit(g, k_new, v_new, q, W, z, w.n_steps, o_scratch=osc, workspace=ws)
    torch.cuda.synchronize()
    assert g.n_tokens == w.n_kv

    say("C4: every page's codes and scales against the oracle's")
    pt_dev = pt.to("cuda", torch.long)
    for lp0 in range(0, n_log, 512):
        lp1 = min(n_log, lp0 + 512)
        idx = pt_dev[lp0:lp1]
        np.testing.assert_array_equal(g.k_pages.index_select(0, idx).cpu().numpy(), ok[lp0:lp1])
        np.testing.assert_array_equal(g.v_pages.index_select(0, idx).cpu().numpy(), ov[lp0:lp1])
        np.testing.assert_array_equal(g.k_scales.index_select(0, idx).cpu().numpy(), oks[lp0:lp1])
        np.testing.assert_array_equal(g.v_scales.index_select(0, idx).cpu().numpy(), ovs[lp0:lp1])

    say("C4: O and z on sampled rows, all 40 heads")
    rows = np.array([0, 1, 255, 256, 1855, 2047, 3000, 3583, 3584, 3711])
    qs = q[rows.tolist()].float().cpu().numpy().astype(np.float64)
    o_want = np.zeros((len(rows), H, D))
    for h in range(H):
        K = fp8c.decode_head(ok, oks, w.n_kv, h, False)
        V = fp8c.decode_head(ov, ovs, w.n_kv, h, True)
        o_want[:, h] = oracle.attention_dense(qs[:, h:h + 1], K[:, None], V[:, None])[:, 0]
        del K, V
    vel = oracle.velocity(o_want, W.double().cpu().numpy())
    e = eps[rows.tolist()].double().cpu().numpy()
    z_want = oracle.euler_solve(e, lambda zz, tau: vel, w.n_steps)
    assert_close(osc[rows.tolist()].float().cpu().numpy(), o_want, FP8_TOL, FP8_REL, what="C4 unit O")
    assert_latents(z[rows.tolist()].cpu().numpy(), z_want, e, FP8_TOL, 1e-2, what="C4 unit")
