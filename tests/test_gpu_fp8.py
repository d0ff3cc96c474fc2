"""fp8 (E4M3FN) KV cache parity: the quantiser bit for bit (codes and
scales) against the oracle's, and attention over the fp8 cache against the
oracle's attention on the K/V that the oracle itself quantised and
dequantised (max-abs 3e-2, relative RMS 1e-2)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, make_caches, np64, say

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


def test_fp8_append_rejects_unaligned_start():
    """An fp8 append must start on a page boundary (no requantisation of a
    partly filled page): the call fails and the cache is unchanged."""
    H, D, ps = 2, 128, 64
    g, _, _ = make_caches(bca, H, D, ps, "fp8", 4 * ps)
    k = workloads.qkv(1, 10, H, D, 0.5, "bf16").cuda()
    bca.kv_append(g, k, k)
    with pytest.raises(bca.BcaError):
        bca.kv_append(g, k, k)
    assert g.n_tokens == 10


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


def test_fp8_c4_full_size():
    """The long-history fp8 workload: 750 units of history (2,784,000 tokens,
    10,875 pages) appended chunk by chunk plus the 3712-token unit, 40 heads
    x 128 (28.5 GB of codes).  Codes and scales bit-exact on sampled pages
    (all heads) against the oracle's quantiser on the regenerated sources;
    one streaming attention call in the bench configuration checked on
    sampled rows of one head against the oracle over the K/V it quantised
    itself."""
    w = workloads.WORKLOADS["v02_long_fp8"]
    H, D, ps, lq = w.n_heads, w.head_dim, w.page_size, w.unit_tokens
    CH = workloads.hist_chunk_tokens(w)
    n_chunks = workloads.n_hist_chunks(w)
    assert CH % ps == 0 and n_chunks * CH == w.n_hist
    n_log = -(-w.n_kv // ps)
    pt = workloads.page_table(n_log, n_log + 1, 4321)
    g = bca.KVCache(H, D, ps, pt, n_log + 1, "fp8")
    say(f"C4: appending {n_chunks} chunks of {CH} tokens")
    for c in range(n_chunks):
        bca.kv_append(g, workloads.hist_chunk(w, "k_hist", c, "cuda"),
                      workloads.hist_chunk(w, "v_hist", c, "cuda"))
    inp = {s: workloads.qkv(workloads.seed_for(w.index, s), lq, H, D, w.qkv_scale, "bf16", "cuda")
           for s in ("q", "k_new", "v_new")}
    bca.kv_append(g, inp["k_new"], inp["v_new"])
    assert g.n_tokens == w.n_kv
    ws = bca.alloc_workspace(bca.workspace_bytes(g, lq, w.n_kv))
    out = bca.block_causal_attn(inp["q"], g, workspace=ws)
    torch.cuda.synchronize()

    # codes: first page, a middle page, the last history page, the unit's
    # first page and its last (half-filled) page
    pt_np = pt.numpy()
    kg_all, vg_all = g.k_pages, g.v_pages
    for lp in (0, 1, 5437, n_chunks * CH // ps - 1, w.n_hist // ps, n_log - 1):
        t0 = lp * ps
        if t0 < w.n_hist:
            c = t0 // CH
            r = t0 - c * CH
            # regenerated on the device: the device and host generators differ
            ks = workloads.hist_chunk(w, "k_hist", c, "cuda")[r:r + ps].cpu()
            vs = workloads.hist_chunk(w, "v_hist", c, "cuda")[r:r + ps].cpu()
        else:
            r = t0 - w.n_hist
            ks = inp["k_new"][r:r + ps].cpu()
            vs = inp["v_new"][r:r + ps].cpu()
        one = oracle.PagedCacheFP8(H, D, ps, [0], 1)
        one.append(ks.float().numpy(), vs.float().numpy())
        page = int(pt_np[lp])
        np.testing.assert_array_equal(kg_all[page].cpu().numpy(), one.k_codes[0])
        np.testing.assert_array_equal(vg_all[page].cpu().numpy(), one.v_codes[0])
        np.testing.assert_array_equal(g.k_scales[page].cpu().numpy(), one.k_scales[0])
        np.testing.assert_array_equal(g.v_scales[page].cpu().numpy(), one.v_scales[0])
    say("C4: sampled pages bit-exact")

    # attention: head 17, sampled rows, oracle quantising every page of that head
    h = 17
    rows = np.array([0, 1, 1000, 1855, 3000, 3711])
    o1 = oracle.PagedCacheFP8(1, D, ps, np.arange(n_log), n_log)
    for c in range(n_chunks):
        kc = workloads.hist_chunk(w, "k_hist", c, "cuda")[:, h:h + 1].float().cpu().numpy()
        vc = workloads.hist_chunk(w, "v_hist", c, "cuda")[:, h:h + 1].float().cpu().numpy()
        o1.append(kc, vc)
    o1.append(inp["k_new"][:, h:h + 1].float().cpu().numpy(),
              inp["v_new"][:, h:h + 1].float().cpu().numpy())
    K, V = o1.gather()
    qh = inp["q"][:, h:h + 1].float().cpu().numpy().astype(np.float64)
    want = oracle.attention_dense(qh, K, V, w.n_hist, lq, rows=rows)
    got = out[rows.tolist(), h:h + 1].float().cpu().numpy()
    assert_close(got, want, FP8_TOL, FP8_REL, what="C4 attention sampled rows")
