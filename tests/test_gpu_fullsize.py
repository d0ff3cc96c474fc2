"""Parity at the full v0.2 sizes, in the launch configuration bench.py times
(workspace given: split key range, fast kernel + exact rerun of flagged
tiles).  Inputs are the seeded device draws of workloads.make_unit_inputs;
the oracle evaluates sampled query rows (all heads) over the whole cache in
float64, head by head."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, assert_latents, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")

ROWS = np.array([0, 1, 31, 32, 255, 256, 1000, 1855, 2047, 3000, 3583, 3584, 3700, 3711])


def _setup(name, qk_factor=1.0, plant=None):
    w = workloads.WORKLOADS[name]
    inp = workloads.make_unit_inputs(w, device="cuda")
    if qk_factor != 1.0:
        for key in ("q", "k_hist", "k_new"):
            inp[key] = workloads.peaky(inp[key], qk_factor)
    if plant:
        k_all_idx = []
        for qi, kj in plant:
            if kj < w.n_hist:
                inp["k_hist"][kj] = inp["q"][qi]
            else:
                inp["k_new"][kj - w.n_hist] = inp["q"][qi]
            k_all_idx.append(kj)
    H, D, ps = w.n_heads, w.head_dim, w.page_size
    n_log = -(-w.n_kv // ps)
    pt = workloads.page_table(n_log, n_log + 1, 1234)
    g = bca.KVCache(H, D, ps, pt, n_log + 1, "bf16")
    bca.kv_append(g, inp["k_hist"], inp["v_hist"])
    ws = bca.alloc_workspace(bca.workspace_bytes(g, w.unit_tokens, w.n_kv, w.n_ch))
    return w, inp, g, ws


def _oracle_rows(w, inp, rows, scale=None):
    """attention of the sampled rows over all keys, per head, float64."""
    H, D = w.n_heads, w.head_dim
    out = np.zeros((len(rows), H, D))
    q = inp["q"][rows.tolist()].float().cpu().numpy().astype(np.float64)
    for h in range(H):
        k = torch.cat([inp["k_hist"][:, h], inp["k_new"][:, h]]).float().cpu().numpy().astype(np.float64)
        v = torch.cat([inp["v_hist"][:, h], inp["v_new"][:, h]]).float().cpu().numpy().astype(np.float64)
        qq = q[:, h:h + 1, :]
        out[:, h:h + 1, :] = oracle.attention_dense(qq, k[:, None, :], v[:, None, :], scale=scale)
    return out


def test_v02_attention_sampled_rows():
    """One streaming block_causal_attn call at the v0.2 unit (40 x 128, 3712
    queries over 122,496 keys in 256-token pages)."""
    say("v0.2 attention full size")
    w, inp, g, ws = _setup("v02_attn")
    bca.kv_append(g, inp["k_new"], inp["v_new"])
    out = bca.block_causal_attn(inp["q"], g, workspace=ws)
    again = bca.block_causal_attn(inp["q"], g, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    want = _oracle_rows(w, inp, ROWS)
    got = out[ROWS.tolist()].float().cpu().numpy()
    assert_close(got, want, 2e-2, 1e-2, what="v0.2 O sampled rows")


def test_v02_share8_attention_sampled_rows():
    """One GPU's share of the v0.2 call under head-sharded context
    parallelism over 8 GPUs (5 x 128 heads, the same 3712 queries over
    122,496 keys), as `bench.py --workload v02_share8 --attn-only` times it:
    few (query tile, head) pairs, so the split count comes from the
    scheduler model (7 splits on 256 CUs).  More sampled rows, all heads."""
    say("v0.2 one-GPU head share (5 heads)")
    w, inp, g, ws = _setup("v02_share8")
    bca.kv_append(g, inp["k_new"], inp["v_new"])
    out = bca.block_causal_attn(inp["q"], g, workspace=ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([ROWS, np.arange(0, 3712, 97), np.arange(3584, 3712, 13)]))
    want = _oracle_rows(w, inp, rows)
    got = out[rows.tolist()].float().cpu().numpy()
    assert_close(got, want, 2e-2, 1e-2, what="v0.2 share O sampled rows")


def test_v02_attention_peaky_planted():
    """Sharp-softmax v0.2 variant: Q and K x4 (logit std ~4) and keys equal
    to chosen queries planted in the first page, at a page boundary, deep in
    the history and inside the current block."""
    say("v0.2 attention peaky")
    plant = [(0, 5), (1, 255), (256, 256), (1000, 60000), (3583, 118784 + 100), (3711, 122495)]
    w, inp, g, ws = _setup("v02_attn", qk_factor=4.0, plant=plant)
    bca.kv_append(g, inp["k_new"], inp["v_new"])
    out = bca.block_causal_attn(inp["q"], g, workspace=ws)
    torch.cuda.synchronize()
    rows = np.array(sorted(set([r for r, _ in plant] + [2, 3000])))
    want = _oracle_rows(w, inp, rows)
    got = out[rows.tolist()].float().cpu().numpy()
    assert_close(got, want, 2e-2, 1e-2, what="v0.2 peaky O")


def test_v02_performer_unit_sampled_rows():
    """The full v0.2 performer unit (append + 4 x (attention + Euler) with the
    5120 x 16 projection), exactly as bench.py runs it."""
    say("v0.2 performer unit full size")
    w, inp, g, ws = _setup("v02_unit")
    z = inp["eps"].clone()
    osc = torch.empty((w.unit_tokens, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    bca.performer_unit(g, inp["k_new"], inp["v_new"], inp["q"], inp["w"], z, w.n_steps,
                       o_scratch=osc, workspace=ws)
    torch.cuda.synchronize()
    assert g.n_tokens == w.n_kv
    o_want = _oracle_rows(w, inp, ROWS)
    v = oracle.velocity(o_want, inp["w"].double().cpu().numpy())
    eps = inp["eps"][ROWS.tolist()].double().cpu().numpy()
    z_want = oracle.euler_solve(eps, lambda zz, tau: v, w.n_steps)
    assert_close(osc[ROWS.tolist()].float().cpu().numpy(), o_want, 2e-2, 1e-2, what="v0.2 unit O")
    assert_latents(z[ROWS.tolist()].cpu().numpy(), z_want, eps, 2e-2, 1e-2, what="v0.2 unit")


def test_v02_catchup_sampled_rows():
    """Multi-block catch-up call at v0.2 shapes, in the configuration
    `bench.py --workload v02_attn --catchup-units 8` times: the queries are
    the last 8 units of the 122,496-key cache (29,696 rows, q_pos0 = 92,800,
    blocks of 3712), so every query tile skips the key tiles of later blocks
    and masks only its own block's.  Sampled rows at block edges (all heads)
    against the oracle over each row's visible keys."""
    say("v0.2 catch-up, 8 units of queries")
    w, inp, g, _ = _setup("v02_attn")
    bca.kv_append(g, inp["k_new"], inp["v_new"])
    U, B = 8, w.unit_tokens
    q_pos0, n_q, _ = workloads.catchup_span(w, U)
    H, D = w.n_heads, w.head_dim
    q = workloads.qkv(workloads.seed_for(w.index, "q_catchup"), n_q, H, D, w.qkv_scale, "bf16", "cuda")
    ws = bca.alloc_workspace(bca.workspace_bytes(g, n_q, w.n_kv, w.n_ch))
    out = bca.block_causal_attn(q, g, n_kv=w.n_kv, q_pos0=q_pos0, block_size=B, workspace=ws)
    torch.cuda.synchronize()
    rows = [0, 1, B - 1, B, 3 * B + 100, 5 * B - 1, 7 * B, n_q - 1]
    k_all = torch.cat([inp["k_hist"], inp["k_new"]])
    v_all = torch.cat([inp["v_hist"], inp["v_new"]])
    qs = q[rows].float().cpu().numpy().astype(np.float64)
    want = np.zeros((len(rows), H, D))
    for h in range(H):
        k = k_all[:, h].float().cpu().numpy().astype(np.float64)[:, None]
        v = v_all[:, h].float().cpu().numpy().astype(np.float64)[:, None]
        for i, r in enumerate(rows):
            # the oracle's own block mask, for the row at global position q_pos0 + r
            want[i, h] = oracle.attention_dense(qs[i:i + 1, None, h], k, v, q_pos0 + r, B)[0, 0]
    got = out[rows].float().cpu().numpy()
    assert_close(got, want, 2e-2, 1e-2, what="v0.2 catch-up sampled rows")
