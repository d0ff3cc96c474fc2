"""block_causal_attn parity against the oracle (fp32 path: max-abs 1e-4; bf16
path: max-abs 2e-2 and relative RMS 1e-2), plus bitwise invariants of the
GPU path (determinism, page-table shuffle, garbage past n_kv)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, make_caches, np64, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")

F32_TOL = 1e-4
BF16_TOL = 2e-2
BF16_REL = 1e-2


def _tiny_inputs():
    w = workloads.WORKLOADS["tiny_f32"]
    n = w.n_kv
    s = lambda slot: workloads.seed_for(w.index, slot)
    q = workloads.qkv(s("q"), n, w.n_heads, w.head_dim, 1.0, "f32")
    k = workloads.qkv(s("k_hist"), n, w.n_heads, w.head_dim, 1.0, "f32")
    v = workloads.qkv(s("v_hist"), n, w.n_heads, w.head_dim, 1.0, "f32")
    return w, q, k, v


@pytest.mark.parametrize("ps,shuffle", [(256, None), (16, None), (16, 7)])
def test_tiny_f32_full_sequence(ps, shuffle):
    """fp32, 4 heads x 64, block 16, 9 blocks: one multi-block call over the
    whole sequence against the dense-mask oracle."""
    w, q, k, v = _tiny_inputs()
    say(f"tiny f32 full ps={ps} shuffle={shuffle}")
    g, _, _ = make_caches(bca, w.n_heads, w.head_dim, ps, "f32", w.n_kv, shuffle)
    bca.kv_append(g, k.cuda(), v.cuda())
    out = bca.block_causal_attn(q.cuda(), g, n_kv=w.n_kv, q_pos0=0, block_size=w.unit_tokens)
    want = oracle.attention_dense(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  0, w.unit_tokens)
    assert_close(np64(out), want, F32_TOL, what="full-sequence f32")


@pytest.mark.parametrize("ps,shuffle", [(256, None), (16, 11)])
def test_tiny_f32_incremental(ps, shuffle):
    """Unit by unit: append a block, attend its queries over the cache."""
    w, q, k, v = _tiny_inputs()
    B = w.unit_tokens
    g, o, _ = make_caches(bca, w.n_heads, w.head_dim, ps, "f32", w.n_kv, shuffle)
    outs = []
    for u0 in range(0, w.n_kv, B):
        bca.kv_append(g, k[u0:u0 + B].cuda(), v[u0:u0 + B].cuda())
        outs.append(bca.block_causal_attn(q[u0:u0 + B].cuda(), g))
    got = np64(torch.cat(outs))
    want = oracle.attention_dense(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0, B)
    assert_close(got, want, F32_TOL, what="incremental f32")


def _ws(g, n_q, n_kv, on):
    """Workspace on: fast kernel (+ split, + exact rerun of flagged tiles);
    off: the exact-rescaling kernel alone."""
    return bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv)) if on else None


def _bf16_case(H, D, n_kv, ps, shuffle, seed, scale=1.0):
    q = workloads.qkv(seed, n_kv, H, D, scale, "bf16")
    k = workloads.qkv(seed + 1, n_kv, H, D, scale, "bf16")
    v = workloads.qkv(seed + 2, n_kv, H, D, 1.0, "bf16")
    g, _, pt = make_caches(bca, H, D, ps, "bf16", n_kv, shuffle)
    bca.kv_append(g, k.cuda(), v.cuda())
    return q, k, v, g, pt


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("ps,shuffle", [(256, None), (16, 4), (64, 9)])
@pytest.mark.parametrize("n_kv,n_q", [(1000, 300), (4160, 777), (300, 300), (70, 5)])
@pytest.mark.parametrize("ws", [False, True])
def test_bf16_streaming(D, ps, shuffle, n_kv, n_q, ws):
    """The streaming call (the binding's defaults: q_pos0 = n_kv - n_q,
    block_size = n_kv): the last n_q tokens form the current block and see
    every cached key, also where the history (700, 3383, 65) is not a
    multiple of n_q; ragged key and query tails."""
    H = 3
    say(f"bf16 streaming D={D} ps={ps} n_kv={n_kv} n_q={n_q} ws={ws}")
    q, k, v, g, _ = _bf16_case(H, D, n_kv, ps, shuffle, 31)
    qq = q[n_kv - n_q:]
    out = bca.block_causal_attn(qq.cuda(), g, workspace=_ws(g, n_q, n_kv, ws))
    want = oracle.attention_dense(qq.double().numpy(), k.double().numpy(), v.double().numpy())
    assert_close(np64(out), want, BF16_TOL, BF16_REL, what="streaming bf16")


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("n_kv,n_q,B", [(1000, 300, 300), (4160, 777, 777), (2000, 600, 256)])
def test_bf16_explicit_grid_cuts_the_queries(n_kv, n_q, B, ws):
    """An explicit block grid that does not line up with the queries: q_pos0
    = n_kv - n_q with block_size B puts the queries in two or more blocks
    of the fixed grid j // B, so their early rows must not see the later
    keys of the call.  The oracle's dense mask with the same grid decides."""
    H, D = 2, 128
    say(f"bf16 explicit grid n_kv={n_kv} n_q={n_q} B={B} ws={ws}")
    q, k, v, g, _ = _bf16_case(H, D, n_kv, 64, 5, 37)
    qq = q[n_kv - n_q:]
    out = bca.block_causal_attn(qq.cuda(), g, q_pos0=n_kv - n_q, block_size=B,
                                workspace=_ws(g, n_q, n_kv, ws))
    want = oracle.attention_dense(qq.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  n_kv - n_q, B)
    assert_close(np64(out), want, BF16_TOL, BF16_REL, what=f"grid B={B}")


@pytest.mark.parametrize("B", [1, 16, 100, 256, 1000])
@pytest.mark.parametrize("ps", [256, 16])
@pytest.mark.parametrize("ws", [False, True])
def test_bf16_multiblock(B, ps, ws):
    """Full-sequence prefill call with many blocks: masked diagonal tiles,
    skipped future tiles; block 1 is causal."""
    H, D, n = 2, 128, 900
    say(f"bf16 multiblock B={B} ps={ps} ws={ws}")
    q, k, v, g, _ = _bf16_case(H, D, n, ps, 3, 57)
    out = bca.block_causal_attn(q.cuda(), g, n_kv=n, q_pos0=0, block_size=B,
                                workspace=_ws(g, n, n, ws))
    want = oracle.attention_dense(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0, B)
    assert_close(np64(out), want, BF16_TOL, BF16_REL, what=f"multiblock B={B}")


@pytest.mark.parametrize("ws", [False, True])
def test_bf16_middle_unit_and_out_f32(ws):
    """Queries of a middle unit (q_pos0 > 0, later keys present but hidden)
    with fp32 output."""
    H, D, n = 2, 128, 1500
    q, k, v, g, _ = _bf16_case(H, D, n, 256, None, 77)
    q_pos0, n_q, B = 600, 300, 300
    qq = q[q_pos0:q_pos0 + n_q]
    out = bca.block_causal_attn(qq.cuda(), g, n_kv=n, q_pos0=q_pos0, block_size=B,
                                out_dtype=torch.float32, workspace=_ws(g, n_q, n, ws))
    assert out.dtype == torch.float32
    want = oracle.attention_dense(qq.double().numpy(), k[:900].double().numpy(),
                                  v[:900].double().numpy(), 600, B)
    assert_close(np64(out), want, BF16_TOL, BF16_REL, what="middle unit f32 out")


def test_split_kv_matches_single_pass():
    """With a workspace the key range is split and merged; both results
    match the oracle, and repeated split calls are bit-identical."""
    H, D, n_kv, n_q = 2, 128, 20000, 256
    q, k, v, g, _ = _bf16_case(H, D, n_kv, 256, 2, 91)
    qq = q[n_kv - n_q:].cuda()
    ws = bca.alloc_workspace(bca.workspace_bytes(g, n_q, n_kv))
    a = bca.block_causal_attn(qq, g)
    b = bca.block_causal_attn(qq, g, workspace=ws)
    c = bca.block_causal_attn(qq, g, workspace=ws)
    torch.cuda.synchronize()
    # the streaming call: every one of the n_kv keys visible (the history,
    # 19,744 tokens, is not a multiple of the 256 queries)
    want = oracle.attention_dense(q[n_kv - n_q:].double().numpy(), k.double().numpy(),
                                  v.double().numpy())
    assert_close(np64(a), want, BF16_TOL, BF16_REL, what="single pass")
    assert_close(np64(b), want, BF16_TOL, BF16_REL, what="split")
    assert torch.equal(b, c)


def _split_ws_bytes(n_q, H, D, s):
    """Workspace bytes that hold block_causal_attn's region for at most s
    key-range splits: 512 bytes per query for fm_euler_step first, then the
    overflow flags (one int32 per 256-row query tile, head, split and wave
    of 8), 256 bytes of queue counters and, for s > 1, the partials: O
    [s][n_q][H][D] in bf16 (normalised by each split's row sum) and (m, l)
    [s][n_q][H][2] in fp32, each part 256-aligned."""
    a = lambda x: -(-x // 256) * 256
    flags = a(-(-n_q // 256) * H * s * 8 * 4)
    parts = a(s * n_q * H * D * 2) + a(s * n_q * H * 2 * 4) if s > 1 else 0
    return a(512 * n_q) + flags + 256 + parts


def test_every_split_count():
    """A shape with 2 (query tile, head) pairs, where every extra split adds
    parallelism, so a workspace that fits the partials of at most s splits
    runs exactly s of them: s = 1 .. 8 (the merge kernel for every count)
    all match the oracle, are deterministic and differ from one another
    bitwise (each count rounds differently)."""
    H, D, n_kv, n_q = 2, 128, 6000, 256
    q, k, v, g, _ = _bf16_case(H, D, n_kv, 256, 2, 93)
    qq = q[n_kv - n_q:].cuda()
    want = oracle.attention_dense(q[n_kv - n_q:].double().numpy(), k.double().numpy(),
                                  v.double().numpy())
    outs = []
    for s in range(1, 9):
        ws = bca.alloc_workspace(_split_ws_bytes(n_q, H, D, s))
        a = bca.block_causal_attn(qq, g, workspace=ws)
        b = bca.block_causal_attn(qq, g, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert_close(np64(a), want, BF16_TOL, BF16_REL, what=f"{s} splits")
        outs.append(a)
    for i in range(8):
        for j in range(i):
            assert not torch.equal(outs[i], outs[j]), (i + 1, j + 1)


@pytest.mark.parametrize("ws", [False, True])
def test_bitwise_invariants(ws):
    """P5 shuffled page table, P7 garbage appended past n_kv, determinism."""
    H, D, n_kv, n_q = 3, 128, 2000, 333
    q = workloads.qkv(5, n_q, H, D, 1.0, "bf16").cuda()
    k = workloads.qkv(6, n_kv, H, D, 1.0, "bf16")
    v = workloads.qkv(7, n_kv, H, D, 1.0, "bf16")
    outs = []
    for shuffle in (None, 12):
        g, _, _ = make_caches(bca, H, D, 256, "bf16", n_kv + 500, shuffle)
        bca.kv_append(g, k.cuda(), v.cuda())
        w = _ws(g, n_q, n_kv, ws)
        outs.append(bca.block_causal_attn(q, g, n_kv=n_kv, workspace=w))
        outs.append(bca.block_causal_attn(q, g, n_kv=n_kv, workspace=w))
        junk = torch.full((500, H, D), float("nan"), dtype=torch.bfloat16)
        bca.kv_append(g, junk.cuda(), junk.cuda())
        outs.append(bca.block_causal_attn(q, g, n_kv=n_kv, workspace=w))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("ws", [False, True])
def test_peaky_planted_keys(ws):
    """Sharp softmax: logits x16 and keys planted equal to chosen queries at
    the first page, a page boundary and inside the current block; a wrong page
    or mask shows as an O(1) error.  With a workspace the planted keys far
    above the first tile's maximum send their query tiles through the
    overflow flag to the exact kernel."""
    H, D, n_kv, n_q = 2, 128, 3000, 200
    q = workloads.qkv(41, n_q, H, D, 1.0, "bf16")
    k = workloads.qkv(42, n_kv, H, D, 1.0, "bf16")
    v = workloads.qkv(43, n_kv, H, D, 1.0, "bf16")
    for qi, kj in [(0, 3), (1, 255), (2, 256), (3, 2899), (4, n_kv - 1), (5, 1000)]:
        k[kj] = q[qi]
    g, _, _ = make_caches(bca, H, D, 256, "bf16", n_kv, 8)
    bca.kv_append(g, k.cuda(), v.cuda())
    scale = 4.0 / np.sqrt(D)
    out = bca.block_causal_attn(q.cuda(), g, softmax_scale=scale, workspace=_ws(g, n_q, n_kv, ws))
    want = oracle.attention_dense(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  scale=scale)
    assert_close(np64(out), want, BF16_TOL, BF16_REL, what="peaky")
