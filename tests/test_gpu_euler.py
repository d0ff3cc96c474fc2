"""fm_euler_step parity: closed-form interpolant with the exact velocity, and
the fused velocity projection against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, np64, say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")


def test_exact_velocity_reproduces_interpolant():
    """tiny fp32 workload: z(1) = eps, v = eps - z0, 4 uniform steps; every
    iterate is (1 - tau) z0 + tau eps and the last is z0."""
    w = workloads.WORKLOADS["tiny_f32"]
    eps = workloads.randn((w.unit_tokens, w.n_ch), workloads.seed_for(w.index, "eps"))
    z0 = workloads.randn((w.unit_tokens, w.n_ch), workloads.seed_for(w.index, "z0"))
    vel = (eps - z0).cuda()
    z = eps.clone().cuda()
    S = w.n_steps
    want = oracle.euler_solve(eps.double().numpy(), lambda zz, t: (eps - z0).double().numpy(), S,
                              record=True)[1]
    for s in range(S):
        bca.fm_euler_step(z, vel, None, 1.0 / S)
        tau = 1.0 - (s + 1) / S
        closed = (1 - tau) * z0.double().numpy() + tau * eps.double().numpy()
        assert_close(np64(z), closed, 1e-4, what=f"step {s} closed form")
        assert_close(np64(z), want[s + 1], 1e-4, what=f"step {s} oracle")
    assert_close(np64(z), z0.double().numpy(), 1e-4, what="z(0) == z0")


@pytest.mark.parametrize("n_tok,H,D", [(3712, 40, 128), (1024, 24, 128), (77, 4, 64), (5, 1, 64),
                                        (1000, 40, 128), (17, 8, 64), (33, 12, 128), (5, 64, 128),
                                        (40, 16, 64)])
@pytest.mark.parametrize("with_ws", [True, False])
def test_bf16_projection(n_tok, H, D, with_ws):
    k = H * D
    say(f"euler bf16 n_tok={n_tok} k={k} ws={with_ws}")
    x = workloads.qkv(3, n_tok, H, D, 0.05, "bf16")
    w = workloads.randn((k, 16), 4)
    z = workloads.randn((n_tok, 16), 5)
    zg = z.clone().cuda()
    ws = None
    if with_ws:
        c = bca.KVCache(H, D, 256, torch.zeros(1, dtype=torch.int32), 1, "bf16")
        ws = bca.alloc_workspace(bca.workspace_bytes(c, n_tok, n_tok))
    for _ in range(2):      # twice: the split counters must come back to zero
        bca.fm_euler_step(zg, x.cuda(), w.cuda(), 0.25, workspace=ws)
    v = oracle.velocity(x.double().numpy(), w.double().numpy())
    want = z.double().numpy() - 0.25 * v - 0.25 * v
    # the projection is exact up to fp32 accumulation and W's 2^-16 split
    assert_close(np64(zg), want, 1e-4, what="bf16 projection")


def test_f32_projection_generic():
    n_tok, k = 16, 256
    x = workloads.randn((n_tok, k), 7, 0.1)
    w = workloads.randn((k, 16), 8)
    z = workloads.randn((n_tok, 16), 9)
    zg = z.clone().cuda()
    bca.fm_euler_step(zg, x.cuda(), w.cuda(), 0.25)
    want = z.double().numpy() - 0.25 * oracle.velocity(x.double().numpy(), w.double().numpy())
    assert_close(np64(zg), want, 1e-5, what="f32 projection")


def test_projection_workspace_contents_do_not_matter():
    """The projection's k-part sums are written whole before they are read,
    so any initial workspace contents work: a workspace of random bytes, of
    all-ones bytes and a reused one give the same z bit for bit, call after
    call (ragged last row block: 1000 tokens)."""
    n_tok, H, D = 1000, 40, 128
    x = workloads.qkv(13, n_tok, H, D, 0.05, "bf16").reshape(n_tok, H * D).cuda()
    w = workloads.randn((H * D, 16), 14).cuda()
    z0 = workloads.randn((n_tok, 16), 15).cuda()
    nbytes = -(-n_tok * 512 // 256) * 256
    g = torch.Generator(device="cuda").manual_seed(16)
    junk = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    ones = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    ref = None
    for ws in (junk, ones, junk, junk):
        z = z0.clone()
        bca.fm_euler_step(z, x, w, 0.25, workspace=ws)
        bca.fm_euler_step(z, x, w, 0.25, workspace=ws)
        torch.cuda.synchronize()
        if ref is None:
            ref = z.clone()
            want = z0.double().cpu().numpy() - 0.5 * oracle.velocity(
                x.double().cpu().numpy().reshape(n_tok, H, D), w.double().cpu().numpy())
            assert_close(np64(z), want, 2e-2, what="two steps from a junk workspace")
        assert torch.equal(z, ref)


@pytest.mark.parametrize("n_tok,k", [(3712, 5120), (1000, 3072), (9, 512)])
def test_projection_is_deterministic(n_tok, k):
    """The projection (k split in eighths, partials added in a fixed order)
    gives the same bits call after call, with or without a workspace (the
    matrix-core path or the fp32 vector path); ragged last row blocks (1000
    and 9 tokens) included."""
    x = workloads.randn((n_tok, k), 21, 0.05).to(torch.bfloat16).cuda()
    w = workloads.randn((k, 16), 22).cuda()
    z0 = workloads.randn((n_tok, 16), 23).cuda()
    c = bca.KVCache(1, 128, 256, torch.zeros(1, dtype=torch.int32), 1, "bf16")
    ws = bca.alloc_workspace(bca.workspace_bytes(c, n_tok, n_tok))
    outs = []
    for _ in range(3):
        z = z0.clone()
        bca.fm_euler_step(z, x, w, 0.25, workspace=ws)
        outs.append(z)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    want = z0.double().cpu().numpy() - 0.25 * oracle.velocity(x.double().cpu().numpy(),
                                                              w.double().cpu().numpy())
    assert_close(np64(outs[0]), want, 1e-4, what="projection")
