"""The Python binding refuses tensors the kernels would misuse (host memory,
wrong element type, short or misshapen buffers, unmapped pages) with
ValueError before calling the library: nothing is launched and the cache's
n_tokens does not move.  A well-formed call right after each refusal still
works."""
import pytest
import torch

import workloads
from _helpers import say

pytestmark = pytest.mark.gpu
bca = pytest.importorskip("block_causal_attention_performer_amd")

H, D, PS, NQ = 2, 128, 64, 32


def _cache():
    pt = torch.tensor([1, 0, -1, -1], dtype=torch.int32)   # pages 2, 3 not mapped
    return bca.KVCache(H, D, PS, pt, 4, "bf16")


def _unit():
    k = workloads.qkv(1, NQ, H, D, 0.5, "bf16").cuda()
    v = workloads.qkv(2, NQ, H, D, 0.5, "bf16").cuda()
    q = workloads.qkv(3, NQ, H, D, 0.5, "bf16").cuda()
    w = workloads.randn((H * D, 16), 4).cuda()
    z = workloads.randn((NQ, 16), 5).cuda()
    o = torch.empty((NQ, H, D), dtype=torch.bfloat16, device="cuda")
    return k, v, q, w, z, o


def test_kv_append_rejects_bad_tensors():
    say("binding: kv_append checks")
    g = _cache()
    k, v, *_ = _unit()
    for kk, vv in ((k.cpu(), v), (k, v.float()), (k, v[:NQ - 1]), (k[:, :1].contiguous(), v),
                   (k.transpose(0, 1), v)):
        with pytest.raises(ValueError):
            bca.kv_append(g, kk, vv)
        assert g.n_tokens == 0
    bca.kv_append(g, k, v)
    assert g.n_tokens == NQ


def test_unmapped_pages_are_refused():
    say("binding: unmapped pages")
    g = _cache()
    k = workloads.qkv(6, 2 * PS + 1, H, D, 0.5, "bf16").cuda()
    with pytest.raises(ValueError, match="not mapped"):
        bca.kv_append(g, k, k)                 # reaches logical page 2
    assert g.n_tokens == 0
    bca.kv_append(g, k[:2 * PS], k[:2 * PS])
    assert g.n_tokens == 2 * PS


def test_attention_and_euler_reject_bad_tensors():
    say("binding: attention / Euler checks")
    g = _cache()
    k, v, q, w, z, o = _unit()
    bca.kv_append(g, k, v)
    with pytest.raises(ValueError):
        bca.block_causal_attn(q.cpu(), g)
    with pytest.raises(ValueError):
        bca.block_causal_attn(q.float(), g)
    with pytest.raises(ValueError):
        bca.block_causal_attn(q, g, out=o[:NQ - 1])
    with pytest.raises(ValueError):
        bca.block_causal_attn(q, g, workspace=torch.empty(1024, dtype=torch.uint8))
    with pytest.raises(ValueError):
        bca.fm_euler_step(z, o, w[:-1], 0.25)              # short W
    with pytest.raises(ValueError):
        bca.fm_euler_step(z.to(torch.bfloat16), o, w, 0.25)
    with pytest.raises(ValueError):
        bca.fm_euler_step(z, o[:NQ // 2], w, 0.25)         # x shorter than z's rows
    with pytest.raises(ValueError):
        bca.fm_euler_step(z, o.float(), None, 0.25)        # plain mode wants [n_tok, n_ch]
    out = bca.block_causal_attn(q, g)
    bca.fm_euler_step(z, out, w, 0.25)
    torch.cuda.synchronize()
    assert torch.isfinite(z).all()


def test_performer_unit_rejects_bad_tensors():
    say("binding: performer_unit checks")
    g = _cache()
    k, v, q, w, z, o = _unit()
    bad = [dict(z=z.to(torch.bfloat16)), dict(z=z[:NQ - 1]), dict(w=w.to(torch.bfloat16)),
           dict(w=w[:, :8].contiguous()), dict(o_scratch=o.float()), dict(q=q.cpu()),
           dict(k_new=k[: NQ - 1])]
    for b in bad:
        a = dict(k_new=k, v_new=v, q=q, w=w, z=z, o_scratch=o)
        a.update(b)
        with pytest.raises(ValueError):
            bca.performer_unit(g, a["k_new"], a["v_new"], a["q"], a["w"], a["z"], 4,
                               o_scratch=a["o_scratch"])
        assert g.n_tokens == 0
    bca.performer_unit(g, k, v, q, w, z, 4, o_scratch=o)
    torch.cuda.synchronize()
    assert g.n_tokens == NQ
