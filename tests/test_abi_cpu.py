"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host (before any launch)
with the documented status codes, leaving the cache's n_tokens untouched."""
import ctypes
import os
import re

import pytest
import torch

import block_causal_attention_performer_amd as bca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # never dereferenced: every case fails validation first


def _header_symbols():
    text = open(os.path.join(ROOT, "include", "bca.h")).read()
    return re.findall(r"BCA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_boundary():
    assert sorted(_header_symbols()) == sorted(bca.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = bca.lib()
    for name in _header_symbols():
        assert hasattr(L, name), name


def test_status_strings():
    assert bca.status_string(0) == "ok"
    assert "invalid" in bca.status_string(-1)
    assert "range" in bca.status_string(-2)


def _cache(**kw):
    c = bca.BcaKvCacheC()
    c.k_pages = FAKE
    c.v_pages = FAKE
    c.page_table = FAKE
    c.max_logical_pages = 4
    c.n_phys_pages = 4
    c.page_size = 256
    c.n_heads = 2
    c.head_dim = 128
    c.dtype = bca.BF16
    c.n_tokens = 0
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _append(c, n=10, src=bca.BF16, k=FAKE, v=FAKE):
    return bca.lib().kv_append(ctypes.byref(c), k, v, n, src, None)


@pytest.mark.parametrize("kw,n,src,want", [
    ({}, 2000, bca.BF16, -2),                        # 2000 > 4 pages * 256
    ({"n_tokens": 1000}, 25, bca.BF16, -2),
    ({}, -1, bca.BF16, -1),
    ({}, 10, bca.F32, -3),                           # bf16 cache, f32 source
    ({"head_dim": 96}, 10, bca.BF16, -3),
    ({"page_size": 100}, 10, bca.BF16, -3),
    ({"page_size": 8}, 10, bca.BF16, -3),
    ({"k_pages": None}, 10, bca.BF16, -1),
    ({"n_heads": 0}, 10, bca.BF16, -1),
    ({"dtype": 7}, 10, bca.BF16, -3),
    ({"dtype": bca.FP8_E4M3}, 10, bca.BF16, -1),    # fp8 without scales
    ({"dtype": bca.FP8_E4M3, "k_scales": FAKE, "v_scales": FAKE, "head_dim": 64}, 10,
     bca.BF16, -3),                                  # fp8 pages only for head dim 128
    ({"dtype": bca.FP8_E4M3, "k_scales": FAKE, "v_scales": FAKE, "page_size": 16}, 10,
     bca.BF16, -3),
])
def test_kv_append_rejects(kw, n, src, want):
    c = _cache(**kw)
    before = c.n_tokens
    assert _append(c, n, src) == want
    assert c.n_tokens == before


def test_kv_append_null_slice():
    c = _cache()
    assert _append(c, 5, k=None) == -1
    assert c.n_tokens == 0


def _attn(c, n_q=16, q_pos0=0, B=16, n_kv=16, qd=bca.BF16, od=bca.BF16, scale=0.0, q=FAKE,
          out=FAKE):
    return bca.lib().block_causal_attn(q, n_q, q_pos0, B, ctypes.byref(c), n_kv, out, qd, od,
                                       scale, None, 0, None)


@pytest.mark.parametrize("kw,args,want", [
    ({"n_tokens": 100}, dict(n_kv=101, n_q=1, q_pos0=100), -2),   # n_kv > n_tokens
    ({"n_tokens": 100}, dict(n_q=0), -1),
    ({"n_tokens": 100}, dict(B=0), -1),
    ({"n_tokens": 100}, dict(q_pos0=-1), -1),
    ({"n_tokens": 100}, dict(n_q=20, q_pos0=90, n_kv=100), -1),  # queries past n_kv
    ({"n_tokens": 100}, dict(qd=bca.F32), -3),
    ({"n_tokens": 100, "dtype": bca.F32, "head_dim": 64}, dict(qd=bca.F32, od=bca.BF16), -3),
    ({"n_tokens": 100}, dict(q=None), -1),
    ({"n_tokens": 100}, dict(out=None), -1),
    ({"n_tokens": 100}, dict(scale=float("nan")), -1),
    ({"n_tokens": 2000}, dict(), -2),                              # cache n_tokens past pages
])
def test_attn_rejects(kw, args, want):
    assert _attn(_cache(**kw), **args) == want


@pytest.mark.parametrize("args,want", [
    (dict(z=None), -1),
    (dict(x=None), -1),
    (dict(n_ch=0), -1),
    (dict(n_ch=65), -3),
    (dict(k=0), -1),
    (dict(dtype=bca.FP8_E4M3), -3),
    (dict(w=None, dtype=bca.BF16), -3),      # plain mode takes fp32 velocities
    (dict(dtau=float("inf")), -1),
])
def test_euler_rejects(args, want):
    """Bad arguments; z or x NULL is refused only when there are tokens."""
    a = dict(z=FAKE, x=FAKE, w=FAKE, n_tok=10, k=64, n_ch=16, dtau=0.25, dtype=bca.BF16)
    a.update(args)
    st = bca.lib().fm_euler_step(a["z"], a["x"], a["w"], a["n_tok"], a["k"], a["n_ch"],
                                 a["dtau"], a["dtype"], None, 0, None)
    assert st == want


def test_euler_zero_tokens_is_a_no_op():
    L = bca.lib()
    assert L.fm_euler_step(None, None, None, 0, 64, 16, 0.25, bca.F32, None, 0, None) == 0
    assert L.fm_euler_step(None, FAKE, FAKE, 1, 64, 16, 0.25, bca.BF16, None, 0, None) == -1


def test_performer_unit_validates_everything_first():
    L = bca.lib()
    # the append would fit but the Euler phase is invalid (n_ch 0): nothing
    # may be enqueued and n_tokens must not move
    c = _cache()
    st = L.performer_unit(ctypes.byref(c), FAKE, FAKE, FAKE, 16, FAKE, FAKE, 0, 4, FAKE, None, 0,
                          None, None)
    assert st == -1 and c.n_tokens == 0
    st = L.performer_unit(ctypes.byref(c), FAKE, FAKE, FAKE, 2000, FAKE, FAKE, 16, 4, FAKE,
                          None, 0, None, None)
    assert st == -2 and c.n_tokens == 0
    st = L.performer_unit(ctypes.byref(c), FAKE, FAKE, FAKE, 16, FAKE, FAKE, 16, 0, FAKE, None,
                          0, None, None)
    assert st == -1 and c.n_tokens == 0


def test_workspace_bytes_host_only():
    c = _cache()
    n = bca.lib().bca_workspace_bytes(ctypes.byref(c), 3712, 122496, 16)
    assert n > 3712 * 2 * 128 * 4
    assert bca.lib().bca_workspace_bytes(None, 1, 1, 16) == 0


def test_session_create_rejects():
    L = bca.lib()
    c = _cache()
    h = ctypes.c_void_p()
    for pages, n in (([0, 1, 1], 3), ([0, 4], 2), ([-1], 1)):   # duplicate, out of range, negative
        arr = (ctypes.c_int32 * len(pages))(*pages)
        assert L.bca_session_create(ctypes.byref(c), arr, n, ctypes.byref(h)) == -1
        assert not h.value
    assert L.bca_session_create(ctypes.byref(c), None, -1, ctypes.byref(h)) == -1
    assert L.bca_session_create(None, None, 0, ctypes.byref(h)) == -1
    assert L.bca_session_create(ctypes.byref(c), None, 0, None) == -1
    assert L.bca_session_free_pages(None) == -1
    L.bca_session_destroy(None)


def test_session_unit_validates_before_mapping():
    """A unit that the free pages cannot cover returns ERANGE, and a unit with
    a bad argument EINVAL, before any page is taken or any launch: the
    session's free-page count and the cache's n_tokens do not move."""
    L = bca.lib()
    c = _cache(max_logical_pages=8, n_phys_pages=8, n_tokens=100)   # logical page 0 mapped
    arr = (ctypes.c_int32 * 2)(5, 6)
    h = ctypes.c_void_p()
    assert L.bca_session_create(ctypes.byref(c), arr, 2, ctypes.byref(h)) == 0 and h.value
    try:
        assert L.bca_session_free_pages(h) == 2
        # 100 + 700 tokens reach logical page 3: three new pages, two free
        st = L.bca_session_unit(h, FAKE, FAKE, FAKE, 700, FAKE, FAKE, 16, 4, FAKE, None, 0, 0, None)
        assert st == -2 and c.n_tokens == 100 and L.bca_session_free_pages(h) == 2
        st = L.bca_session_unit(h, FAKE, FAKE, FAKE, 200, FAKE, FAKE, 0, 4, FAKE, None, 0, 0, None)
        assert st == -1 and c.n_tokens == 100 and L.bca_session_free_pages(h) == 2
        assert L.bca_session_unit(None, FAKE, FAKE, FAKE, 200, FAKE, FAKE, 16, 4, FAKE, None, 0, 0,
                                  None) == -1
    finally:
        L.bca_session_destroy(h)


# ------------------------------------------------- binding argument checks


def test_binding_rejects_host_cache():
    """The kernels take raw device pointers: a cache on the host is refused
    before anything is allocated or launched."""
    pt = torch.arange(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="not a CUDA"):
        bca.KVCache(2, 128, 256, pt, 4, "bf16", device="cpu")


@pytest.mark.parametrize("pt,n_phys,msg", [
    ([0, 1, 1], 4, "twice"),
    ([0, 4], 4, "outside"),
    ([-2, 0], 4, "outside"),
    ([], 4, "empty"),
])
def test_binding_checks_page_table(pt, n_phys, msg):
    with pytest.raises(ValueError, match=msg):
        bca.check_page_table(torch.tensor(pt, dtype=torch.int32), n_phys)


def test_binding_page_table_allows_unmapped():
    assert bca.check_page_table(torch.tensor([3, -1, 0, -1]), 4) == [3, -1, 0, -1]


def test_binding_tensor_checks():
    dev = torch.device("cpu")
    t = torch.zeros((4, 2, 8), dtype=torch.bfloat16)
    bca._need(t, "t", dev, (torch.bfloat16,), (4, 2, 8))
    with pytest.raises(ValueError, match="dtype"):
        bca._need(t.float(), "t", dev, (torch.bfloat16,), (4, 2, 8))
    with pytest.raises(ValueError, match="shape"):
        bca._need(t[:3], "t", dev, (torch.bfloat16,), (4, 2, 8))
    with pytest.raises(ValueError, match="contiguous"):
        bca._need(t.transpose(0, 1), "t", dev, (torch.bfloat16,))
    with pytest.raises(ValueError, match="elements"):
        bca._need(t, "t", dev, (torch.bfloat16,), numel=63)
    with pytest.raises(ValueError, match="on meta"):
        bca._need(torch.empty(4, device="meta"), "t", dev, (torch.float32,))
    with pytest.raises(ValueError, match="required"):
        bca._need(None, "t", dev, (torch.float32,))


def test_performer_unit_noalloc_validates_on_the_host():
    """The entry point that allocates nothing checks every argument, and that
    the unit's least scratch need fits its fixed array, before any HIP call:
    EINVAL for a bad argument, ERANGE for a unit of 600,000 queries (512
    bytes each of velocity partials alone pass 256 MiB)."""
    L = bca.lib()
    c = _cache()
    assert L.performer_unit_noalloc(ctypes.byref(c), FAKE, FAKE, FAKE, 16, FAKE, FAKE, 0, 4, FAKE,
                                    None) == -1
    assert L.performer_unit_noalloc(ctypes.byref(c), FAKE, FAKE, FAKE, 16, FAKE, FAKE, 16, 4, None,
                                    None) == -1
    big = _cache(max_logical_pages=4096, n_phys_pages=4096)
    assert L.performer_unit_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, 600000, FAKE, FAKE, 16, 4,
                                    FAKE, None) == -2
    assert c.n_tokens == 0 and big.n_tokens == 0
    assert bca.NOALLOC_SCRATCH_BYTES == 256 << 20
