"""Python binding of libbca, the block-causal performer step for MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
libbca.so (built from csrc/ by ``python -m
block_causal_attention_performer_amd.build``).  torch provides device memory
and streams.  There is no fallback: if the library is missing or fails to
load, every entry point raises.

Entry points mirror the C ABI in include/bca.h:
    kv_append, block_causal_attn, fm_euler_step, performer_unit,
    workspace_bytes, status_string
plus KVCache, a holder of the paged cache's device tensors and its C
descriptor.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

F32, BF16, FP8_E4M3 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbca.so")


class BcaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


class BcaKvCacheC(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("max_logical_pages", ctypes.c_int32),
        ("n_phys_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbca.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_causal_attention_performer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    cp = ctypes.POINTER(BcaKvCacheC)
    L.kv_append.argtypes = [cp, vp, vp, i64, i32, vp]
    L.kv_append.restype = i32
    L.block_causal_attn.argtypes = [vp, i64, i64, i32, cp, i64, vp, i32, i32, f32, vp, sz, vp]
    L.block_causal_attn.restype = i32
    L.fm_euler_step.argtypes = [vp, vp, vp, i64, i32, i32, f32, i32, vp, sz, vp]
    L.fm_euler_step.restype = i32
    L.performer_unit.argtypes = [cp, vp, vp, vp, i64, vp, vp, i32, i32, vp, vp, sz, vp, vp]
    L.performer_unit.restype = i32
    L.bca_workspace_bytes.argtypes = [cp, i64, i64, i32]
    L.bca_workspace_bytes.restype = sz
    L.bca_status_string.argtypes = [i32]
    L.bca_status_string.restype = ctypes.c_char_p
    L.performer_unit_noalloc.argtypes = [cp, vp, vp, vp, i64, vp, vp, i32, i32, vp, vp]
    L.performer_unit_noalloc.restype = i32
    L.bca_session_create.argtypes = [cp, ctypes.POINTER(i32), i32, ctypes.POINTER(vp)]
    L.bca_session_create.restype = i32
    L.bca_session_unit.argtypes = [vp, vp, vp, vp, i64, vp, vp, i32, i32, vp, vp, sz, i32, vp]
    L.bca_session_unit.restype = i32
    L.bca_session_free_pages.argtypes = [vp]
    L.bca_session_free_pages.restype = i64
    L.bca_session_destroy.argtypes = [vp]
    L.bca_session_destroy.restype = None
    _lib = L
    return L


NOALLOC_SCRATCH_BYTES = 256 << 20       # BCA_NOALLOC_SCRATCH_BYTES

EXPORTS = ("kv_append", "block_causal_attn", "fm_euler_step", "performer_unit",
           "performer_unit_noalloc",
           "bca_workspace_bytes", "bca_status_string", "bca_session_create", "bca_session_unit",
           "bca_session_free_pages", "bca_session_destroy")


def status_string(status: int) -> str:
    return lib().bca_status_string(status).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libbca must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st: int, where: str) -> None:
    if st != 0:
        raise BcaError(st, where)


def _need(t: Optional[torch.Tensor], name: str, device: torch.device,
          dtypes: Sequence[torch.dtype], shape: Optional[Sequence[int]] = None,
          numel: Optional[int] = None) -> None:
    """Raise ValueError unless t is a contiguous tensor on `device` with one
    of `dtypes` and the given shape (or element count).  The kernels take
    raw pointers, so a host tensor, a short buffer or a wrong element type
    would be read or written out of bounds on the GPU."""
    if t is None:
        raise ValueError(f"{name}: a tensor is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, the cache is on {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _cuda_device(device) -> torch.device:
    d = torch.device(device)
    if d.type != "cuda":
        raise ValueError(f"libbca runs on a GPU: device {d} is not a CUDA (HIP) device")
    if d.index is None:
        d = torch.device("cuda", torch.cuda.current_device())
    return d


def check_page_table(page_table, n_phys_pages: int):
    """Host check of a page table: every entry is -1 (not mapped yet) or a
    physical page in [0, n_phys_pages), no physical page twice.  Returns the
    entries as a host list."""
    pt = [int(x) for x in torch.as_tensor(page_table).reshape(-1).tolist()]
    if not pt:
        raise ValueError("page_table is empty")
    seen = set()
    for lp, p in enumerate(pt):
        if p == -1:
            continue
        if not 0 <= p < n_phys_pages:
            raise ValueError(f"page_table[{lp}] = {p} is outside [0, {n_phys_pages})")
        if p in seen:
            raise ValueError(f"page_table maps physical page {p} twice")
        seen.add(p)
    return pt


class KVCache:
    """Paged full-history KV cache in device memory.

    K pages [n_phys][H][page_size][D], V pages [n_phys][H][D][page_size]
    (d-major), elements f32, bf16 or uint8 E4M3FN codes (+ fp32 scales
    [n_phys][H] for K and V).  Pages are zero-filled at allocation.  The page
    table's entries are checked on the host (-1 = not mapped yet, else a
    distinct physical page); a host copy of it follows the pages that
    sessions map, so every call can check that the logical pages it touches
    are mapped.
    """

    def __init__(self, n_heads: int, head_dim: int, page_size: int,
                 page_table: torch.Tensor, n_phys_pages: int, dtype: str,
                 device="cuda"):
        if dtype not in ("f32", "bf16", "fp8"):
            raise ValueError(f"cache dtype {dtype!r}: expected 'f32', 'bf16' or 'fp8'")
        if n_heads <= 0 or head_dim <= 0 or page_size <= 0 or n_phys_pages <= 0:
            raise ValueError("n_heads, head_dim, page_size and n_phys_pages must be positive")
        self.pt_host = check_page_table(page_table, n_phys_pages)
        self.device = _cuda_device(device)
        self.dtype_name = dtype
        code = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}[dtype]
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]
        self.page_table = torch.as_tensor(page_table).to(device=self.device, dtype=torch.int32).contiguous()
        self.k_pages = torch.zeros((n_phys_pages, n_heads, page_size, head_dim), dtype=tdt, device=self.device)
        self.v_pages = torch.zeros((n_phys_pages, n_heads, head_dim, page_size), dtype=tdt, device=self.device)
        self.k_scales = self.v_scales = None
        if dtype == "fp8":
            self.k_scales = torch.ones((n_phys_pages, n_heads), dtype=torch.float32, device=self.device)
            self.v_scales = torch.ones((n_phys_pages, n_heads), dtype=torch.float32, device=self.device)
        self.c = BcaKvCacheC(
            _ptr(self.k_pages).value, _ptr(self.v_pages).value,
            None if self.k_scales is None else self.k_scales.data_ptr(),
            None if self.v_scales is None else self.v_scales.data_ptr(),
            self.page_table.data_ptr(), self.page_table.numel(), n_phys_pages,
            page_size, n_heads, head_dim, code, 0)

    @property
    def n_tokens(self) -> int:
        return int(self.c.n_tokens)

    @property
    def n_heads(self) -> int:
        return int(self.c.n_heads)

    @property
    def head_dim(self) -> int:
        return int(self.c.head_dim)

    @property
    def page_size(self) -> int:
        return int(self.c.page_size)

    @property
    def compute_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype_name == "f32" else torch.bfloat16

    def require_mapped(self, n_tok: int, where: str) -> None:
        """Raise ValueError unless logical pages [0, ceil(n_tok / page_size))
        exist and are mapped (the kernels read the page table unchecked)."""
        need = -(-n_tok // self.page_size)
        if need > len(self.pt_host):
            return                       # past the table: the library returns ERANGE
        for lp in range(need):
            if self.pt_host[lp] < 0:
                raise ValueError(f"{where}: logical page {lp} is not mapped to a physical page")

    def _qkv(self, t, name: str, n: int) -> None:
        _need(t, name, self.device, (self.compute_dtype,), (n, self.n_heads, self.head_dim))


def workspace_bytes(cache: KVCache, n_q: int, n_kv: int, n_ch: int = 16) -> int:
    return int(lib().bca_workspace_bytes(ctypes.byref(cache.c), n_q, n_kv, n_ch))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Device workspace of at least nbytes (the kernels need no particular
    initial contents)."""
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _ws(workspace: Optional[torch.Tensor], device: torch.device):
    """(pointer, bytes) of an optional workspace on the cache's device."""
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError(f"workspace: must be a tensor on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def kv_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    if not isinstance(k_new, torch.Tensor) or k_new.dim() != 3:
        raise ValueError("k_new: expected a [n_new, n_heads, head_dim] tensor")
    n_new = k_new.shape[0]
    cache._qkv(k_new, "k_new", n_new)
    cache._qkv(v_new, "v_new", n_new)
    cache.require_mapped(cache.n_tokens + n_new, "kv_append")
    st = lib().kv_append(ctypes.byref(cache.c), _ptr(k_new), _ptr(v_new), n_new,
                         _DT[k_new.dtype], _stream(stream))
    _check(st, "kv_append")


def block_causal_attn(q: torch.Tensor, cache: KVCache, n_kv: Optional[int] = None,
                      q_pos0: Optional[int] = None, block_size: Optional[int] = None,
                      out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Defaults give the streaming call: all n_tokens keys, q_pos0 = n_kv - n_q
    and block_size = n_kv, so every query sees every key below n_kv (its own
    block included) whatever the history length."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q: expected a [n_q, n_heads, head_dim] tensor")
    n_q = q.shape[0]
    cache._qkv(q, "q", n_q)
    n_kv = cache.n_tokens if n_kv is None else int(n_kv)
    q_pos0 = n_kv - n_q if q_pos0 is None else int(q_pos0)
    block_size = n_kv if block_size is None else int(block_size)
    if not 0 < block_size < 2 ** 31:
        raise ValueError(f"block_size {block_size}: must be in [1, 2^31)")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out", cache.device, (torch.bfloat16, torch.float32), tuple(q.shape))
    cache.require_mapped(min(n_kv, cache.n_tokens), "block_causal_attn")
    wp, wb = _ws(workspace, cache.device)
    st = lib().block_causal_attn(
        _ptr(q), n_q, q_pos0, block_size, ctypes.byref(cache.c), n_kv, _ptr(out),
        _DT[q.dtype], _DT[out.dtype], softmax_scale, wp, wb, _stream(stream))
    _check(st, "block_causal_attn")
    return out


def fm_euler_step(z: torch.Tensor, x: torch.Tensor, w: Optional[torch.Tensor], dtau: float,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """z <- z - dtau * (x @ w)  (x flattened to [n_tok, k]);  w None: z <- z - dtau * x."""
    if not isinstance(z, torch.Tensor) or z.dim() != 2 or not z.is_cuda:
        raise ValueError("z: expected a [n_tok, n_ch] float32 tensor on a GPU")
    dev = z.device
    n_tok, n_ch = z.shape
    _need(z, "z", dev, (torch.float32,))
    if w is not None:
        if not isinstance(w, torch.Tensor) or w.dim() != 2:
            raise ValueError("w: expected a [k, n_ch] float32 tensor")
        k = w.shape[0]
        _need(w, "w", dev, (torch.float32,), (k, n_ch))
        _need(x, "x", dev, (torch.bfloat16, torch.float32), numel=n_tok * k)
    else:
        k = n_ch
        _need(x, "x", dev, (torch.float32,), numel=n_tok * n_ch)
    wp, wb = _ws(workspace, dev)
    st = lib().fm_euler_step(
        _ptr(z), _ptr(x), _ptr(w), n_tok, k, n_ch, dtau, _DT[x.dtype], wp, wb, _stream(stream))
    _check(st, "fm_euler_step")
    return z


def _check_unit(cache: KVCache, k_new, v_new, q, w, z, o_scratch) -> None:
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q: expected a [n_q, n_heads, head_dim] tensor")
    n_q = q.shape[0]
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (q, "q"), (o_scratch, "o_scratch")):
        cache._qkv(t, name, n_q)
    if not isinstance(z, torch.Tensor) or z.dim() != 2:
        raise ValueError("z: expected a [n_q, n_ch] float32 tensor")
    n_ch = z.shape[1]
    _need(z, "z", cache.device, (torch.float32,), (n_q, n_ch))
    _need(w, "w", cache.device, (torch.float32,), (cache.n_heads * cache.head_dim, n_ch))


def performer_unit(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                   w: torch.Tensor, z: torch.Tensor, n_steps: int,
                   o_scratch: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   attn_events: Optional[Sequence[int]] = None, stream=None) -> torch.Tensor:
    """Append the unit's K/V, then n_steps x (attention, Euler); z in/out."""
    if o_scratch is None and isinstance(q, torch.Tensor):
        o_scratch = torch.empty(q.shape, dtype=cache.compute_dtype, device=cache.device)
    _check_unit(cache, k_new, v_new, q, w, z, o_scratch)
    cache.require_mapped(cache.n_tokens + q.shape[0], "performer_unit")
    ev = None
    if attn_events is not None:
        if len(attn_events) != 3 * n_steps:
            raise ValueError("attn_events needs 3 events per solver step")
        ev = (ctypes.c_void_p * len(attn_events))(*attn_events)
    wp, wb = _ws(workspace, cache.device)
    st = lib().performer_unit(
        ctypes.byref(cache.c), _ptr(k_new), _ptr(v_new), _ptr(q), q.shape[0], _ptr(w), _ptr(z),
        z.shape[1], n_steps, _ptr(o_scratch), wp, wb, ev, _stream(stream))
    _check(st, "performer_unit")
    return z


def performer_unit_noalloc(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                           q: torch.Tensor, w: torch.Tensor, z: torch.Tensor, n_steps: int,
                           o_scratch: torch.Tensor, stream=None) -> torch.Tensor:
    """performer_unit through the entry point that allocates nothing: its
    scratch is the library's fixed per-GPU array (NOALLOC_SCRATCH_BYTES).
    Calls that overlap on one GPU race on that array."""
    _check_unit(cache, k_new, v_new, q, w, z, o_scratch)
    cache.require_mapped(cache.n_tokens + q.shape[0], "performer_unit_noalloc")
    st = lib().performer_unit_noalloc(
        ctypes.byref(cache.c), _ptr(k_new), _ptr(v_new), _ptr(q), q.shape[0], _ptr(w), _ptr(z),
        z.shape[1], n_steps, _ptr(o_scratch), _stream(stream))
    _check(st, "performer_unit_noalloc")
    return z


class Session:
    """Streaming session over one growing cache (bca_session_*): each unit()
    maps the logical pages the unit reaches onto the next free physical
    pages, then runs one performer unit, optionally as a replayed HIP graph.
    The cache's host copy of its page table follows the pages the session
    maps (the library hands them out in free-list order)."""

    def __init__(self, cache: KVCache, free_pages: Sequence[int]):
        self.cache = cache
        self._free = [int(p) for p in free_pages]
        self._next = 0
        cache.require_mapped(cache.n_tokens, "Session")
        in_use = {p for p in cache.pt_host if p >= 0}
        clash = in_use.intersection(self._free)
        if clash:
            raise ValueError(f"free_pages holds pages the page table already maps: {sorted(clash)[:4]}")
        arr = (ctypes.c_int32 * len(self._free))(*self._free)
        h = ctypes.c_void_p()
        _check(lib().bca_session_create(ctypes.byref(cache.c), arr, len(self._free), ctypes.byref(h)),
               "bca_session_create")
        self.h = h
        self._mapped = -(-cache.n_tokens // cache.page_size)

    def unit(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, w: torch.Tensor,
             z: torch.Tensor, n_steps: int, o_scratch: torch.Tensor,
             workspace: Optional[torch.Tensor] = None, use_graph: bool = False,
             stream=None) -> torch.Tensor:
        c = self.cache
        _check_unit(c, k_new, v_new, q, w, z, o_scratch)
        wp, wb = _ws(workspace, c.device)
        st = lib().bca_session_unit(
            self.h, _ptr(k_new), _ptr(v_new), _ptr(q), q.shape[0], _ptr(w), _ptr(z), z.shape[1],
            n_steps, _ptr(o_scratch), wp, wb, 1 if use_graph else 0, _stream(stream))
        _check(st, "bca_session_unit")
        mapped = -(-c.n_tokens // c.page_size)
        for lp in range(self._mapped, mapped):
            c.pt_host[lp] = self._free[self._next]
            self._next += 1
        self._mapped = max(self._mapped, mapped)
        return z

    @property
    def free_pages(self) -> int:
        return int(lib().bca_session_free_pages(self.h))

    def close(self) -> None:
        if self.h is not None and self.h.value:
            lib().bca_session_destroy(self.h)
        self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
