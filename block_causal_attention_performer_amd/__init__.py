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


EXPORTS = ("kv_append", "block_causal_attn", "fm_euler_step", "performer_unit",
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


class KVCache:
    """Paged full-history KV cache in device memory.

    K pages [n_phys][H][page_size][D], V pages [n_phys][H][D][page_size]
    (d-major), elements f32, bf16 or uint8 E4M3FN codes (+ fp32 scales
    [n_phys][H] for K and V).  Pages are zero-filled at allocation.
    """

    def __init__(self, n_heads: int, head_dim: int, page_size: int,
                 page_table: torch.Tensor, n_phys_pages: int, dtype: str,
                 device="cuda"):
        self.dtype_name = dtype
        code = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}[dtype]
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]
        self.page_table = page_table.to(device=device, dtype=torch.int32).contiguous()
        self.k_pages = torch.zeros((n_phys_pages, n_heads, page_size, head_dim), dtype=tdt, device=device)
        self.v_pages = torch.zeros((n_phys_pages, n_heads, head_dim, page_size), dtype=tdt, device=device)
        self.k_scales = self.v_scales = None
        if dtype == "fp8":
            self.k_scales = torch.ones((n_phys_pages, n_heads), dtype=torch.float32, device=device)
            self.v_scales = torch.ones((n_phys_pages, n_heads), dtype=torch.float32, device=device)
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
    def compute_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype_name == "f32" else torch.bfloat16


def workspace_bytes(cache: KVCache, n_q: int, n_kv: int, n_ch: int = 16) -> int:
    return int(lib().bca_workspace_bytes(ctypes.byref(cache.c), n_q, n_kv, n_ch))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Device workspace of at least nbytes (the kernels need no particular
    initial contents)."""
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def kv_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    st = lib().kv_append(ctypes.byref(cache.c), _ptr(k_new), _ptr(v_new), k_new.shape[0],
                         _DT[k_new.dtype], _stream(stream))
    _check(st, "kv_append")


def block_causal_attn(q: torch.Tensor, cache: KVCache, n_kv: Optional[int] = None,
                      q_pos0: Optional[int] = None, block_size: Optional[int] = None,
                      out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Defaults give the streaming call: all n_tokens keys, q_pos0 = n_kv - n_q,
    block_size = n_q."""
    n_q = q.shape[0]
    n_kv = cache.n_tokens if n_kv is None else n_kv
    q_pos0 = n_kv - n_q if q_pos0 is None else q_pos0
    block_size = n_q if block_size is None else block_size
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    st = lib().block_causal_attn(
        _ptr(q), n_q, q_pos0, block_size, ctypes.byref(cache.c), n_kv, _ptr(out),
        _DT[q.dtype], _DT[out.dtype], softmax_scale, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "block_causal_attn")
    return out


def fm_euler_step(z: torch.Tensor, x: torch.Tensor, w: Optional[torch.Tensor], dtau: float,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """z <- z - dtau * (x @ w)  (x flattened to [n_tok, k]);  w None: z <- z - dtau * x."""
    n_tok, n_ch = z.shape
    k = x.numel() // n_tok if w is not None else n_ch
    st = lib().fm_euler_step(
        _ptr(z), _ptr(x), _ptr(w), n_tok, k, n_ch, dtau, _DT[x.dtype], _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "fm_euler_step")
    return z


def performer_unit(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                   w: torch.Tensor, z: torch.Tensor, n_steps: int,
                   o_scratch: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   attn_events: Optional[Sequence[int]] = None, stream=None) -> torch.Tensor:
    """Append the unit's K/V, then n_steps x (attention, Euler); z in/out."""
    if o_scratch is None:
        o_scratch = torch.empty(q.shape, dtype=cache.compute_dtype, device=q.device)
    ev = None
    if attn_events is not None:
        if len(attn_events) != 3 * n_steps:
            raise ValueError("attn_events needs 3 events per solver step")
        ev = (ctypes.c_void_p * len(attn_events))(*attn_events)
    st = lib().performer_unit(
        ctypes.byref(cache.c), _ptr(k_new), _ptr(v_new), _ptr(q), q.shape[0], _ptr(w), _ptr(z),
        z.shape[1], n_steps, _ptr(o_scratch), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        ev, _stream(stream))
    _check(st, "performer_unit")
    return z


class Session:
    """Streaming session over one growing cache (bca_session_*): each unit()
    maps the logical pages the unit reaches onto the next free physical
    pages, then runs one performer unit, optionally as a replayed HIP graph."""

    def __init__(self, cache: KVCache, free_pages: Sequence[int]):
        self.cache = cache
        arr = (ctypes.c_int32 * len(free_pages))(*[int(p) for p in free_pages])
        h = ctypes.c_void_p()
        _check(lib().bca_session_create(ctypes.byref(cache.c), arr, len(free_pages), ctypes.byref(h)),
               "bca_session_create")
        self.h = h

    def unit(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, w: torch.Tensor,
             z: torch.Tensor, n_steps: int, o_scratch: torch.Tensor,
             workspace: Optional[torch.Tensor] = None, use_graph: bool = False,
             stream=None) -> torch.Tensor:
        st = lib().bca_session_unit(
            self.h, _ptr(k_new), _ptr(v_new), _ptr(q), q.shape[0], _ptr(w), _ptr(z), z.shape[1],
            n_steps, _ptr(o_scratch), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            1 if use_graph else 0, _stream(stream))
        _check(st, "bca_session_unit")
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
