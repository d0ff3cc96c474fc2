"""numpy front end of oracle/fp8_cache.c, the plain C part of the CPU oracle
(the fp8 KV-cache quantiser and decoder).  TEST INFRASTRUCTURE ONLY: used by
tests/ for the long fp8 history, where the numpy encoder of
oracle/performer.py is too slow; the GPU library never calls it.

build() compiles the C file with gcc (C11, no floating-point contraction,
OpenMP); the functions build it on first use when the shared object is
missing or older than its source.  See fp8_cache.c for the definitions and
tests/test_oracle_fp8c.py for the pins (bitwise equality with the numpy
oracle and torch's float8_e4m3fn cast).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "fp8_cache.c")
LIB = os.path.join(_HERE, "_fp8_cache.so")
_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           "-Werror", SRC, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle C build failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    L = ctypes.CDLL(LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.orc_e4m3_encode.argtypes = [vp, vp, i64]
    L.orc_e4m3_decode.argtypes = [vp, vp, i64]
    L.orc_quantize_pages.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp]
    L.orc_decode_head.argtypes = [vp, vp, i64, i32, i32, i32, i32, i32, vp]
    for f in (L.orc_e4m3_encode, L.orc_e4m3_decode, L.orc_quantize_pages, L.orc_decode_head):
        f.restype = None
    _lib = L
    return L


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN codes of float32 values (round to nearest even, saturating)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_encode(_p(x), _p(out), x.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_decode(_p(c), _p(out), c.size)
    return out


def quantize_pages(src_bf16_bits, page_size: int, v_layout: bool, codes=None, scales=None):
    """Quantise a page-aligned slice [n_tok][H][D] given as bf16 bit patterns
    (uint16 / int16).  Returns (codes [n_pages][H][ps][D], or [n_pages][H][D][ps]
    for V, uint8; scales [n_pages][H] float32); codes / scales may be given
    (views of larger arrays) to be filled in place."""
    src = np.ascontiguousarray(src_bf16_bits).view(np.uint16)
    n_tok, H, D = src.shape
    n_pages = -(-n_tok // page_size)
    shape = (n_pages, H, D, page_size) if v_layout else (n_pages, H, page_size, D)
    if codes is None:
        codes = np.empty(shape, dtype=np.uint8)
    if scales is None:
        scales = np.empty((n_pages, H), dtype=np.float32)
    assert codes.shape == shape and codes.dtype == np.uint8
    assert scales.shape == (n_pages, H) and scales.dtype == np.float32
    _load().orc_quantize_pages(_p(src), n_tok, H, D, page_size, int(v_layout), _p(codes), _p(scales))
    return codes, scales


def decode_head(codes, scales, n_tok: int, head: int, v_layout: bool) -> np.ndarray:
    """Dequantised K or V of one head, [n_tok][D] float64, from codes and
    scales laid out as quantize_pages writes them (pages in logical order)."""
    n_pages, H = scales.shape
    D = codes.shape[2] if v_layout else codes.shape[3]
    ps = codes.shape[3] if v_layout else codes.shape[2]
    assert n_tok <= n_pages * ps and 0 <= head < H
    out = np.empty((n_tok, D), dtype=np.float64)
    _load().orc_decode_head(_p(codes), _p(scales), n_tok, H, D, ps, head, int(v_layout), _p(out))
    return out
