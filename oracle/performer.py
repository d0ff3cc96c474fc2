"""Plain float64 CPU oracle of the Wan-Streamer performer step.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the GPU library.

Sources (the web pages about Wan-Streamer; cited by title and section):
  [explainer]  xiaohu-jiedu.pages.dev "wan-streamer-realtime-av", section on
               listening while speaking and its block-causal figure caption;
               deployment section.
  [deep-read]  alwayszhang.cn "全双工语音模型精读⑫：Wan-Streamer", section 3.2
               (noise interpolant and velocity equation), section 4
               (inference schedule, performer step 3).
  [article]    youleyou.com "阿里通义万相发布亚秒级同步AI视频通话基础模型",
               sections 3.1 (block-causal attention) and 3.3 (performer runs
               only the flow-matching solver).
  [wiki]       "Wan-Streamer v0.1: End-to-end Real-time Interactive Foundation
               Models", contribution 3 table (performer: receive KV slice ->
               flow-matching solver -> return clean latents).

Readings where the pages are silent (each also listed in the design notes):
  * a block is one streaming unit of B tokens, blk(t) = t // B;
  * softmax scale 1/sqrt(D), no bias, MHA (query head h reads KV head h);
  * explicit Euler on the uniform grid tau_s = 1 - s/S from tau = 1 (noise);
  * the velocity stand-in is v = O_flat @ W, O_flat[i, h*D + d] = O[i, h, d];
  * cache layout (the library's contract): K pages [P][H][ps][D],
    V pages [P][H][D][ps] (d-major), logical token t at physical page
    page_table[t // ps], slot t % ps;
  * fp8 storage: OCP E4M3FN codes with one fp32 scale per (page, head, K|V),
    scale = amax/448, code = RNE-saturate(x * (448/amax)) in fp32; an append
    that starts inside a page re-quantises that page from its stored values.

Pins (tests/test_oracle_pins.py): brute-force two-key closed form, torch's
scaled_dot_product_attention in float64, dense-mask vs incremental paged
formulation, invariants, the Euler closed form, the OCP E4M3 value table and
torch's float8_e4m3fn cast.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# block-causal visibility  [explainer, listening-while-speaking section and
# figure caption; article 3.1]: tokens of one block see each other both ways,
# a block sees every earlier block and never a later one.
# --------------------------------------------------------------------------


def visibility_mask(n_q: int, q_pos0: int, n_kv: int, block_size: int) -> np.ndarray:
    """bool [n_q, n_kv]: query at global position q_pos0+i sees key j iff
    blk(j) <= blk(q_pos0+i)."""
    qb = (q_pos0 + np.arange(n_q)) // block_size
    kb = np.arange(n_kv) // block_size
    return kb[None, :] <= qb[:, None]


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / np.sum(p, axis=-1, keepdims=True)


def attention_dense(q, k, v, q_pos0: int = 0, block_size: Optional[int] = None,
                    scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
                    heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Formulation (1a): explicit dense mask over the whole key range.

    q [n_q, H, D], k/v [n_kv, H, D].  Returns float64 [len(rows), len(heads), D]
    (all rows / heads by default).  block_size None means every key visible.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, H, D = q.shape
    n_kv = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    heads = np.arange(H) if heads is None else np.asarray(heads)
    if block_size is None:
        mask = np.ones((len(rows), n_kv), dtype=bool)
    else:
        # the rule of visibility_mask, evaluated for the selected rows only
        qb = (q_pos0 + rows) // block_size
        mask = (np.arange(n_kv) // block_size)[None, :] <= qb[:, None]
    out = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    for a, h in enumerate(heads):
        s = (q[rows, h, :] @ k[:, h, :].T) * scale
        s = np.where(mask, s, -np.inf)
        out[:, a, :] = _softmax_rows(s) @ v[:, h, :]
    return out


# --------------------------------------------------------------------------
# paged full-history KV cache  [deep-read section 4 step 3: the performer
# appends the received KV slice to its own full-history cache; wiki
# contribution 3 table].  Paging itself is this library's storage contract.
# --------------------------------------------------------------------------


class PagedCache:
    """float storage (f32 or bf16 values held as float64 here)."""

    def __init__(self, n_heads: int, head_dim: int, page_size: int,
                 page_table: Sequence[int], n_phys: int):
        self.H, self.D, self.ps = n_heads, head_dim, page_size
        self.pt = np.asarray(page_table, dtype=np.int64)
        self.k_pages = np.zeros((n_phys, n_heads, page_size, head_dim))
        self.v_pages = np.zeros((n_phys, n_heads, head_dim, page_size))
        self.n_tokens = 0

    def append(self, k_new, v_new) -> None:
        k_new = np.asarray(k_new, dtype=np.float64)
        v_new = np.asarray(v_new, dtype=np.float64)
        n0 = self.n_tokens
        if n0 + k_new.shape[0] > len(self.pt) * self.ps:
            raise ValueError("append past the mapped pages")
        for r in range(k_new.shape[0]):
            t = n0 + r
            page, slot = self.pt[t // self.ps], t % self.ps
            self.k_pages[page, :, slot, :] = k_new[r]
            self.v_pages[page, :, :, slot] = v_new[r]
        self.n_tokens = n0 + k_new.shape[0]

    def gather(self, n: Optional[int] = None):
        n = self.n_tokens if n is None else n
        K = np.zeros((n, self.H, self.D))
        V = np.zeros((n, self.H, self.D))
        for t in range(n):
            page, slot = self.pt[t // self.ps], t % self.ps
            K[t] = self.k_pages[page, :, slot, :]
            V[t] = self.v_pages[page, :, :, slot]
        return K, V


def attention_over_cache(q_unit, cache, n_kv: Optional[int] = None,
                         scale: Optional[float] = None) -> np.ndarray:
    """Formulation (1b), the streaming call: the current unit's queries attend
    to every cached token [0, n_kv) -- earlier blocks plus their own block,
    which is the whole cache when the unit's slice was the last append."""
    q_unit = np.asarray(q_unit, dtype=np.float64)
    K, V = cache.gather(n_kv)
    n_q, H, D = q_unit.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((n_q, H, D))
    for h in range(H):
        for i in range(n_q):
            s = (K[:, h, :] @ q_unit[i, h, :]) * scale
            w = np.exp(s - s.max())
            out[i, h, :] = (w @ V[:, h, :]) / w.sum()
    return out


def attention_incremental(q, k, v, block_size: int, page_size: int,
                          page_table: Sequence[int], n_phys: int) -> np.ndarray:
    """Unit-by-unit streaming: start from an empty cache; for each block u,
    append its K/V slice, then attend its queries over the cache.  The result
    equals attention_dense(q, k, v, 0, block_size) in exact arithmetic."""
    q = np.asarray(q, dtype=np.float64)
    n, H, D = q.shape
    cache = PagedCache(H, D, page_size, page_table, n_phys)
    out = np.zeros((n, H, D))
    for u0 in range(0, n, block_size):
        u1 = min(n, u0 + block_size)
        cache.append(k[u0:u1], v[u0:u1])
        out[u0:u1] = attention_over_cache(q[u0:u1], cache)
    return out


# --------------------------------------------------------------------------
# fp8 storage (OCP 8-bit floating point spec, E4M3FN: bias 7, 3 mantissa bits,
# subnormals at exponent field 0, S.1111.111 is NaN, no infinities, largest
# finite 448).  Not from the pages: the storage format of the long-history
# cache.
# --------------------------------------------------------------------------


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


_E4M3_POS = e4m3_decode(np.arange(0x7F))     # codes 0x00..0x7E, increasing


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even onto the finite E4M3FN values, saturating at
    +-448.  Ties go to the code with an even (zero) mantissa LSB.  The sign
    bit is copied from x (so -0.0 and tiny negatives give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first >= a
    hi = np.clip(hi, 0, len(_E4M3_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_E4M3_POS) - 1)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_rows(x_rows) -> tuple:
    """Quantise the valid rows of one (page, head, K|V) block.

    x_rows: float32-representable values [n_valid, ...].  Returns
    (codes uint8 same shape, scale float32).  amax over the valid rows;
    scale = amax/448 and inv = 448/amax, both correctly rounded fp32;
    code = e4m3_encode(fp32(x * inv)).  amax = 0 gives scale 1, codes 0.
    """
    x = np.asarray(x_rows, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(1.0)
    scale = np.float32(amax / np.float32(448.0))
    inv = np.float32(np.float32(448.0) / amax)
    prod = (x * inv).astype(np.float32)            # the fp32 decision
    return e4m3_encode(prod), scale


class PagedCacheFP8:
    """fp8 pages: codes in the same layouts as PagedCache, one fp32 scale per
    (physical page, head) for K and for V; rows past the valid length of a
    page hold code 0 and do not enter amax.

    An append that starts inside a partly filled page re-quantises that
    page: the cache holds only codes, so the values of its rows already
    stored are their dequantised values, fp32(decode(code) * scale), and the
    page's block becomes those rows followed by the new ones, quantised by
    the same rule as a fresh page (amax over all its valid rows).  (One scale
    per page and head leaves no other plain choice: keeping the old scale
    would saturate new rows larger than the old ones.)"""

    def __init__(self, n_heads, head_dim, page_size, page_table, n_phys):
        self.H, self.D, self.ps = n_heads, head_dim, page_size
        self.pt = np.asarray(page_table, dtype=np.int64)
        self.k_codes = np.zeros((n_phys, n_heads, page_size, head_dim), np.uint8)
        self.v_codes = np.zeros((n_phys, n_heads, head_dim, page_size), np.uint8)
        self.k_scales = np.ones((n_phys, n_heads), np.float32)
        self.v_scales = np.ones((n_phys, n_heads), np.float32)
        self.n_tokens = 0

    def stored_rows(self, page: int, h: int, n_rows: int):
        """The values the cache holds for the first n_rows rows of (page, h):
        fp32(decode(code) * scale), K and V, each [n_rows, D] float32."""
        k = (e4m3_decode(self.k_codes[page, h, :n_rows, :]) * np.float64(self.k_scales[page, h]))
        v = (e4m3_decode(self.v_codes[page, h, :, :n_rows].T) * np.float64(self.v_scales[page, h]))
        return k.astype(np.float32), v.astype(np.float32)

    def append(self, k_new, v_new) -> None:
        k_new = np.asarray(k_new, dtype=np.float32)
        v_new = np.asarray(v_new, dtype=np.float32)
        n0, n = self.n_tokens, k_new.shape[0]
        if n0 + n > len(self.pt) * self.ps:
            raise ValueError("append past the mapped pages")
        for lp in range(n0 // self.ps, -(-(n0 + n) // self.ps)):
            t0 = lp * self.ps
            r0, r1 = max(t0 - n0, 0), min(n, t0 + self.ps - n0)
            n_old = max(n0 - t0, 0)           # rows already in this page
            page = self.pt[lp]
            for h in range(self.H):
                kb, vb = k_new[r0:r1, h, :], v_new[r0:r1, h, :]
                if n_old:
                    ko, vo = self.stored_rows(page, h, n_old)
                    kb, vb = np.concatenate([ko, kb]), np.concatenate([vo, vb])
                kc, ks = quantize_rows(kb)
                vc, vs = quantize_rows(vb)
                self.k_codes[page, h] = 0
                self.v_codes[page, h] = 0
                self.k_codes[page, h, :len(kb), :] = kc
                self.v_codes[page, h, :, :len(vb)] = vc.T
                self.k_scales[page, h] = ks
                self.v_scales[page, h] = vs
        self.n_tokens = n0 + n

    def gather(self, n: Optional[int] = None):
        """Dequantised K, V [n, H, D] float64: decode(code) * scale, page by
        page (logical page lp holds tokens lp*ps .. lp*ps + ps - 1)."""
        n = self.n_tokens if n is None else n
        K = np.zeros((n, self.H, self.D))
        V = np.zeros((n, self.H, self.D))
        for lp in range(-(-n // self.ps)):
            t0, t1 = lp * self.ps, min(n, (lp + 1) * self.ps)
            page = self.pt[lp]
            ks = self.k_scales[page].astype(np.float64)[:, None, None]   # [H,1,1]
            vs = self.v_scales[page].astype(np.float64)[:, None, None]
            kd = e4m3_decode(self.k_codes[page, :, : t1 - t0, :]) * ks   # [H, rows, D]
            vd = e4m3_decode(self.v_codes[page, :, :, : t1 - t0]) * vs   # [H, D, rows]
            K[t0:t1] = kd.transpose(1, 0, 2)
            V[t0:t1] = vd.transpose(2, 0, 1)
        return K, V


# --------------------------------------------------------------------------
# velocity stand-in and flow-matching Euler solver
# [deep-read 3.2: z_tau = (1-tau) z0 + tau eps, dz/dtau = eps - z0, tau = 1 is
# noise, tau = 0 clean; deep-read section 4 and article 3.3: the performer runs
# only the flow-matching solver for the next unit]
# --------------------------------------------------------------------------


def velocity(o, w) -> np.ndarray:
    """v[i, c] = sum_{h,d} O[i, h, d] * W[h*D + d, c]."""
    o = np.asarray(o, dtype=np.float64)
    n = o.shape[0]
    return o.reshape(n, -1) @ np.asarray(w, dtype=np.float64)


def euler_solve(z1, vel: Callable[[np.ndarray, float], np.ndarray],
                n_steps: int, record: bool = False):
    """Explicit Euler from tau = 1 to tau = 0 on tau_s = 1 - s/S:
    z <- z - (1/S) * v(z, tau_s).  Returns z(0) (and every iterate if
    record)."""
    z = np.asarray(z1, dtype=np.float64).copy()
    dtau = 1.0 / n_steps
    traj = [z.copy()]
    for s in range(n_steps):
        tau = 1.0 - s / n_steps
        z = z - dtau * vel(z, tau)
        traj.append(z.copy())
    return (z, traj) if record else z


def performer_unit(cache, k_new, v_new, q, w, eps, n_steps: int,
                   scale: Optional[float] = None, rows: Optional[Sequence[int]] = None):
    """One performer unit: append the unit's K/V slice, then run the solver
    whose velocity is the attention output of the unit's queries over the
    whole cache, projected by W.  Q/K/V do not change across solver steps,
    so the attention output is computed once.  Returns (z(0), O).  With rows
    given, only those query rows are evaluated (all heads are needed for the
    projection).

    The unit is one block [explainer, figure caption: the tokens of a block
    see each other in both directions and every earlier block]: its slice is
    the last append, so each of its queries sees every cached key, its own
    slice included, whatever the history length.  (A fixed grid t // n_q
    would cut the unit in two when the history is not a multiple of n_q.)"""
    cache.append(k_new, v_new)
    K, V = cache.gather()
    o = attention_dense(q, K, V, scale=scale, rows=rows)
    v = velocity(o, w)
    eps = np.asarray(eps, dtype=np.float64)
    if rows is not None:
        eps = eps[np.asarray(rows)]
    z = euler_solve(eps, lambda z, tau: v, n_steps)
    return z, o
