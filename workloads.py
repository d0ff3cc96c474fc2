"""Seeded synthetic inputs for the performer step.

This module holds no arithmetic of the method: it only draws random tensors,
rounds them to the storage dtype the workload names and builds page tables.
Both the CPU oracle (tests) and the GPU path (tests, bench) take their inputs
from here, so the two sides see the same values.

Workloads (token counts follow the resolutions quoted on the pages at an
assumed latent stride of 16 and 4 latent frames per 160 ms unit; the 160 ms
unit and 25 FPS come from the youleyou.com article, section 2 item 4, and the
alwayszhang.cn deep read, section 3.3):

  tiny_f32     fp32, 4 heads x 64, block 16, 8 history units + 1, 144 tokens
  v01_unit     bf16, 24 x 128, unit 1024 = 4*(12*21)+16, history 64 units
  v02_attn     bf16, 40 x 128, unit 3712 = 4*(40*23)+32, history 32 units,
               current slice pre-appended, one attention call
  v02_unit     v02 shapes, append + 4 x (attention + Euler), W 5120x16
  v02_long_fp8 v02 unit over 750 history units in an fp8-e4m3 cache
  v02_share8   one GPU's head share of the v02 attention call under
               head-sharded (Ulysses) context parallelism over 8 GPUs:
               5 x 128, the same 3712 queries over 122,496 keys

Draw recipe: every tensor has its own sub-stream, seed = 1000*cfg_index +
slot, slots in the order Q, K_hist, V_hist, K_new, V_new, eps, z0, W.
Q/K/V ~ scale * N(0,1) drawn in fp32 and rounded to nearest-even bf16 where
the workload is bf16; eps, z0, W ~ N(0,1) fp32.  The long fp8 history is
drawn in chunks of two units (a whole number of 256-token pages), chunk c of
slot K_hist / V_hist from seed (1000*cfg_index + slot) * 100000 + c + 1, as
bf16 sources that the cache quantises on append.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

SLOTS = {"q": 0, "k_hist": 1, "v_hist": 2, "k_new": 3, "v_new": 4,
         "eps": 5, "z0": 6, "w": 7, "q_catchup": 8}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    dtype: str            # "f32" | "bf16" | "fp8" (cache dtype; Q is bf16 for fp8)
    n_heads: int
    head_dim: int
    unit_tokens: int      # Lq = block size
    hist_units: int
    qkv_scale: float
    n_ch: int = 16
    n_steps: int = 4
    page_size: int = 256

    @property
    def n_hist(self) -> int:
        return self.hist_units * self.unit_tokens

    @property
    def n_kv(self) -> int:
        return self.n_hist + self.unit_tokens

    @property
    def proj_k(self) -> int:
        return self.n_heads * self.head_dim

    def attn_flops(self) -> float:
        """Algorithmic FLOPs of one streaming attention call: QK^T and PV over
        every visible (query, key) pair, 2*D each."""
        return 4.0 * self.n_heads * self.head_dim * self.unit_tokens * self.n_kv


def catchup_span(w: Workload, units: int):
    """Catch-up (multi-block) call on a workload's cache: the queries are
    the last `units` units of the cache (q_pos0 = n_kv - units * B, block
    size B = one unit), drawn from their own seed slot.  Returns (q_pos0,
    n_q, algorithmic FLOPs): each block sees every earlier key and its own
    block, so block b (0-based) costs 4*H*D*B*(q_pos0 + (b + 1) * B)."""
    B = w.unit_tokens
    n_q = units * B
    q_pos0 = w.n_kv - n_q
    keys = sum(q_pos0 + (b + 1) * B for b in range(units))
    return q_pos0, n_q, 4.0 * w.n_heads * w.head_dim * B * keys


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 0, "f32", 4, 64, 16, 8, 1.0),
    "v01_unit": Workload("v01_unit", 1, "bf16", 24, 128, 1024, 64, 0.5),
    "v02_attn": Workload("v02_attn", 2, "bf16", 40, 128, 3712, 32, 0.5),
    "v02_unit": Workload("v02_unit", 3, "bf16", 40, 128, 3712, 32, 0.5),
    "v02_long_fp8": Workload("v02_long_fp8", 4, "fp8", 40, 128, 3712, 750, 0.5),
    "v02_share8": Workload("v02_share8", 5, "bf16", 5, 128, 3712, 32, 0.5),
}


def seed_for(index: int, slot: str) -> int:
    return 1000 * index + SLOTS[slot]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed: int, scale: float = 1.0, device="cpu") -> torch.Tensor:
    """fp32 N(0, scale^2) draw from its own seeded stream."""
    t = torch.randn(*shape, generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t


def to_storage(t: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round an fp32 draw to the storage dtype (nearest-even for bf16)."""
    if dtype == "f32":
        return t
    return t.to(torch.bfloat16)


def qkv(seed: int, n_tok: int, n_heads: int, head_dim: int, scale: float,
        dtype: str, device="cpu") -> torch.Tensor:
    """[n_tok, n_heads, head_dim] tensor ~ scale*N(0,1), rounded to dtype
    (fp8 caches are fed bf16 sources)."""
    t = randn((n_tok, n_heads, head_dim), seed, scale, device)
    return to_storage(t, "f32" if dtype == "f32" else "bf16")


def page_table(n_logical: int, n_phys: int, seed: Optional[int],
               device="cpu") -> torch.Tensor:
    """Logical page -> physical page.  seed=None gives the identity mapping;
    otherwise a seeded random injection into [0, n_phys)."""
    if seed is None:
        pt = torch.arange(n_logical, dtype=torch.int32)
    else:
        perm = torch.randperm(n_phys, generator=_gen(seed, "cpu"))
        pt = perm[:n_logical].to(torch.int32)
    return pt.to(device)


def make_unit_inputs(w: Workload, device="cpu", hist_units: Optional[int] = None,
                     unit_tokens: Optional[int] = None):
    """All tensors of one performer unit.  hist_units / unit_tokens override
    the workload's sizes (used by reduced-size parity cases that keep the
    workload's heads, head_dim and recipe)."""
    hu = w.hist_units if hist_units is None else hist_units
    lq = w.unit_tokens if unit_tokens is None else unit_tokens
    H, D, s = w.n_heads, w.head_dim, w.qkv_scale
    i = w.index
    dt = w.dtype
    out = {
        "q": qkv(seed_for(i, "q"), lq, H, D, s, dt, device),
        "k_hist": qkv(seed_for(i, "k_hist"), hu * lq, H, D, s, dt, device),
        "v_hist": qkv(seed_for(i, "v_hist"), hu * lq, H, D, s, dt, device),
        "k_new": qkv(seed_for(i, "k_new"), lq, H, D, s, dt, device),
        "v_new": qkv(seed_for(i, "v_new"), lq, H, D, s, dt, device),
        "eps": randn((lq, w.n_ch), seed_for(i, "eps"), 1.0, device),
        "z0": randn((lq, w.n_ch), seed_for(i, "z0"), 1.0, device),
        "w": randn((H * D, w.n_ch), seed_for(i, "w"), 1.0, device),
    }
    return out


def peaky(t: torch.Tensor, factor: float) -> torch.Tensor:
    """Scale a bf16/f32 tensor by an exact power of two (keeps values
    representable), used for the sharp-softmax variants."""
    return (t.float() * factor).to(t.dtype)


def hist_chunk_tokens(w: Workload) -> int:
    """Tokens per history chunk: two units (7424 at v0.2 = 29 pages)."""
    return 2 * w.unit_tokens


def hist_chunk(w: Workload, slot: str, c: int, device="cpu") -> torch.Tensor:
    """History chunk c ([hist_chunk_tokens, H, D] bf16) of K_hist or V_hist."""
    if slot not in ("k_hist", "v_hist"):
        raise ValueError(slot)
    n = hist_chunk_tokens(w)
    if (c + 1) * n > w.n_hist:
        raise ValueError("chunk past the history")
    seed = seed_for(w.index, slot) * 100000 + c + 1
    return qkv(seed, n, w.n_heads, w.head_dim, w.qkv_scale, "bf16", device)


def n_hist_chunks(w: Workload) -> int:
    return w.n_hist // hist_chunk_tokens(w)
