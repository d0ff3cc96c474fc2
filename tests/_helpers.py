"""Shared helpers of the GPU parity tests (input plumbing and error metrics
only; the expected values always come from the oracle package)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errs(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = got - want
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    ref = float(np.max(np.abs(want))) if want.size else 0.0
    rel_rms = float(np.sqrt(np.mean(d * d)) / max(np.sqrt(np.mean(want * want)), 1e-30))
    return max_abs, rel_rms, ref


def assert_close(got, want, max_abs, rel_rms=None, what=""):
    ma, rr, ref = errs(got, want)
    say(f"  {what}: max_abs={ma:.3e} rel_rms={rr:.3e} max|ref|={ref:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert ma <= max_abs, f"{what}: max_abs {ma:.3e} > {max_abs:.3e}"
    if rel_rms is not None:
        assert rr <= rel_rms, f"{what}: rel_rms {rr:.3e} > {rel_rms:.3e}"


def make_caches(bca, H, D, ps, dtype, capacity, shuffle=None, extra=2, device="cuda"):
    """A GPU cache and an oracle cache over the same page table."""
    n_log = -(-capacity // ps)
    n_phys = n_log + extra
    pt = workloads.page_table(n_log, n_phys, shuffle)
    g = bca.KVCache(H, D, ps, pt, n_phys, dtype, device=device)
    if dtype == "fp8":
        o = oracle.PagedCacheFP8(H, D, ps, pt.numpy(), n_phys)
    else:
        o = oracle.PagedCache(H, D, ps, pt.numpy(), n_phys)
    return g, o, pt


def assert_latents(z_got, z_want, eps, max_abs, rel_rms=1e-2, what=""):
    """Latents after the solver: z itself within max_abs, and the solver's
    move z - eps (= -sum of dtau * v) within relative RMS `rel_rms`.  With
    |eps| ~ 1 and a move of ~0.1, a check of z alone at rel_rms would let a
    velocity several percent off pass."""
    z_got = np.asarray(z_got, dtype=np.float64)
    z_want = np.asarray(z_want, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    assert_close(z_got, z_want, max_abs, what=f"{what} z")
    assert_close(z_got - eps, z_want - eps, max_abs, rel_rms, what=f"{what} z - eps")
