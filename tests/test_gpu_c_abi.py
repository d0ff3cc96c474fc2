"""The C ABI driven from plain C: tests/c_abi/performer_unit_c (gcc, built
by __graft_entry__.build()) reads a unit's inputs, appends the history and
runs performer_unit with its own hipMalloc'd buffers and workspace; its
outputs must match the oracle's performer unit as the Python binding's do
(bf16 2e-2 max-abs, relative RMS 1e-2 for O)."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import assert_close, assert_latents, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi", "performer_unit_c")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n_hist,n_q,ps", [(320, 100, 64), (0, 256, 256), (1000, 200, 16)])
def test_c_driver_performer_unit(tmp_path, n_hist, n_q, ps):
    assert os.path.exists(DRIVER), "build the C driver first (__graft_entry__.build())"
    H, D, n_ch, steps = 2, 128, 16, 4
    n_log = -(-(n_hist + n_q) // ps)
    n_phys = n_log + 2
    say(f"C driver: n_hist={n_hist} n_q={n_q} ps={ps}")
    pt = workloads.page_table(n_log, n_phys, 17)
    kh = workloads.qkv(71, n_hist, H, D, 0.5, "bf16")
    vh = workloads.qkv(72, n_hist, H, D, 0.5, "bf16")
    kn = workloads.qkv(73, n_q, H, D, 0.5, "bf16")
    vn = workloads.qkv(74, n_q, H, D, 0.5, "bf16")
    q = workloads.qkv(75, n_q, H, D, 0.5, "bf16")
    w = workloads.randn((H * D, n_ch), 76)
    eps = workloads.randn((n_q, n_ch), 77)
    src = tmp_path / "in.bin"
    dst = tmp_path / "out.bin"
    with open(src, "wb") as f:
        np.array([H, D, ps, n_hist, n_q, n_ch, steps, n_phys], dtype="<i8").tofile(f)
        pt.numpy().astype("<i4").tofile(f)
        for t in (kh, vh, kn, vn, q):
            _bits(t).astype("<u2").tofile(f)
        w.numpy().astype("<f4").tofile(f)
        eps.numpy().astype("<f4").tofile(f)
    r = subprocess.run([DRIVER, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(dst, dtype=np.uint8)
    o_bytes = n_q * H * D * 2
    assert raw.size == o_bytes + n_q * n_ch * 4
    o_bits = raw[:o_bytes].view("<u2").reshape(n_q, H, D)
    o = torch.from_numpy(o_bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    z = raw[o_bytes:].view("<f4").reshape(n_q, n_ch).astype(np.float64)

    cache = oracle.PagedCache(H, D, ps, pt.numpy(), n_phys)
    if n_hist:
        cache.append(kh.double().numpy(), vh.double().numpy())
    zw, ow = oracle.performer_unit(cache, kn.double().numpy(), vn.double().numpy(),
                                   q.double().numpy(), w.double().numpy(),
                                   eps.double().numpy(), steps)
    assert_close(o, ow, 2e-2, 1e-2, what="C driver O")
    assert_latents(z, zw, eps.double().numpy(), 2e-2, 1e-2, what="C driver")
