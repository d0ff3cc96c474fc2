"""Pins of the oracle's plain C fp8 quantiser and decoder (oracle/fp8c.py,
oracle/fp8_cache.c) against facts outside it: torch's float8_e4m3fn cast
(a library routine) after the clamp to +-448, the OCP E4M3 value table of
tests/golden/e4m3_ocp_values.txt, and bitwise equality with the numpy
oracle, which has its own pins.  CPU only."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8c


def _load_golden(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def _inputs():
    """Every finite bf16 value as fp32, log-uniform random fp32 values over
    2^-16 .. 2^10 of both signs, every midpoint between neighbouring E4M3
    values and the fp32 values next to it, zeros, 448, 464 and beyond."""
    b = np.arange(1 << 16, dtype=np.uint32) << 16
    bf = b.view(np.float32)
    bf = bf[np.isfinite(bf)]
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-16, 10, 1 << 20)).astype(np.float32)
    rnd = np.where(rng.random(1 << 20) < 0.5, -mag, mag).astype(np.float32)
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    special = np.array([0.0, -0.0, 448.0, -448.0, 464.0, 500.0, -1e30, 2.0 ** -9, 2.0 ** -10,
                        3 * 2.0 ** -10, 2.0 ** -6], dtype=np.float32)
    return np.concatenate([bf, rnd, near, -near, special]).astype(np.float32)


def test_c_encoder_equals_numpy_oracle_and_torch_cast():
    x = _inputs()
    got = fp8c.e4m3_encode(x)
    np.testing.assert_array_equal(got, oracle.e4m3_encode(x))
    t = torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, t)


def test_c_decoder_matches_ocp_table_and_torch(golden_path):
    codes = np.arange(256, dtype=np.uint8)
    got = fp8c.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], want[~nan])
    for code, val in _load_golden(golden_path("e4m3_ocp_values.txt")):
        g = got[int(code, 16)]
        if val == "nan":
            assert np.isnan(g)
        else:
            assert g == float(val) and np.signbit(g) == val.startswith("-"), (code, val, g)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


@pytest.mark.parametrize("n_tok,H,D,ps", [(300, 3, 128, 64), (256, 2, 128, 256), (37, 1, 32, 16),
                                          (1000, 2, 64, 128)])
def test_c_quantiser_equals_numpy_cache(n_tok, H, D, ps):
    """Codes and scales of a page-aligned slice (ragged last page) bit for
    bit equal to oracle.PagedCacheFP8.append, K and V layouts; the dequantised
    heads equal its gather.  One block holds crafted ties and the 448 bound,
    one is all zeros (scale 1, codes 0), one holds only -0."""
    rng = np.random.default_rng(n_tok)
    k = (rng.standard_normal((n_tok, H, D)) * 0.5).astype(np.float32)
    v = (rng.standard_normal((n_tok, H, D)) * 0.5).astype(np.float32)
    ties = np.array([1.0625, 17.0, 2.0 ** -10, 232.0, 1.9375, 448.0, -1.0625, -(2.0 ** -10)])
    k[:min(ps, n_tok), 0] = rng.choice(ties, size=(min(ps, n_tok), D))
    v[:min(ps, n_tok), H - 1] = 0.0
    if n_tok > ps:
        k[ps:2 * ps, H - 1] = -0.0
    kb, vb = _bf16_bits(k), _bf16_bits(v)
    kf = torch.from_numpy(kb).view(torch.bfloat16).float().numpy()
    vf = torch.from_numpy(vb).view(torch.bfloat16).float().numpy()
    n_pages = -(-n_tok // ps)
    ref = oracle.PagedCacheFP8(H, D, ps, np.arange(n_pages), n_pages)
    ref.append(kf, vf)
    kc, ks = fp8c.quantize_pages(kb, ps, v_layout=False)
    vc, vs = fp8c.quantize_pages(vb, ps, v_layout=True)
    np.testing.assert_array_equal(kc, ref.k_codes)
    np.testing.assert_array_equal(vc, ref.v_codes)
    np.testing.assert_array_equal(ks, ref.k_scales)
    np.testing.assert_array_equal(vs, ref.v_scales)
    K, V = ref.gather()
    for h in range(H):
        np.testing.assert_array_equal(fp8c.decode_head(kc, ks, n_tok, h, False), K[:, h])
        np.testing.assert_array_equal(fp8c.decode_head(vc, vs, n_tok, h, True), V[:, h])


def test_c_quantiser_fills_views_in_place():
    """Chunks quantised into views of one large array give the same codes as
    one call over the whole slice (chunks of whole pages)."""
    rng = np.random.default_rng(3)
    x = _bf16_bits((rng.standard_normal((640, 2, 64)) * 0.5).astype(np.float32))
    whole, ws = fp8c.quantize_pages(x, 64, v_layout=True)
    codes = np.zeros_like(whole)
    scales = np.zeros_like(ws)
    for c0 in range(0, 640, 128):
        p0 = c0 // 64
        fp8c.quantize_pages(x[c0:c0 + 128], 64, True, codes[p0:p0 + 2], scales[p0:p0 + 2])
    np.testing.assert_array_equal(codes, whole)
    np.testing.assert_array_equal(scales, ws)
