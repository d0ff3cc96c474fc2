"""Pins of the CPU oracle against facts fixed outside it: worked examples from
the pages (golden fixtures), closed forms, library routines (torch float64
attention, torch float8 cast) and invariants.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0, rng=RNG):
    return rng.standard_normal(shape) * scale


def _load_golden(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


# ---------------------------------------------------------------- visibility


def test_block_visibility_matches_page_figure(golden_path):
    want = np.array(_load_golden(golden_path("block_visibility.txt")), dtype=int)
    # block level: one token per block
    got = oracle.visibility_mask(4, 0, 4, 1).astype(int)
    np.testing.assert_array_equal(got, want)
    # token level, 3 tokens per block: expands the block matrix
    tok = oracle.visibility_mask(12, 0, 12, 3).astype(int)
    np.testing.assert_array_equal(tok, np.kron(want, np.ones((3, 3), dtype=int)))


def test_visibility_streaming_call_sees_everything():
    # the last unit's queries at positions [n-B, n) with block B see all n keys
    m = oracle.visibility_mask(16, 128, 144, 16)
    assert m.all()
    # a key one block ahead is hidden
    m = oracle.visibility_mask(16, 128, 160, 16)
    assert m[:, :144].all() and not m[:, 144:].any()


# ---------------------------------------------------------------- attention


def test_two_key_closed_form():
    """1 query, 2 keys: o = sigma(s1 - s0) v1 + (1 - sigma(s1 - s0)) v0."""
    D = 8
    q = _rand(1, 1, D)
    k = _rand(2, 1, D)
    v = _rand(2, 1, D)
    s = (k[:, 0, :] @ q[0, 0, :]) / math.sqrt(D)
    sig = 1.0 / (1.0 + math.exp(-(s[1] - s[0])))
    want = sig * v[1, 0] + (1.0 - sig) * v[0, 0]
    got = oracle.attention_dense(q, k, v, 1, 2)[0, 0]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)
    # the same query placed in block 0 with block size 1 sees only key 0
    got0 = oracle.attention_dense(q, k[:1], v[:1], 0, 1)[0, 0]
    np.testing.assert_allclose(got0, v[0, 0], rtol=0, atol=1e-15)


def _sdpa(q, k, v, mask=None, is_causal=False):
    # torch float64 on CPU, layout [H, L, D]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, is_causal=is_causal)
    return o.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("B", [1, 3, 16, 64])
def test_dense_matches_torch_sdpa(B):
    L, H, D = 48, 3, 16
    q, k, v = (_rand(L, H, D) for _ in range(3))
    got = oracle.attention_dense(q, k, v, 0, B)
    if B == 1:
        want = _sdpa(q, k, v, is_causal=True)      # block 1 == causal
    elif B >= L:
        want = _sdpa(q, k, v)                      # one block == no mask
    else:
        blk = np.arange(L) // B
        want = _sdpa(q, k, v, mask=blk[None, :] <= blk[:, None])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_dense_offset_queries_match_sdpa():
    """queries of the last unit over a longer history (q_pos0 > 0)."""
    n_kv, n_q, H, D, B = 70, 10, 2, 8, 10
    q = _rand(n_q, H, D)
    k = _rand(n_kv, H, D)
    v = _rand(n_kv, H, D)
    got = oracle.attention_dense(q, k, v, n_kv - n_q, B)
    want = _sdpa(q, k, v)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # a middle unit: q_pos0 = 30 sees keys < 40 only
    got = oracle.attention_dense(q, k, v, 30, B)
    want = _sdpa(q, k[:40], v[:40])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def _tiny():
    w = workloads.WORKLOADS["tiny_f32"]
    n = w.n_kv
    q = workloads.qkv(11, n, w.n_heads, w.head_dim, 1.0, "f32").numpy()
    k = workloads.qkv(12, n, w.n_heads, w.head_dim, 1.0, "f32").numpy()
    v = workloads.qkv(13, n, w.n_heads, w.head_dim, 1.0, "f32").numpy()
    return w, q, k, v


@pytest.mark.parametrize("ps,shuffle", [(256, None), (16, None), (16, 5), (32, 9)])
def test_incremental_equals_full_sequence(ps, shuffle):
    """Unit-by-unit streaming over a paged cache equals one full-sequence call
    under the explicit block mask (exact up to float64 rounding order)."""
    w, q, k, v = _tiny()
    n_log = -(-w.n_kv // ps)
    n_phys = n_log + 3
    pt = workloads.page_table(n_log, n_phys, shuffle).numpy()
    inc = oracle.attention_incremental(q, k, v, w.unit_tokens, ps, pt, n_phys)
    full = oracle.attention_dense(q, k, v, 0, w.unit_tokens)
    np.testing.assert_allclose(inc, full, rtol=1e-12, atol=1e-13)


def test_invariants():
    w, q, k, v = _tiny()
    B = w.unit_tokens
    base = oracle.attention_dense(q, k, v, 0, B)
    # P1 constant V gives that constant
    c = _rand(1, w.n_heads, w.head_dim)
    o = oracle.attention_dense(q, k, np.broadcast_to(c, v.shape), 0, B)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-13, atol=1e-13)
    # P2 one planted dominant key: its value comes out
    qq = q.copy()
    kk = k.copy()
    kk[5] = qq[-1] * 40.0
    o = oracle.attention_dense(qq, kk, v, 0, B)
    np.testing.assert_allclose(o[-1], v[5], atol=1e-8)
    # P4 a joint permutation of earlier blocks' keys/values leaves the last
    # unit's output unchanged
    perm = RNG.permutation(w.n_hist)
    k2, v2 = k.copy(), v.copy()
    k2[:w.n_hist], v2[:w.n_hist] = k[perm], v[perm]
    o = oracle.attention_dense(q, k2, v2, 0, B)
    np.testing.assert_allclose(o[w.n_hist:], base[w.n_hist:], rtol=1e-12, atol=1e-13)
    # P6 permuting tokens inside the current unit permutes its output rows
    p6 = w.n_hist + RNG.permutation(B)
    idx = np.concatenate([np.arange(w.n_hist), p6])
    o = oracle.attention_dense(q[idx], k[idx], v[idx], 0, B)
    np.testing.assert_allclose(o[w.n_hist:], base[p6], rtol=1e-12, atol=1e-13)
    # P7 a future block changes nothing before it
    kf = np.concatenate([k, _rand(B, w.n_heads, w.head_dim) * 100])
    vf = np.concatenate([v, _rand(B, w.n_heads, w.head_dim) * 100])
    qf = np.concatenate([q, _rand(B, w.n_heads, w.head_dim)])
    o = oracle.attention_dense(qf, kf, vf, 0, B)
    # (float64 matmul blocking depends on the key count: rounding order only)
    np.testing.assert_allclose(o[:w.n_kv], base, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- paging


@pytest.mark.parametrize("ps", [16, 64, 256])
def test_paging_gather_equals_concat(ps):
    H, D = 3, 8
    sizes = [37, 5, 64, 100, 1]
    n = sum(sizes)
    n_log = -(-n // ps)
    pt = workloads.page_table(n_log, n_log + 4, 77).numpy()
    c = oracle.PagedCache(H, D, ps, pt, n_log + 4)
    ks, vs = [], []
    for s in sizes:
        kk, vv = _rand(s, H, D), _rand(s, H, D)
        c.append(kk, vv)
        ks.append(kk)
        vs.append(vv)
    K, V = c.gather()
    np.testing.assert_array_equal(K, np.concatenate(ks))
    np.testing.assert_array_equal(V, np.concatenate(vs))
    # layout pin: token t sits at page pt[t // ps], slot t % ps; V is d-major
    t = n - 1
    np.testing.assert_array_equal(c.k_pages[pt[t // ps], :, t % ps, :], ks[-1][-1])
    np.testing.assert_array_equal(c.v_pages[pt[t // ps], 2, :, t % ps], vs[-1][-1][2])
    with pytest.raises(ValueError):
        c.append(_rand(n_log * ps, H, D), _rand(n_log * ps, H, D))


# ---------------------------------------------------------------- fp8


def test_e4m3_spec_values(golden_path):
    for code, val in _load_golden(golden_path("e4m3_ocp_values.txt")):
        got = oracle.e4m3_decode(int(code, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes.numpy())
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])


def test_e4m3_encode_roundtrip_midpoints_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = oracle.e4m3_encode(mids)
    lo, hi = np.arange(0x7E), np.arange(1, 0x7F)
    np.testing.assert_array_equal(enc, np.where(lo % 2 == 0, lo, hi))
    assert oracle.e4m3_encode(np.array([1e6, -500.0, 464.0])).tolist() == [0x7E, 0xFE, 0x7E]


def test_e4m3_encode_vs_torch_cast():
    x = np.concatenate([_rand(20000, scale=30.0), _rand(2000, scale=0.01),
                        _rand(2000, scale=1e-4)]).astype(np.float32)
    clamped = np.clip(x, -448, 448)
    want = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(x), want)


def test_quantize_rows_rules():
    x = _rand(100, 16, scale=3.0).astype(np.float32)
    codes, scale = oracle.quantize_rows(x)
    amax = np.float32(np.abs(x).max())
    assert scale == np.float32(amax / np.float32(448))
    # the largest magnitude maps to +-448 exactly
    assert np.abs(oracle.e4m3_decode(codes)).max() == 448.0
    deq = oracle.e4m3_decode(codes) * np.float64(scale)
    # RNE onto 3 mantissa bits: relative error <= 2^-4 for normals
    big = np.abs(x) > amax * 2.0 ** -6
    assert np.all(np.abs(deq[big] - x[big]) <= np.abs(x[big]) * 2.0 ** -4 * 1.0001)
    z, s = oracle.quantize_rows(np.zeros((4, 4), np.float32))
    assert s == 1.0 and not z.any()


def test_fp8_cache_rows_past_valid_are_zero():
    H, D, ps = 2, 8, 16
    c = oracle.PagedCacheFP8(H, D, ps, [3, 1, 0], 4)
    c.append(_rand(20, H, D), _rand(20, H, D))
    assert not c.k_codes[1, :, 4:, :].any() and not c.v_codes[1, :, :, 4:].any()
    # a mid-page append re-quantises page 1: its valid rows grow to 8 and the
    # rows past them stay code 0
    c.append(_rand(4, H, D), _rand(4, H, D))
    assert c.k_codes[1, :, :8, :].any() and not c.k_codes[1, :, 8:, :].any()
    assert not c.v_codes[1, :, :, 8:].any()


def test_fp8_cache_gather_is_identity_on_the_grid():
    """Values on the E4M3 grid with each page's amax = 448 have scale 1 and
    inv 1 exactly, so append + gather returns them unchanged: a transposed
    V block, a wrong page or slot, or a dropped scale shows up as a
    mismatch.  Pages are shuffled and the last page is partial."""
    H, D, ps = 3, 8, 16
    rng = np.random.default_rng(7)
    n = 3 * ps + 5
    grid = oracle.e4m3_decode(np.arange(0x7F))           # 0 .. 448
    k = rng.choice(grid, size=(n, H, D)) * rng.choice([-1.0, 1.0], size=(n, H, D))
    v = rng.choice(grid, size=(n, H, D)) * rng.choice([-1.0, 1.0], size=(n, H, D))
    for t0 in range(0, n, ps):                            # amax 448 in every page and head
        k[t0, :, 0] = 448.0
        v[t0, :, 1] = -448.0
    c = oracle.PagedCacheFP8(H, D, ps, [2, 0, 3, 1], 4)
    c.append(k.astype(np.float32), v.astype(np.float32))
    assert np.all(c.k_scales[[2, 0, 3, 1]] == 1.0) and np.all(c.v_scales[[2, 0, 3, 1]] == 1.0)
    K, V = c.gather()
    np.testing.assert_array_equal(K, k)
    np.testing.assert_array_equal(V, v)
    # a non-unit scale multiplies back: halve every value, scale 0.5
    c2 = oracle.PagedCacheFP8(H, D, ps, [1, 3, 0, 2], 4)
    c2.append((k / 2).astype(np.float32), (v / 2).astype(np.float32))
    K2, V2 = c2.gather()
    np.testing.assert_array_equal(K2, k / 2)
    np.testing.assert_array_equal(V2, v / 2)


# ---------------------------------------------------------------- velocity / Euler


def test_velocity_index_order():
    # O[0, h, d] = 1 only at h=1, d=0 with H=2, D=3: picks row h*D + d = 3 of W
    o = np.zeros((1, 2, 3))
    o[0, 1, 0] = 1.0
    w = np.arange(12.0).reshape(6, 2)
    np.testing.assert_array_equal(oracle.velocity(o, w), [[6.0, 7.0]])
    o = _rand(5, 4, 6)
    w = _rand(24, 16)
    want = torch.from_numpy(o.reshape(5, 24)) @ torch.from_numpy(w)
    np.testing.assert_allclose(oracle.velocity(o, w), want.numpy(), rtol=1e-14, atol=1e-14)


def test_euler_golden_interpolant(golden_path):
    rows = np.array(_load_golden(golden_path("euler_interpolant.txt")), dtype=float)
    z0, eps = rows[-1, 1:], rows[0, 1:]
    z, traj = oracle.euler_solve(eps, lambda z, tau: eps - z0, 4, record=True)
    for s, zz in enumerate(traj):
        assert rows[s, 0] == 1.0 - s / 4
        np.testing.assert_array_equal(zz, rows[s, 1:])


def test_euler_closed_form_random():
    """exact velocity eps - z0: every iterate is (1-tau)z0 + tau*eps and the
    last one is z0 (within a few ulp)."""
    for S in (1, 4, 7):
        z0 = _rand(16, 16)
        eps = _rand(16, 16)
        z, traj = oracle.euler_solve(eps, lambda z, tau: eps - z0, S, record=True)
        bound = 8 * np.finfo(np.float64).eps * np.maximum(np.abs(z0), np.abs(eps)).max()
        for s, zz in enumerate(traj):
            tau = 1.0 - s / S
            np.testing.assert_allclose(zz, (1 - tau) * z0 + tau * eps, rtol=0, atol=bound)
        np.testing.assert_allclose(z, z0, rtol=0, atol=bound)


def test_euler_direction_and_tau_grid():
    taus = []
    oracle.euler_solve(np.zeros(1), lambda z, t: taus.append(t) or np.ones(1), 4)
    assert taus == [1.0, 0.75, 0.5, 0.25]
    z = oracle.euler_solve(np.zeros(1), lambda z, t: np.ones(1), 4)
    assert z[0] == -1.0          # moving tau 1 -> 0 subtracts dtau * v


def test_performer_unit_composes_pieces():
    H, D, B, ps = 2, 8, 4, 16
    pt = [2, 0, 1]
    c = oracle.PagedCache(H, D, ps, pt, 3)
    hist_k, hist_v = _rand(12, H, D), _rand(12, H, D)
    c.append(hist_k, hist_v)
    kn, vn, q = _rand(B, H, D), _rand(B, H, D), _rand(B, H, D)
    w = _rand(H * D, 3)
    eps = _rand(B, 3)
    z, o = oracle.performer_unit(c, kn, vn, q, w, eps, 4)
    K = np.concatenate([hist_k, kn])
    V = np.concatenate([hist_v, vn])
    want_o = _sdpa(q, K, V)
    np.testing.assert_allclose(o, want_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z, eps - (want_o.reshape(B, -1) @ w), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n_hist,B", [(12, 5), (7, 4), (0, 3), (30, 7)])
def test_performer_unit_sees_its_whole_slice_on_any_history(n_hist, B):
    """The unit is one block whose tokens see each other both ways (explainer,
    figure caption of the block-causal mask), also when the history is not a
    multiple of the unit: with a 12-token history and a 5-token unit, query 0
    (global position 12) must see key 16, the unit's last.  A key planted
    there as a large multiple of query 0 takes all of that query's weight,
    so its output is that key's value; and every row equals unmasked
    attention over the whole cache (torch float64)."""
    H, D, ps = 2, 8, 4
    n_pages = -(-(n_hist + B) // ps)
    pt = list(np.random.default_rng(n_hist).permutation(n_pages))
    c = oracle.PagedCache(H, D, ps, pt, n_pages)
    hist_k, hist_v = _rand(n_hist, H, D), _rand(n_hist, H, D)
    if n_hist:
        c.append(hist_k, hist_v)
    kn, vn, q = _rand(B, H, D), _rand(B, H, D), _rand(B, H, D)
    # the unit's last key, matched to query 0: logit 200/sqrt(D) ~ 70 per head
    kn[B - 1] = q[0] * (200.0 / np.sum(q[0] * q[0], axis=-1, keepdims=True))
    w = _rand(H * D, 3)
    z, o = oracle.performer_unit(c, kn, vn, q, w, _rand(B, 3), 4)
    np.testing.assert_allclose(o[0], vn[B - 1], rtol=0, atol=1e-9)
    K = np.concatenate([hist_k, kn])
    V = np.concatenate([hist_v, vn])
    np.testing.assert_allclose(o, _sdpa(q, K, V), rtol=1e-12, atol=1e-13)


# ------------------------------------------- fp8 appends inside a page


def _e4m3_half_step(y):
    """Half the spacing of the E4M3 grid around |y| <= 448 (in the units of
    y): 2^-10 in the subnormal range, else 2^(e-4) for y in [2^e, 2^(e+1))."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))


def test_fp8_requant_keeps_values_already_on_the_grid():
    """A page whose first rows have amax 448 * 2^-3 (scale 2^-3, exact) and lie
    on that scale's E4M3 grid, then a mid-page append of smaller rows on the
    same grid: the scale cannot change, so re-quantising changes nothing and
    the split append equals one append of all rows, bit for bit."""
    H, D, ps = 2, 16, 64
    rng = np.random.default_rng(5)
    grid = oracle.e4m3_decode(np.arange(0x7F)) * 2.0 ** -3          # non-negative grid values
    x = rng.choice(grid[:100], size=(40, H, D)) * rng.choice([-1.0, 1.0], size=(40, H, D))
    x[0] = 448.0 * 2.0 ** -3                                       # the amax, in the old rows
    y = rng.choice(grid[:100], size=(40, H, D))
    y[5] = 448.0 * 2.0 ** -3
    split = oracle.PagedCacheFP8(H, D, ps, [1, 0], 2)
    split.append(x[:23].astype(np.float32), y[:23].astype(np.float32))
    split.append(x[23:].astype(np.float32), y[23:].astype(np.float32))
    whole = oracle.PagedCacheFP8(H, D, ps, [1, 0], 2)
    whole.append(x.astype(np.float32), y.astype(np.float32))
    np.testing.assert_array_equal(split.k_codes, whole.k_codes)
    np.testing.assert_array_equal(split.v_codes, whole.v_codes)
    np.testing.assert_array_equal(split.k_scales, whole.k_scales)
    K, V = split.gather()
    np.testing.assert_array_equal(K, x)                              # exact: on the grid
    np.testing.assert_array_equal(V, y)


@pytest.mark.parametrize("n_old,grow", [(37, 4.0), (1, 0.25), (63, 1.0)])
def test_fp8_requant_rounding_bounds(n_old, grow):
    """Random rows, then a mid-page append whose rows are `grow` times larger:
    every value the page now holds is one round-to-nearest of its input (the
    old rows' input being the values they held) onto the new scale's grid,
    within half a step; an old row also stays within half a step at the old
    scale plus half a step at the new one of its original source; pages
    after the split page are those of a single append, bit for bit."""
    H, D, ps = 3, 32, 64
    rng = np.random.default_rng(n_old)
    n = 150
    x = (rng.standard_normal((n, H, D)) * 0.5).astype(np.float32)
    x[n_old:] *= np.float32(grow)
    c = oracle.PagedCacheFP8(H, D, ps, [2, 0, 1], 3)
    c.append(x[:n_old], x[:n_old])
    held = c.gather()[0][:n_old]                                   # values before the append
    s_old = c.k_scales[2].astype(np.float64)
    c.append(x[n_old:], x[n_old:])
    K, V = c.gather()
    np.testing.assert_array_equal(K, V)                              # K and V follow one rule
    s_new = c.k_scales[2].astype(np.float64)                         # page of the split (logical 0)
    src = np.concatenate([held, x[n_old:ps]]).astype(np.float64)     # inputs of the split page
    for h in range(H):
        y = src[:, h] / s_new[h]
        assert np.all(np.abs(K[:ps, h] / s_new[h] - y) <= _e4m3_half_step(y) * (1 + 1e-6))
        assert np.all(np.abs(K[:n_old, h] - x[:n_old, h]) <=
                      (_e4m3_half_step(x[:n_old, h] / s_old[h]) * s_old[h] +
                       _e4m3_half_step(held[:, h] / s_new[h]) * s_new[h]) * (1 + 1e-6))
    whole = oracle.PagedCacheFP8(H, D, ps, [2, 0, 1], 3)
    whole.append(x, x)
    np.testing.assert_array_equal(c.k_codes[[0, 1]], whole.k_codes[[0, 1]])
    np.testing.assert_array_equal(c.k_scales[[0, 1]], whole.k_scales[[0, 1]])
