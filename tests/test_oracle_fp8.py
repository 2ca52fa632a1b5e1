"""Pins of the oracle's fp8 E4M3 state: the codec against torch's
float8_e4m3fn conversion (a library routine), a brute-force nearest search
over the finite values and the format's named values; the fp8 scan against
an elementwise numpy model of the binary32 update, and its invariants."""
import numpy as np
import pytest

import oracle
import sdm_inputs as S


def _table():
    return np.array([oracle.fp8_to_double(c) for c in range(256)])


def test_named_values_and_order():
    t = _table()
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x00] == 0.0
    assert np.all(np.diff(t[:0x7F]) > 0)  # codes 0..0x7E increase
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def _library_codes(x):
    import torch

    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _inputs():
    t = _table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2  # exact in binary32 (4 significant bits)
    x = [t, -t, mids, -mids]
    f32 = mids.astype(np.float32)
    x += [np.nextafter(f32, np.float32(np.inf)), np.nextafter(f32, np.float32(-np.inf))]
    rng = np.random.default_rng(0)
    for s in (1e-3, 0.02, 1.0, 30.0):
        x.append(rng.standard_normal(20000) * s)
    x.append(np.array([464.0 - 2 ** -15, 447.9, 2.0 ** -10, 3 * 2.0 ** -11, 0.0]))
    x = np.concatenate([np.asarray(a, np.float64) for a in x]).astype(np.float32)
    return x[np.abs(x) <= 448.0]


def test_codec_matches_library_conversion():
    x = _inputs()
    ours = np.array([oracle.fp8_from_float(float(v)) for v in x], np.uint8)
    lib = _library_codes(x)
    bad = np.nonzero(ours != lib)[0]
    assert bad.size == 0, [(float(x[i]), int(ours[i]), int(lib[i])) for i in bad[:5]]


def test_codec_is_nearest_ties_to_even():
    t = _table()[:0x7F]
    codes = np.arange(0x7F)
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(0, 448, 3000), rng.uniform(0, 0.05, 3000),
                        (t[:-1] + t[1:]) / 2]).astype(np.float32)
    for v in x:
        d = np.abs(t - float(v))
        best = codes[d == d.min()]
        want = best[0] if best.size == 1 else best[best % 2 == 0][0]
        assert oracle.fp8_from_float(float(v)) == want, float(v)
        assert oracle.fp8_from_float(-float(v)) == (want | 0x80 if v != 0 else 0x80)


def test_saturates_beyond_largest():
    assert oracle.fp8_from_float(1000.0) == 0x7E
    assert oracle.fp8_from_float(-1e30) == 0xFE


def _f32_update_model(M, widx, wk, ridx, rw, v, alpha, beta):
    """Elementwise numpy model of the fp8 write: binary32 products and
    difference, the fused multiply-add evaluated in float64 (a product of two
    binary32 values is exact there) and rounded to binary32, then E4M3 by
    torch's conversion.  Read in float64."""
    T, d_v = v.shape
    out = np.zeros((T, d_v))
    tab = _table()
    for t in range(T):
        a, b = np.float32(alpha[t]), np.float32(beta[t])
        for j, f in enumerate(widx[t]):
            m = tab[M[f]].astype(np.float32)
            mt = (a * m).astype(np.float32)
            d = (v[t].astype(np.float32) - mt).astype(np.float32)
            g = np.float32(b * np.float32(wk[t, j]))
            u = (np.float64(g) * d.astype(np.float64) + mt.astype(np.float64)).astype(np.float32)
            M[f] = _library_codes(u)
        for j, g_ in enumerate(ridx[t]):
            out[t] += rw[t, j] * tab[M[g_]]
    return out


def _tiny_case(cfg=None):
    cfg = cfg or S.CONFIGS["tiny"]
    host = {k: S.host_block(cfg, k)[0, 0] for k in ("s1", "s2", "q1", "q2", "v", "alpha", "beta")}
    M0 = S.host_block(cfg, "M0")
    wi, _, wk = oracle.select(host["s1"], host["s2"], cfg.W)
    ri, _, rw = oracle.select(host["q1"], host["q2"], cfg.R)
    wk32 = wk.astype(np.float32).astype(np.float64)  # binary32 weights, as the contract needs
    return cfg, host, M0, wi, wk32, ri, rw


def test_fp8_scan_matches_numpy_model():
    cfg, host, M0, wi, wk, ri, rw = _tiny_case()
    M = oracle.state_init(M0, 1, oracle.FP8)[0, 0].copy()
    Mm = M.copy()
    out = oracle.scan(M, oracle.FP8, wi, wk, ri, rw, host["v"], host["alpha"], host["beta"])
    want = _f32_update_model(Mm, wi, wk, ri, rw, host["v"], host["alpha"], host["beta"])
    assert np.array_equal(M, Mm)
    assert np.abs(out - want).max() <= 1e-6
    assert np.array_equal(oracle.state_init(M0, 1, oracle.FP8)[0, 0], _library_codes(M0[0]))


def test_fp8_scan_invariants():
    cfg, host, M0, wi, wk, ri, rw = _tiny_case()
    M = oracle.state_init(M0, 1, oracle.FP8)[0, 0].copy()
    before = M.copy()
    oracle.scan(M, oracle.FP8, wi, wk, ri, rw, host["v"], host["alpha"], host["beta"])
    untouched = np.setdiff1d(np.arange(cfg.N), wi.ravel())
    assert np.array_equal(M[untouched], before[untouched])
    # alpha = 1, beta = 0 keeps every value (a -0 code may come back as +0:
    # fma(0, d, -0) is +0 when d > 0)
    M2 = before.copy()
    oracle.scan(M2, oracle.FP8, wi, wk, ri, rw, host["v"], np.ones(cfg.T, np.float32),
                np.zeros(cfg.T, np.float32))
    assert np.array_equal(oracle.fp8_codes_to_f32(M2), oracle.fp8_codes_to_f32(before))
    assert np.array_equal(M2[before != 0x80], before[before != 0x80])


def _library_table():
    """Value of every E4M3 code by torch's float8_e4m3fn decoding (a library
    routine), as float64."""
    import torch

    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _nearest_even_codes(u):
    """float64 values -> E4M3 codes by brute-force nearest search over the
    finite positive codes 0x00..0x7E (ties to the even code, magnitudes past
    448 to 0x7E), sign in bit 7."""
    pos = _library_table()[:0x7F]
    a = np.abs(np.asarray(u, np.float64))
    hi = np.clip(np.searchsorted(pos, a), 1, 0x7E)
    lo = hi - 1
    dl, dh = a - pos[lo], pos[hi] - a
    code = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= pos[0x7E], 0x7E, code)
    return (code | np.where(np.signbit(u), 0x80, 0)).astype(np.uint8)


def _plain_write_check(tab, pre, post, rows, k64, v, alpha, beta):
    """Compare one step's stored codes `post[rows]` with the plain definition
    applied to `pre`; return how many element writes differ (each must be a
    neighbouring code on the other side of a rounding boundary that the exact
    update lies within binary32 rounding distance of)."""
    m = tab[pre[rows]]
    mt = float(alpha) * m
    vt = np.asarray(v, np.float64)
    u = mt + float(beta) * np.asarray(k64, np.float64)[:, None] * (vt - mt)
    want = _nearest_even_codes(u)
    got = post[rows]
    boundary = 0
    for r, c in zip(*np.nonzero(tab[got] != tab[want])):
        g_, w_ = int(got[r, c]), int(want[r, c])
        assert (g_ & 0x80) == (w_ & 0x80) and abs((g_ & 0x7F) - (w_ & 0x7F)) == 1, (r, c, g_, w_)
        mid = (tab[g_] + tab[w_]) / 2
        # binary32 evaluation error of three rounded operations and an fma,
        # plus the binary32 weight: a few units in 2^-24 of the operands
        scale = max(abs(mt[r, c]), abs(vt[c]), abs(u[r, c]))
        assert abs(u[r, c] - mid) <= 2.0 ** -20 * scale, (r, c, u[r, c], mid)
        boundary += 1
    return boundary


def test_fp8_write_matches_plain_definition():
    """The fp8 write against the pages' formula evaluated plainly ("Meccanismo
    Core", item 3): Mt = alpha*M and Mt + beta*k*(v - Mt) in float64 from the
    stored codes, with the float64 softmax weights, rounded once to the
    nearest E4M3 value.  The oracle takes the update in binary32 (so the code
    is a function of binary32 inputs on every implementation); the two can
    only differ where the exact update lies within binary32 rounding distance
    of an E4M3 rounding boundary, and then by one code.  Checked step by step
    from the same pre-step state, on the tiny workload's distributions made
    wider and longer (2M element writes)."""
    cfg, host, M0, wi, wk32, ri, rw = _tiny_case(
        S.CONFIGS["tiny"].with_(d_v=64, T=1024, W=32, R=32, seed=7))
    _, _, wk64 = oracle.select(host["s1"], host["s2"], cfg.W)
    tab = _library_table()
    M = oracle.state_init(M0, 1, oracle.FP8)[0, 0].copy()
    writes = boundary = 0
    for t in range(cfg.T):
        pre = M.copy()
        out = oracle.scan(M, oracle.FP8, wi[t:t + 1], wk32[t:t + 1], ri[t:t + 1], rw[t:t + 1],
                          host["v"][t:t + 1], host["alpha"][t:t + 1], host["beta"][t:t + 1])
        boundary += _plain_write_check(tab, pre, M, wi[t], wk64[t], host["v"][t],
                                       host["alpha"][t], host["beta"][t])
        writes += cfg.W * cfg.d_v
        # untouched rows keep their codes; the read is the weighted sum of the
        # stored post-write codes
        mask = np.ones(cfg.N, bool)
        mask[wi[t]] = False
        assert np.array_equal(M[mask], pre[mask])
        ref = (rw[t][:, None] * tab[M[ri[t]]]).sum(0)
        assert np.abs(out[0] - ref).max() <= 1e-6
    assert boundary <= writes // 1000, boundary
    print(f"fp8 write: {boundary} of {writes} element writes next to an E4M3 rounding boundary")


def test_fp8_write_rounding_boundary_case():
    """A write whose exact value lies just above the midpoint 1.0625 of the
    codes for 1.0 and 1.125: with k = 0.5 + 2^-30, alpha = beta = 1, M = 1 and
    v = 1.125 the exact update is 1.0625 + 2^-33 (nearest code: 1.125), while
    the binary32 weight is 0.5 and the binary32 update is the midpoint itself
    (ties to the even code: 1.0).  The plain definition and the oracle differ
    there by one code, and nowhere else."""
    tab = _library_table()
    N, d_v = 8, 32
    M = np.full((N, d_v), 0x38, np.uint8)  # 1.0 everywhere
    k64 = np.array([[0.5 + 2.0 ** -30, 0.25]])
    v = np.full((1, d_v), 1.125, np.float32)
    # odd columns: row 2's exact update 1.1875 + 0.375*2^-30 is above the
    # midpoint of 1.125 and 1.25, and the binary32 tie goes to the even code
    # 1.25 as well, so they agree
    v[0, 1::2] = 1.375
    pre = M.copy()
    oracle.scan(M, oracle.FP8, np.array([[2, 5]], np.int32), k64, np.array([[2]], np.int32),
                np.ones((1, 1)), v, np.ones(1, np.float32), np.ones(1, np.float32))
    assert tab[M[2, 0]] == 1.0 and tab[_nearest_even_codes(np.array([1.0625 + 2.0 ** -33]))[0]] \
        == 1.125
    n = _plain_write_check(tab, pre, M, np.array([2, 5]), k64[0], v[0], 1.0, 1.0)
    assert n == d_v // 2  # the even columns of row 2


def test_nearest_even_codes_pins():
    tab = _library_table()
    assert _nearest_even_codes(np.array([1.0]))[0] == 0x38
    assert _nearest_even_codes(np.array([1.0625]))[0] == 0x38      # tie 1 | 1.125 -> even code
    assert _nearest_even_codes(np.array([1.1875]))[0] == 0x3A      # tie 1.125 | 1.25 -> even
    assert _nearest_even_codes(np.array([-448.0, 500.0]))[0] == 0xFE
    assert _nearest_even_codes(np.array([500.0]))[0] == 0x7E
    assert _nearest_even_codes(np.array([2.0 ** -10]))[0] == 0x00  # tie 0 | 2^-9 -> even
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(5000) * 3).astype(np.float32)
    assert np.array_equal(_nearest_even_codes(x.astype(np.float64)), _library_codes(x))
    assert np.all(np.abs(tab[_nearest_even_codes(x)] - x) <= np.abs(x) / 16 + 2.0 ** -10)
