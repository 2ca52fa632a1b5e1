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


def _tiny_case():
    cfg = S.CONFIGS["tiny"]
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
