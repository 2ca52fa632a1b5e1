"""Pins of the oracle's gated delta write and sparse read.

Source: page "Riepilogo Tecnico: Sparse Delta Memory (SDM)", section
"Meccanismo Core": item 3 (forget gate Mt[i] = alpha_t M[i], delta update
M[i] = Mt[i] + beta_t k_i (v_t - Mt[i]) on the selected write rows, other
rows unchanged) and item 4 (output = weighted sum of the selected read rows);
section "Stato Iniziale Appreso" (memory starts from a learned M0).

Each test pins the oracle to something other than its own code: invariants
the formulas imply, closed forms of the recurrence, exact scaling and
linearity properties, and an independent numpy model that selects by
brute force over all N sums.
"""
import numpy as np
import pytest

import oracle
import sdm_inputs as S

F32, BF16 = oracle.F32, oracle.BF16


def tiny_inputs(cfg=None):
    cfg = cfg or S.CONFIGS["tiny"]
    g = {k: S.host_block(cfg, k, 0, 1, 0, 1) for k in ("s1", "s2", "q1", "q2", "v", "alpha",
                                                        "beta")}
    g = {k: v[0, 0] for k, v in g.items()}
    g["M0"] = S.host_block(cfg, "M0")
    return cfg, g


def run_oracle(cfg, g, M=None, dtype=F32, cols=None):
    if M is None:
        M = oracle.state_init(g["M0"], 1, dtype)[0, 0].copy()
    r = oracle.run_memory(M, dtype, g["s1"], g["s2"], g["q1"], g["q2"], g["v"], g["alpha"],
                          g["beta"], cfg.W, cfg.R, cols=cols)
    return M, r


# ----------------------------------------------------------------- invariants

def test_untouched_rows_bitwise_unchanged_each_step():
    cfg, g = tiny_inputs()
    M = oracle.state_init(g["M0"], 1)[0, 0].copy()
    widx, _, wk = oracle.select(g["s1"], g["s2"], cfg.W)
    ridx, _, rw = oracle.select(g["q1"], g["q2"], cfg.R)
    for t in range(cfg.T):
        before = M.copy()
        oracle.scan(M, F32, widx[t:t + 1], wk[t:t + 1], ridx[t:t + 1], rw[t:t + 1],
                    g["v"][t:t + 1], g["alpha"][t:t + 1], g["beta"][t:t + 1])
        mask = np.ones(cfg.N, bool)
        mask[widx[t]] = False
        assert np.array_equal(before[mask].view(np.uint32), M[mask].view(np.uint32))
        # the selected rows move (beta*k > 0 and v differs from the row)
        assert not np.array_equal(before[widx[t]], M[widx[t]])


def test_alpha_one_beta_zero_leaves_memory():
    cfg, g = tiny_inputs()
    g["alpha"] = np.ones_like(g["alpha"])
    g["beta"] = np.zeros_like(g["beta"])
    M0 = oracle.state_init(g["M0"], 1)[0, 0]
    M, r = run_oracle(cfg, g)
    assert np.array_equal(M.view(np.uint32), M0.view(np.uint32))
    # and the read is then a fixed weighted sum of M0 rows
    exp = np.einsum("tj,tjc->tc", r["rw"], M0[r["ridx"]].astype(np.float64))
    np.testing.assert_allclose(r["out"], exp, rtol=0, atol=1e-7)


def _dominant_inputs(n, T, d_v, a_star, b_star, rng):
    """Halves where slot (a*, b*) is the unique best at every step."""
    s1 = rng.standard_normal((T, n)).astype(np.float32)
    s2 = rng.standard_normal((T, n)).astype(np.float32)
    s1[:, a_star] = 20.0
    s2[:, b_star] = 20.0
    return s1, s2


def test_closed_form_constant_gates():
    # W = R = 1, one slot chosen every step, constant alpha, beta, v:
    # m_t = a m_{t-1} + beta v with a = alpha (1 - beta), so
    # m_T = a^T m_0 + beta v (1 - a^T) / (1 - a).
    rng = np.random.default_rng(7)
    n, T, d_v = 16, 40, 8
    a_s, b_s = 3, 11
    s1, s2 = _dominant_inputs(n, T, d_v, a_s, b_s, rng)
    alpha, beta = np.float32(0.93), np.float32(0.3)
    v1 = rng.standard_normal(d_v).astype(np.float32)
    M0 = (0.02 * rng.standard_normal((1, n * n, d_v))).astype(np.float32)
    M = oracle.state_init(M0, 1)[0, 0].copy()
    r = oracle.run_memory(M, F32, s1, s2, s1, s2, np.tile(v1, (T, 1)),
                          np.full(T, alpha, np.float32), np.full(T, beta, np.float32), 1, 1)
    f = a_s * n + b_s
    assert np.all(r["widx"][:, 0] == f) and np.all(r["wk"] == 1.0)
    a = float(alpha) * (1.0 - float(beta))
    for t in (1, 7, T):
        mt = a ** t * M0[0, f].astype(np.float64) + float(beta) * v1 * (1 - a ** t) / (1 - a)
        if t == T:
            np.testing.assert_allclose(M[f], mt, rtol=0, atol=1e-6)
            np.testing.assert_allclose(r["out"][T - 1], mt, rtol=0, atol=1e-6)
        else:
            np.testing.assert_allclose(r["out"][t - 1], mt, rtol=0, atol=1e-6)


def test_beta_times_k_one_overwrites_row():
    rng = np.random.default_rng(8)
    n, T, d_v = 8, 5, 16
    s1, s2 = _dominant_inputs(n, T, d_v, 2, 5, rng)
    v = rng.standard_normal((T, d_v)).astype(np.float32)
    M0 = rng.standard_normal((1, n * n, d_v)).astype(np.float32)
    for dtype in (F32, BF16):
        M = oracle.state_init(M0, 1, dtype)[0, 0].copy()
        r = oracle.run_memory(M, dtype, s1, s2, s1, s2, v, rng.uniform(0.5, 1, T).astype(
            np.float32), np.ones(T, np.float32), 1, 1)
        row = M[2 * n + 5]
        if dtype == F32:
            assert np.array_equal(row, v[-1])
            assert np.array_equal(r["out"][-1], v[-1])
        else:
            exp = np.array([oracle.bf16_from_double(x) for x in v[-1].astype(np.float64)],
                           np.uint16)
            assert np.array_equal(row, exp)


def test_convexity_bound():
    cfg, g = tiny_inputs()
    M, r = run_oracle(cfg, g)
    lo = min(0.0, g["M0"].min(), g["v"].min())
    hi = max(0.0, g["M0"].max(), g["v"].max())
    assert M.min() >= lo and M.max() <= hi
    assert np.abs(r["out"]).max() <= max(abs(lo), abs(hi)) + 1e-6


def test_power_of_two_homogeneity_bitwise():
    cfg, g = tiny_inputs()
    M1, r1 = run_oracle(cfg, g)
    g2 = dict(g)
    g2["M0"] = g["M0"] * np.float32(2)
    g2["v"] = g["v"] * np.float32(2)
    M2, r2 = run_oracle(cfg, g2)
    assert np.array_equal((M1 * 2).view(np.uint32), M2.view(np.uint32))
    assert np.array_equal((r1["out"] * 2).view(np.uint32), r2["out"].view(np.uint32))


def test_superposition():
    cfg, g = tiny_inputs()
    _, r = run_oracle(cfg, g)
    ga, gb = dict(g), dict(g)
    ga["v"] = np.zeros_like(g["v"])
    gb["M0"] = np.zeros_like(g["M0"])
    Ma, ra = run_oracle(cfg, ga)
    Mb, rb = run_oracle(cfg, gb)
    M, _ = run_oracle(cfg, g)
    np.testing.assert_allclose(M, Ma.astype(np.float64) + Mb, rtol=0, atol=1e-6)
    np.testing.assert_allclose(r["out"], ra["out"].astype(np.float64) + rb["out"], rtol=0,
                               atol=1e-6)


def test_single_read_row_returns_row():
    cfg, g = tiny_inputs()
    cfg1 = cfg.with_(R=1)
    M = oracle.state_init(g["M0"], 1)[0, 0].copy()
    widx, _, wk = oracle.select(g["s1"], g["s2"], cfg.W)
    ridx, _, rw = oracle.select(g["q1"], g["q2"], 1)
    assert np.all(rw == 1.0)
    for t in range(0, cfg1.T, 17):
        o = oracle.scan(M, F32, widx[t:t + 1], wk[t:t + 1], ridx[t:t + 1], rw[t:t + 1],
                        g["v"][t:t + 1], g["alpha"][t:t + 1], g["beta"][t:t + 1])
        assert np.array_equal(o[0], M[ridx[t, 0]])


def test_read_sees_this_steps_write():
    # Read halves equal to the write halves: the read rows are the written
    # rows, and the read must return their values after the write.
    cfg, g = tiny_inputs()
    g["q1"], g["q2"] = g["s1"], g["s2"]
    M = oracle.state_init(g["M0"], 1)[0, 0].copy()
    widx, _, wk = oracle.select(g["s1"], g["s2"], cfg.W)
    for t in range(cfg.T):
        o = oracle.scan(M, F32, widx[t:t + 1], wk[t:t + 1], widx[t:t + 1], wk[t:t + 1],
                        g["v"][t:t + 1], g["alpha"][t:t + 1], g["beta"][t:t + 1])
        exp = (wk[t][:, None] * M[widx[t]].astype(np.float64)).sum(0)
        np.testing.assert_allclose(o[0], exp, rtol=0, atol=1e-7)


def test_chunked_equals_whole_bitwise():
    cfg, g = tiny_inputs()
    M1, r1 = run_oracle(cfg, g)
    M2 = oracle.state_init(g["M0"], 1)[0, 0].copy()
    outs = []
    for t0, t1 in ((0, 100), (100, 101), (101, cfg.T)):
        part = {k: (v[t0:t1] if k != "M0" else v) for k, v in g.items()}
        _, r = run_oracle(cfg, part, M=M2)
        outs.append(r["out"])
    assert np.array_equal(M1.view(np.uint32), M2.view(np.uint32))
    assert np.array_equal(r1["out"].view(np.uint32), np.concatenate(outs).view(np.uint32))


def test_column_range_equals_full():
    cfg, g = tiny_inputs()
    M1, r1 = run_oracle(cfg, g)
    M2, r2 = run_oracle(cfg, g, cols=(3, 11))
    assert np.array_equal(M1[:, 3:11], M2[:, 3:11])
    assert np.array_equal(r1["out"][:, 3:11], r2["out"][:, 3:11])


@pytest.mark.parametrize("dtype", [F32, BF16, oracle.FP8])
def test_decode_steps_equal_scan(dtype):
    cfg = S.CONFIGS["tiny"].with_(B=2, H=3, T=40)
    names = ("s1", "s2", "q1", "q2", "v", "alpha", "beta")
    g = {k: S.host_block(cfg, k) for k in names}
    M0 = S.host_block(cfg, "M0")
    Md = oracle.state_init(M0, cfg.B, dtype)
    outs = []
    for t in range(cfg.T):
        o, wi, ri = oracle.step_decode(Md, dtype, *(g[k][:, :, t] for k in names), cfg.W, cfg.R)
        outs.append(o)
    outd = np.stack(outs, axis=2)
    Ms = oracle.state_init(M0, cfg.B, dtype)
    for b in range(cfg.B):
        for h in range(cfg.H):
            r = oracle.run_memory(Ms[b, h], dtype, *(g[k][b, h] for k in names), cfg.W, cfg.R)
            assert np.array_equal(r["out"].view(np.uint32), outd[b, h].view(np.uint32))
    assert np.array_equal(Md, Ms)


# --------------------------------------------------------- bf16 rounding pins

def test_bf16_round_to_nearest_even():
    one = 1.0
    assert oracle.bf16_from_double(one) == 0x3F80
    assert oracle.bf16_from_double(1 + 2 ** -8) == 0x3F80          # tie -> even (down)
    assert oracle.bf16_from_double(1 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert oracle.bf16_from_double(1 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert oracle.bf16_from_double(-2.0) == 0xC000
    assert oracle.bf16_from_double(-0.0) == 0x8000
    assert oracle.bf16_from_double(3.0e38) == 0x7F62
    assert oracle.bf16_from_double(3.4e38) == 0x7F80                # overflow -> inf
    # binary32 inputs: agree with the textbook integer rounding of the bits
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    ref = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------ independent numpy model

def bf16_rne_f64(u):
    """float64 values -> the nearest bf16 values (ties to even), as float32.
    Integer rounding of the float64 bit pattern: bf16 keeps the sign, the
    exponent and the top 7 of the 52 fraction bits, so the low 45 bits are
    rounded away (a carry into the exponent is the correct round-up).  Valid
    for zero and for magnitudes in binary32's normal range, which the callers
    assert."""
    u = np.asarray(u, np.float64)
    a = np.abs(u)
    assert np.all((a == 0) | ((a >= 2.0 ** -126) & (a < 2.0 ** 128))), "outside the normal range"
    b = u.view(np.uint64)
    one = np.uint64(1)
    r = ((b + np.uint64((1 << 44) - 1) + ((b >> np.uint64(45)) & one)) >> np.uint64(45)) \
        << np.uint64(45)
    return r.view(np.float64).astype(np.float32)  # exact: 8 significant bits


def numpy_model(g, W, R, dtype=F32):
    """Whole sequence with brute-force global selection over all N sums and
    the update written elementwise; no code shared with the oracle.  bf16
    state: M0 and every stored row are rounded to bf16 (nearest even), the
    update itself is taken in float64 from the stored values."""
    n = g["s1"].shape[1]
    M = g["M0"][0].astype(np.float32).copy()
    if dtype == BF16:
        b = M.view(np.uint32).astype(np.uint64)
        M = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    T = g["s1"].shape[0]
    out = np.zeros((T, M.shape[1]), np.float32)
    f = np.arange(n * n)

    def sel(x1, x2, K):
        s = (x1[:, None] + x2[None, :]).astype(np.float32).reshape(-1)
        o = np.lexsort((f, -s))[:K]
        e = np.exp(s[o].astype(np.float64) - float(s[o[0]]))
        return o, e / e.sum()

    for t in range(T):
        wi, wk = sel(g["s1"][t], g["s2"][t], W)
        ri, rw = sel(g["q1"][t], g["q2"][t], R)
        m = M[wi].astype(np.float64)
        mt = float(g["alpha"][t]) * m
        u = mt + float(g["beta"][t]) * wk[:, None] * (g["v"][t].astype(np.float64) - mt)
        M[wi] = bf16_rne_f64(u) if dtype == BF16 else u.astype(np.float32)
        out[t] = (rw[:, None] * M[ri].astype(np.float64)).sum(0).astype(np.float32)
    return M, out


def test_numpy_model_tiny_config():
    cfg, g = tiny_inputs()
    M, r = run_oracle(cfg, g)
    g1 = dict(g)
    g1["M0"] = g["M0"]
    Mn, outn = numpy_model(g1, cfg.W, cfg.R)
    np.testing.assert_allclose(M, Mn, rtol=0, atol=2e-7)
    np.testing.assert_allclose(r["out"], outn, rtol=0, atol=2e-7)


def test_numpy_model_tiny_config_bf16():
    """bf16 state: the oracle's stored rows equal, bit for bit, an elementwise
    float64 update rounded once per store to bf16 by integer rounding of the
    float64 bits (the oracle rounds with frexp and nearbyint instead)."""
    cfg, g = tiny_inputs()
    M, r = run_oracle(cfg, g, dtype=BF16)
    Mn, outn = numpy_model(g, cfg.W, cfg.R, dtype=BF16)
    got = oracle.bf16_bits_to_f32(M)
    assert np.array_equal(got.view(np.uint32), Mn.view(np.uint32))
    np.testing.assert_allclose(r["out"], outn, rtol=0, atol=2e-7)
    # the rows really were rewritten (and rounded) many times
    assert np.count_nonzero(got != oracle.bf16_bits_to_f32(
        oracle.state_init(g["M0"], 1, BF16)[0, 0])) > 1000


def test_bf16_rne_f64_pins():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -2.0,
                  1 + 255 * 2 ** -8 + 2 ** -9, 0.0, 3.0e38])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -2.0, 2.0, 0.0, 3.0e38], np.float64)
    want[-1] = float(np.float32(np.uint32(0x7F620000).view(np.float32)))
    got = bf16_rne_f64(x)
    assert np.array_equal(got.astype(np.float64), want), got
    # agrees with the oracle's rounding on random float64 values
    rng = np.random.default_rng(5)
    y = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    ref = np.array([oracle.bf16_from_double(float(v)) for v in y], np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f32(ref).view(np.uint32),
                          bf16_rne_f64(y).view(np.uint32))


def test_rejects_repeated_write_row():
    M = np.zeros((16, 4), np.float32)
    widx = np.array([[3, 3]], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.scan(M, F32, widx, np.full((1, 2), 0.5), widx, np.full((1, 2), 0.5),
                    np.zeros((1, 4), np.float32), np.ones(1, np.float32), np.ones(1, np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.scan(M, F32, np.array([[16]], np.int32), np.ones((1, 1)),
                    np.array([[0]], np.int32), np.ones((1, 1)), np.zeros((1, 4), np.float32),
                    np.ones(1, np.float32), np.ones(1, np.float32))
