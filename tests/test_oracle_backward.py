"""Pins of the oracle's backward pass (gradients of the write and read of
"Meccanismo Core" items 3-4 and of the selection weights, selections fixed).

The oracle is checked against things other than itself:
  * central finite differences of an independent float64 forward written
    here elementwise (no rounding to fp32 anywhere);
  * the adjoint identity of the part that is linear in (M0, v), against the
    oracle's own forward scan (a separate function);
  * closed forms for alpha = 1, beta = 0 and for a single untouched row;
  * the tape (pre-write rows) and the read rows against step-by-step
    forward runs and the forward's outputs;
  * the softmax-through-halves gradient against finite differences.
"""
import numpy as np
import pytest

import oracle


def _case(rng, N=8, d_v=3, T=6, W=3, R=2, reuse=True):
    """Random selections (distinct rows per step) with heavy row reuse, weights
    summing to one, gates in the workload ranges."""
    widx = np.stack([rng.choice(N, W, replace=False) for _ in range(T)]).astype(np.int32)
    ridx = np.stack([rng.choice(N, R, replace=False) for _ in range(T)]).astype(np.int32)
    if reuse and T > 1 and R > 0 and widx[1, 0] not in ridx[1]:
        ridx[1, 0] = widx[1, 0]  # a read of a row written in the same step
    wk = rng.random((T, W)) + 0.1
    wk /= wk.sum(1, keepdims=True)
    rw = rng.random((T, R)) + 0.1
    rw /= rw.sum(1, keepdims=True)
    return dict(
        M0=(0.5 * rng.standard_normal((N, d_v))).astype(np.float32),
        widx=widx, wk=wk, ridx=ridx, rw=rw,
        v=rng.standard_normal((T, d_v)).astype(np.float32),
        alpha=rng.uniform(0.9, 1.0, T).astype(np.float32),
        beta=rng.uniform(0.0, 1.0, T).astype(np.float32),
    )


def _fwd64(M0, widx, wk, ridx, rw, v, alpha, beta):
    """Independent float64 forward: elementwise loops, no rounding."""
    M = np.array(M0, np.float64)
    T, d_v = v.shape
    out = np.zeros((T, d_v))
    for t in range(T):
        for j, f in enumerate(widx[t]):
            for c in range(d_v):
                mt = alpha[t] * M[f, c]
                M[f, c] = mt + beta[t] * wk[t, j] * (v[t, c] - mt)
        for j, g in enumerate(ridx[t]):
            out[t] += rw[t, j] * M[g]
    return out, M


def _loss(case, dout, dMT, **over):
    c = {k: np.array(v, np.float64) if k not in ("widx", "ridx") else v for k, v in case.items()}
    c.update(over)
    out, MT = _fwd64(c["M0"], c["widx"], c["wk"], c["ridx"], c["rw"], c["v"], c["alpha"],
                     c["beta"])
    return float((dout * out).sum() + (dMT * MT).sum())


def _bwd(case, dout, dMT):
    return oracle.scan_backward(case["M0"], case["widx"], case["wk"], case["ridx"], case["rw"],
                                case["v"], case["alpha"], case["beta"], dout, dMT)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_finite_differences(seed):
    rng = np.random.default_rng(seed)
    case = _case(rng)
    T, d_v = case["v"].shape
    N = case["M0"].shape[0]
    dout = rng.standard_normal((T, d_v)).astype(np.float32)
    dMT = rng.standard_normal((N, d_v))
    g = _bwd(case, dout, dMT)
    h = 1e-6
    # every parameter entry of the small case
    for name, grad in (("v", g["dv"]), ("alpha", g["dalpha"]), ("beta", g["dbeta"]),
                       ("wk", g["dwk"]), ("rw", g["drw"]), ("M0", g["dM0"])):
        base = np.array(case[name], np.float64)
        num = np.zeros_like(base)
        for pos in np.ndindex(base.shape):
            xp, xm = base.copy(), base.copy()
            xp[pos] += h
            xm[pos] -= h
            num[pos] = (_loss(case, dout, dMT, **{name: xp}) -
                        _loss(case, dout, dMT, **{name: xm})) / (2 * h)
        scale = max(1.0, float(np.abs(num).max()))
        assert np.abs(grad - num).max() <= 2e-6 * scale, name


def test_adjoint_identity_linear_part():
    """For fixed selections and gates the step is linear in (M0, v), so
    <dout, o> + <dMT, MT> = <dM0, M0> + <dv, v> (here the forward is the
    oracle's fp32 scan, so the two sides agree to fp32 rounding)."""
    rng = np.random.default_rng(7)
    case = _case(rng, N=64, d_v=8, T=40, W=6, R=5)
    T, d_v = case["v"].shape
    N = case["M0"].shape[0]
    dout = rng.standard_normal((T, d_v)).astype(np.float32)
    dMT = rng.standard_normal((N, d_v))
    g = _bwd(case, dout, dMT)
    M = case["M0"].copy()
    out = oracle.scan(M, oracle.F32, case["widx"], case["wk"], case["ridx"], case["rw"],
                      case["v"], case["alpha"], case["beta"])
    lhs = float((dout.astype(np.float64) * out).sum() + (dMT * M).sum())
    rhs = float((g["dM0"] * case["M0"]).sum() + (g["dv"] * case["v"]).sum())
    assert abs(lhs - rhs) <= 1e-5 * max(1.0, abs(lhs))
    assert np.array_equal(g["MT"], M)  # the backward's replay is the forward


def test_alpha_one_beta_zero_closed_form():
    """alpha = 1, beta = 0: the write is the identity, so the state gradient is
    the final gradient plus every read's r_j * do_t at its row, dv = 0, and
    dalpha_t = sum_j <G_t[f_j], M[f_j]> with M = M0 throughout."""
    rng = np.random.default_rng(3)
    case = _case(rng, N=16, d_v=4, T=10, W=3, R=3)
    T, d_v = case["v"].shape
    case["alpha"][:] = 1.0
    case["beta"][:] = 0.0
    dout = rng.standard_normal((T, d_v)).astype(np.float32)
    dMT = rng.standard_normal((16, d_v))
    g = _bwd(case, dout, dMT)
    want = dMT.copy()
    Gt = [None] * T
    for t in range(T - 1, -1, -1):
        for j, r in enumerate(case["ridx"][t]):
            want[r] += case["rw"][t, j] * dout[t]
        Gt[t] = want.copy()
    assert np.allclose(g["dM0"], want, rtol=0, atol=1e-12)
    assert np.all(g["dv"] == 0.0)
    assert np.all(g["dwk"] == 0.0)  # dk = beta * d(beta k) = 0
    for t in range(T):
        da = sum(float(Gt[t][f] @ case["M0"][f].astype(np.float64)) for f in case["widx"][t])
        assert abs(g["dalpha"][t] - da) <= 1e-12 * max(1.0, abs(da))
    # dbeta_t = sum_j k_j <G_t[f_j], v_t - M0[f_j]>
    for t in range(T):
        db = sum(case["wk"][t, j] * float(Gt[t][f] @ (case["v"][t].astype(np.float64) -
                                                      case["M0"][f].astype(np.float64)))
                 for j, f in enumerate(case["widx"][t]))
        assert abs(g["dbeta"][t] - db) <= 1e-12 * max(1.0, abs(db))


def test_overwrite_cuts_the_gradient():
    """beta * k = 1 overwrites a row with v: the row's carried gradient is
    zero (alpha * (1 - beta k) = 0) and all of it goes to v."""
    rng = np.random.default_rng(4)
    case = _case(rng, N=8, d_v=3, T=3, W=1, R=1, reuse=False)
    case["wk"][:] = 1.0
    case["beta"][:] = 1.0
    case["widx"][:, 0] = 5
    case["ridx"][:, 0] = 2
    dMT = np.zeros((8, 3))
    dMT[5] = [1.0, -2.0, 0.5]
    dout = np.zeros((3, 3), np.float32)
    g = _bwd(case, dout, dMT)
    assert np.all(g["dM0"][5] == 0.0)
    assert np.array_equal(g["dv"][2], dMT[5])
    assert np.all(g["dv"][:2] == 0.0)


def test_untouched_row_passes_gradient_through():
    rng = np.random.default_rng(5)
    case = _case(rng, N=32, d_v=4, T=8, W=3, R=3)
    used = set(case["widx"].ravel()) | set(case["ridx"].ravel())
    free = [i for i in range(32) if i not in used]
    assert free
    dMT = rng.standard_normal((32, 4))
    g = _bwd(case, np.zeros((8, 4), np.float32), dMT)
    assert np.array_equal(g["dM0"][free], dMT[free])


def test_tape_holds_pre_write_rows():
    rng = np.random.default_rng(6)
    case = _case(rng, N=16, d_v=5, T=12, W=4, R=3)
    g = _bwd(case, np.zeros((12, 5), np.float32), None)
    M = case["M0"].copy()
    for t in range(12):
        assert np.array_equal(g["tape"][t], M[case["widx"][t]])
        oracle.scan(M, oracle.F32, case["widx"][t:t + 1], case["wk"][t:t + 1],
                    case["ridx"][t:t + 1], case["rw"][t:t + 1], case["v"][t:t + 1],
                    case["alpha"][t:t + 1], case["beta"][t:t + 1])
    assert np.array_equal(g["MT"], M)


def test_read_rows_are_what_each_read_saw():
    """rtape[t, j] is row ridx[t, j] of the memory after step t's write: equal
    to a step-by-step run of the forward oracle, and its rw-weighted sum is
    that forward's output (the read of "Meccanismo Core" item 4)."""
    rng = np.random.default_rng(9)
    T, d_v = 14, 6
    case = _case(rng, N=12, d_v=d_v, T=T, W=4, R=5)
    g = _bwd(case, np.zeros((T, d_v), np.float32), None)
    M = case["M0"].copy()
    outs = []
    for t in range(T):
        outs.append(oracle.scan(M, oracle.F32, case["widx"][t:t + 1], case["wk"][t:t + 1],
                                case["ridx"][t:t + 1], case["rw"][t:t + 1], case["v"][t:t + 1],
                                case["alpha"][t:t + 1], case["beta"][t:t + 1])[0])
        assert np.array_equal(g["rtape"][t], M[case["ridx"][t]])
    weighted = np.einsum("tj,tjc->tc", case["rw"], g["rtape"].astype(np.float64))
    outs = np.array(outs, np.float64)  # binary32 outputs: one rounding each
    assert np.all(np.abs(weighted - outs) <= 2.0 ** -23 * np.abs(outs))


def test_backward_rejects_repeated_read_rows():
    rng = np.random.default_rng(8)
    case = _case(rng, N=16, d_v=2, T=2, W=2, R=2, reuse=False)
    case["ridx"][1] = [3, 3]
    with pytest.raises(oracle.OracleError):
        _bwd(case, np.zeros((2, 2), np.float32), None)


def _weights_of(x1, x2, idx, n):
    s = x1[idx // n] + x2[idx % n]
    e = np.exp(s - s.max())
    return e / e.sum()


@pytest.mark.parametrize("n,K", [(4, 3), (8, 5), (16, 16)])
def test_select_backward_finite_differences(n, K):
    rng = np.random.default_rng(n * 31 + K)
    x1 = rng.standard_normal(n)
    x2 = rng.standard_normal(n)
    idx, _, w = oracle.select(x1.astype(np.float32), x2.astype(np.float32), K)
    dw = rng.standard_normal(K)
    dx1, dx2 = oracle.select_backward(idx, w, dw, n)
    h = 1e-6
    for which, x, d in ((0, x1, dx1), (1, x2, dx2)):
        for i in range(n):
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            a = (xp, x2) if which == 0 else (x1, xp)
            b = (xm, x2) if which == 0 else (x1, xm)
            num = (dw @ _weights_of(*a, idx, n) - dw @ _weights_of(*b, idx, n)) / (2 * h)
            assert abs(d[i] - num) <= 1e-7, (which, i)
    # softmax gradients sum to zero, and every selected pair feeds both halves
    assert abs(dx1.sum()) <= 1e-12 and abs(dx2.sum()) <= 1e-12
    unused1 = np.setdiff1d(np.arange(n), idx // n)
    assert np.all(dx1[unused1] == 0.0)


def test_select_backward_k1_is_zero():
    """One selected slot has weight exactly 1 whatever the scores."""
    x1 = np.array([0.3, -1.0, 2.0, 0.1], np.float32)
    x2 = np.array([1.0, 0.2, -0.5, 0.0], np.float32)
    idx, _, w = oracle.select(x1, x2, 1)
    dx1, dx2 = oracle.select_backward(idx, w, np.array([3.5]), 4)
    assert np.all(dx1 == 0.0) and np.all(dx2 == 0.0)


def test_state_init_backward_sums_sequences():
    rng = np.random.default_rng(9)
    dM = rng.standard_normal((3, 2, 5, 4)).astype(np.float32)
    got = oracle.state_init_backward(dM)
    assert np.array_equal(oracle.state_init_backward(dM[:1]), dM[0].astype(np.float64))
    assert np.allclose(got, dM.astype(np.float64).sum(0), rtol=0, atol=1e-12)


def test_chunked_backward_equals_whole():
    """Training a sequence in two chunks -- the second chunk's reverse pass
    starting from the final gradient, the first's from the gradient the second
    returns, each from its own starting state -- gives the whole-sequence
    gradients (the reverse recurrence carries only G between steps)."""
    rng = np.random.default_rng(11)
    case = _case(rng, N=32, d_v=6, T=30, W=4, R=3)
    T, d_v = case["v"].shape
    dout = rng.standard_normal((T, d_v)).astype(np.float32)
    dMT = rng.standard_normal((32, d_v))
    whole = _bwd(case, dout, dMT)
    T1 = 13
    first = {k: (v[:T1] if k not in ("M0",) else v) for k, v in case.items()}
    M1 = case["M0"].copy()
    oracle.scan(M1, oracle.F32, case["widx"][:T1], case["wk"][:T1], case["ridx"][:T1],
                case["rw"][:T1], case["v"][:T1], case["alpha"][:T1], case["beta"][:T1])
    second = {k: (v[T1:] if k not in ("M0",) else M1) for k, v in case.items()}
    g2 = _bwd(second, dout[T1:], dMT)
    g1 = _bwd(first, dout[:T1], g2["dM0"])
    assert np.allclose(g1["dM0"], whole["dM0"], rtol=0, atol=1e-12)
    for k in ("dv", "dwk", "drw", "dalpha", "dbeta"):
        assert np.allclose(np.concatenate([g1[k], g2[k]]), whole[k], rtol=0, atol=1e-12), k
