"""GPU parity of the token projections (sdm_project) against the oracle's
float64 dot products, and of the selections run on the projected scores.

Bar: each projected value is a binary32 sum of d_model exact bf16 products
(a bf16 x bf16 product has at most 16 significant bits, so it is exact in
binary32), so whatever the summation order the matrix cores use, its error
is at most (d_model - 1) * u * sum |x_i w_i| with u the unit roundoff of one
binary32 addition.  The test takes u = 2^-23, which also covers additions
rounded toward zero inside the matrix unit.  The gates go through the
logistic function, whose slope is at most 1/4, plus a few ulps of binary32
expf and division: |alpha - sigma(y)| <= bound/4 + 2^-21."""
import numpy as np
import pytest

import oracle
import sdm_inputs as S

pytestmark = pytest.mark.gpu

U = 2.0 ** -23
GATE_ATOL = 2.0 ** -21


def _run(B, T, d_model, H, n, d_v, seed):
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    P = 4 * n + d_v + 2
    Xb, Wb = S.projection_inputs(B, T, d_model, H, P, seed=seed)
    X = torch.from_numpy(Xb.view(np.int16)).cuda().view(torch.bfloat16)
    Wt = torch.from_numpy(Wb.view(np.int16)).cuda().view(torch.bfloat16)
    outs = sdm.project(X, Wt, n)
    torch.cuda.synchronize()
    return Xb, Wb, [o.cpu().numpy() for o in outs], outs


def _check(Xb, Wb, got, B, T, H, n, d_v, tokens=None, threads=8):
    """Compare the GPU outputs with the oracle on every token (or the listed
    flat tokens m = b*T + t)."""
    d_model = Xb.shape[-1]
    X = Xb.reshape(B * T, d_model)
    toks = np.arange(B * T) if tokens is None else np.asarray(tokens)
    y, ya = oracle.project(X[toks], Wb, H, threads=threads)  # [m, H, P]
    bound = (d_model - 1) * U * ya
    b_of, t_of = toks // T, toks % T
    s1, s2, q1, q2, v, alpha, beta = got
    parts = [(s1, 0, n), (s2, n, n), (q1, 2 * n, n), (q2, 3 * n, n), (v, 4 * n, d_v)]
    worst = 0.0
    for arr, off, width in parts:
        g = arr[b_of, :, t_of, :].astype(np.float64)  # [m, H, width]
        want = y[:, :, off:off + width]
        err = np.abs(g - want)
        lim = bound[:, :, off:off + width]
        assert np.all(err <= lim), (
            f"projection columns {off}..{off + width}: max excess "
            f"{np.max(err - lim):.3e} at {np.unravel_index(np.argmax(err - lim), err.shape)}")
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(lim > 0, err / lim, 0.0)
        worst = max(worst, float(np.max(r)) if r.size else 0.0)
    for arr, col in ((alpha, 4 * n + d_v), (beta, 4 * n + d_v + 1)):
        g = arr[b_of, :, t_of].astype(np.float64)
        want = oracle.sigmoid(y[:, :, col])
        lim = bound[:, :, col] / 4 + GATE_ATOL
        assert np.all(np.abs(g - want) <= lim), f"gate column {col}"
    return worst


@pytest.mark.parametrize("B,T,d_model,H,n,d_v", [
    (2, 150, 320, 3, 64, 16),    # 3 row tiles (ragged), 7 column tiles (ragged), 5 k steps
    (1, 129, 64, 1, 1, 1),       # P = 7: one partial column tile; one k step
    (3, 64, 128, 2, 37, 32),     # odd n: parts cross tile edges mid-row
    (1, 300, 512, 2, 256, 64),   # several full column tiles per head
    (300, 1, 128, 1, 8, 16),     # T = 1: every row of a tile is another sequence
    (37, 3, 64, 2, 16, 16),      # T = 3: sequences change inside each lane's rows
    (2, 700, 1024, 1, 128, 128), # row tiles of 256 with a ragged last one; 16 k stages
])
def test_project_parity(B, T, d_model, H, n, d_v):
    Xb, Wb, got, _ = _run(B, T, d_model, H, n, d_v, seed=B * 1000 + T + n)
    worst = _check(Xb, Wb, got, B, T, H, n, d_v)
    print(f"worst |err| / bound = {worst:.3e}")


def test_project_integer_inputs_exact():
    # Small integers: every partial sum is an integer below 2^24, so every
    # summation order gives the exact value.
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    B, T, d_model, H, n, d_v = 2, 70, 192, 2, 16, 16
    P = 4 * n + d_v + 2
    rng = np.random.default_rng(5)
    X = rng.integers(-8, 9, (B, T, d_model)).astype(np.float32)
    W = rng.integers(-8, 9, (H, P, d_model)).astype(np.float32)
    Xt = torch.from_numpy(X).to(torch.bfloat16).cuda()
    Wt = torch.from_numpy(W).to(torch.bfloat16).cuda()
    s1, s2, q1, q2, v, _, _ = (o.cpu().numpy() for o in sdm.project(Xt, Wt, n))
    y = np.einsum("btd,hpd->bhtp", X.astype(np.int64), W.astype(np.int64))
    assert np.array_equal(s1, y[..., :n]) and np.array_equal(s2, y[..., n:2 * n])
    assert np.array_equal(q1, y[..., 2 * n:3 * n]) and np.array_equal(q2, y[..., 3 * n:4 * n])
    assert np.array_equal(v, y[..., 4 * n:4 * n + d_v])


def test_project_then_select_bit_exact():
    # The front end feeding the selection: the GPU selection of the projected
    # halves equals the oracle's selection of the same binary32 halves.
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    B, T, d_model, H, n, d_v, K = 2, 100, 256, 2, 128, 32, 32
    _, _, got, outs = _run(B, T, d_model, H, n, d_v, seed=77)
    for a, b in ((0, 1), (2, 3)):
        gi, gs, gw = sdm.select(outs[a], outs[b], K)
        torch.cuda.synchronize()
        oi, os_, ow = oracle.select(got[a], got[b], K, threads=8)
        assert np.array_equal(gi.cpu().numpy(), oi)
        assert np.array_equal(gs.cpu().numpy(), os_)
        assert np.max(np.abs(gw.cpu().numpy() - ow)) <= 1e-6


def test_project_empty_and_errors():
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    X = torch.empty((0, 5, 64), dtype=torch.bfloat16, device="cuda")
    Wt = torch.zeros((1, 4 * 2 + 4 + 2, 64), dtype=torch.bfloat16, device="cuda")
    outs = sdm.project(X, Wt, 2)
    assert outs[0].shape == (0, 1, 5, 2)
    X = torch.zeros((1, 5, 96), dtype=torch.bfloat16, device="cuda")
    Wt = torch.zeros((1, 14, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdm.SDMError, match="multiple of 64"):
        sdm.project(X, Wt, 2)


@pytest.mark.slow
def test_project_front_full_size_sampled():
    """The front end at the mid workload's size (B=8, T=4096, H=8, n=1024,
    d_v=128, d_model = 2nH = 16384), in the launch the bench times: sampled
    tokens (first, last, both ends of a row tile and of a sequence) against
    the oracle on every head and every column."""
    B, T, d_model, H, n, d_v = 8, 4096, 16384, 8, 1024, 128
    Xb, Wb, got, _ = _run(B, T, d_model, H, n, d_v, seed=2024)
    toks = [0, 1, 255, 256, T - 1, T, 5 * T + 777, B * T - 257, B * T - 1]
    worst = _check(Xb, Wb, got, B, T, H, n, d_v, tokens=toks, threads=16)
    print(f"worst |err| / bound = {worst:.3e}")
