"""Pins of the oracle's token projections (page "Riepilogo Tecnico: Sparse
Delta Memory (SDM)", "Meccanismo Core" item 2: projected keys and queries
split in two halves; "Design IsoFLOP": projections sized like the
baseline's) and of its gate function: exact cases (integer inputs, unit
weight rows that pick one input), an independent float64 matmul (numpy) of
the decoded bf16 arrays, the absolute-value sums, torch's bf16 decoding,
and the logistic function's closed forms."""
import math

import numpy as np
import torch

import oracle


def _bf16_bits(a):
    """float32 values -> bf16 bits by torch's conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _decode(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


def test_integer_inputs_are_exact():
    rng = np.random.default_rng(1)
    M, d, H, P = 7, 96, 3, 11
    X = rng.integers(-8, 9, (M, d)).astype(np.float32)
    Wt = rng.integers(-8, 9, (H, P, d)).astype(np.float32)
    y, ya = oracle.project(_bf16_bits(X), _bf16_bits(Wt), H)
    want = np.einsum("md,hpd->mhp", X.astype(np.int64), Wt.astype(np.int64))
    assert np.array_equal(y, want.astype(np.float64))
    assert np.array_equal(ya, np.einsum("md,hpd->mhp", np.abs(X).astype(np.int64),
                                        np.abs(Wt).astype(np.int64)).astype(np.float64))


def test_unit_weight_rows_pick_one_input():
    rng = np.random.default_rng(2)
    M, d, H, P = 5, 64, 2, 40
    Xb = _bf16_bits(rng.standard_normal((M, d)))
    Wt = np.zeros((H, P, d), np.float32)
    for h in range(H):
        for p in range(P):
            Wt[h, p, (h * P + p) % d] = 1.0
    y, _ = oracle.project(Xb, _bf16_bits(Wt), H)
    x = _decode(Xb)
    for h in range(H):
        for p in range(P):
            assert np.array_equal(y[:, h, p], x[:, (h * P + p) % d])


def test_matches_float64_matmul_of_the_decoded_arrays():
    rng = np.random.default_rng(3)
    M, d, H, P = 33, 256, 2, 70
    Xb = _bf16_bits(rng.standard_normal((M, d)))
    Wb = _bf16_bits(rng.standard_normal((H, P, d)) * 0.05)
    y, ya = oracle.project(Xb, Wb, H, threads=4)
    x, w = _decode(Xb), _decode(Wb)
    ref = np.einsum("md,hpd->mhp", x, w)
    refabs = np.einsum("md,hpd->mhp", np.abs(x), np.abs(w))
    assert np.abs(y - ref).max() <= 1e-12 * refabs.max()
    assert np.abs(ya - refabs).max() <= 1e-12 * refabs.max()
    assert np.all(ya >= np.abs(y))


def test_bf16_decoding_matches_torch():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]  # finite values only
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(got, _decode(bits))


def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(float(oracle.sigmoid(math.log(3.0))) - 0.75) <= 1e-15
    y = np.linspace(-30, 30, 121)
    s = oracle.sigmoid(y)
    assert np.all(np.diff(s) > 0) and np.all((s > 0) & (s < 1))
    assert np.abs(s + oracle.sigmoid(-y) - 1.0).max() <= 1e-15
