"""Checks of the seeded input generator (sdm_inputs), which both the oracle
and the GPU path consume.  It is pinned to the published Philox4x32-10
known-answer vectors and to the statistics of the distributions it claims."""
import os

import numpy as np
import pytest
from scipy import stats

import sdm_inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        assert S.philox4x32_10(v[0:4], v[4:6]) == v[6:10]


def test_normal_statistics():
    cfg = S.CONFIGS["tiny"].with_(T=4096)
    z = S.host_block(cfg, "s1").reshape(-1).astype(np.float64)  # 262144 draws
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-3
    assert not np.any(np.signbit(z[z == 0]))


def test_uniform_statistics():
    cfg = S.CONFIGS["tiny"].with_(T=200000)
    a = S.host_block(cfg, "alpha").reshape(-1)
    b = S.host_block(cfg, "beta").reshape(-1)
    assert a.min() >= 0.9 and a.max() < 1.0
    assert b.min() >= 0.0 and b.max() < 1.0
    assert stats.kstest((a.astype(np.float64) - 0.9) / 0.1, "uniform").pvalue > 1e-3
    assert stats.kstest(b.astype(np.float64), "uniform").pvalue > 1e-3


def test_m0_scale():
    m = S.host_block(S.CONFIGS["small"], "M0", h0=1, nh=1, t0=0, nt=4096)
    assert abs(m.std() - 0.02) < 0.0005


def test_block_is_slice_of_whole():
    cfg = S.CONFIGS["small"].with_(B=2, H=3, T=20, n=32, d_v=8)
    for name in ("s1", "q2", "v", "alpha"):
        whole = S.host_block(cfg, name)
        part = S.host_block(cfg, name, 1, 1, 2, 1, 5, 9)
        np.testing.assert_array_equal(part, whole[1:2, 2:3, 5:14])
    whole = S.host_block(cfg, "M0")
    np.testing.assert_array_equal(S.host_block(cfg, "M0", h0=1, nh=2, t0=100, nt=33),
                                  whole[1:3, 100:133])


def test_streams_differ_and_are_seeded():
    cfg = S.CONFIGS["tiny"]
    a = S.host_block(cfg, "s1")
    assert np.array_equal(a, S.host_block(cfg, "s1"))
    assert not np.array_equal(a, S.host_block(cfg, "s2"))
    assert not np.array_equal(a, S.host_block(cfg.with_(seed=cfg.seed + 1), "s1"))


def test_mid_mixture_shares_component_across_heads():
    cfg = S.CONFIGS["mid"].with_(T=64)
    s = S.host_block(cfg, "s1", 0, 1, 0, 8).astype(np.float64)  # [1,8,64,1024]
    # s = g + 0.5 e: variance 1.25, covariance across heads 1.0
    assert abs(s.var() - 1.25) < 0.03
    c = np.mean(s[0, 0] * s[0, 1])
    assert abs(c - 1.0) < 0.03
    q = S.host_block(cfg, "q1", 0, 1, 0, 2).astype(np.float64)
    assert abs(np.mean(q[0, 0] * q[0, 1])) < 0.03


def test_planted_pattern():
    cfg = S.CONFIGS["long"].with_(T=2048, H=2)
    i_s, j_s = S.planted_slot(cfg)
    s1 = S.host_block(cfg, "s1", 0, 1, 0, 2, 990, 20)
    s2 = S.host_block(cfg, "s2", 0, 1, 0, 2, 1000, 1)
    assert np.all(s1[:, :, 10, i_s] == 16.0) and np.all(s2[:, :, 0, j_s] == 16.0)
    assert np.all(s1[:, :, :10, i_s] < 16.0)
    v = S.host_block(cfg, "v", 0, 1, 0, 2, 1000, 1)
    assert np.all(v[..., 0] == 1.0) and np.all(v[..., 1:] == 0.0)
    assert np.all(S.host_block(cfg, "alpha", 0, 1, 0, 2, 1000, 1) == 1.0)
    q1 = S.host_block(cfg, "q1", 0, 1, 0, 2, cfg.T - 1, 1)
    assert np.all(q1[..., i_s] == 16.0)


def test_projection_inputs_bf16_rounding_and_scale():
    """The projection inputs: float32 draws rounded once to bf16 to nearest
    even (against torch's conversion, ties included), seeded, with the
    weights scaled by 1/sqrt(d_model)."""
    import torch

    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130,
                     3.0e38, -0.0], np.float32)  # halfway cases round to the even neighbour
    want = torch.from_numpy(ties).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(S._bf16_bits_rne(ties), want)
    X1, W1 = S.projection_inputs(2, 5, 256, 3, 11, seed=9)
    X2, W2 = S.projection_inputs(2, 5, 256, 3, 11, seed=9)
    X3, _ = S.projection_inputs(2, 5, 256, 3, 11, seed=10)
    assert np.array_equal(X1, X2) and np.array_equal(W1, W2) and not np.array_equal(X1, X3)
    assert X1.shape == (2, 5, 256) and W1.shape == (3, 11, 256) and X1.dtype == np.uint16
    w = torch.from_numpy(W1.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(float(w.std()) * 16.0 - 1.0) < 0.05  # N(0, 1/256)
