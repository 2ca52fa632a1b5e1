"""Shared helpers of the GPU parity tests: seeded inputs on both sides, the
HIP path through the C ABI, the oracle, and the comparison bars."""
import numpy as np

import oracle
import sdm_inputs as S

# Bars.  Indices: bit-exact.  fp32 state: elementwise max-abs 1e-5.  bf16
# state: normwise per (b,h) slice, max|x - y| <= 2e-2 * max|y|.  Weights: the
# GPU uses binary32 expf and sums, the oracle double; both are within a few
# ulps of the exact softmax, so 1e-6 absolute is ample.
FP32_ATOL = 1e-5
BF16_REL = 2e-2
WEIGHT_ATOL = 1e-6

NAMES = ("s1", "s2", "q1", "q2", "v", "alpha", "beta")


def host_inputs(cfg, b0=0, nb=None, h0=0, nh=None, t0=0, nt=None):
    nb = cfg.B - b0 if nb is None else nb
    nh = cfg.H - h0 if nh is None else nh
    nt = cfg.T - t0 if nt is None else nt
    return {k: S.host_block(cfg, k, b0, nb, h0, nh, t0, nt) for k in NAMES}


def to_dev(d):
    import torch

    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}


def gpu_sequence(cfg, dev, M):
    """Selections and scan on the GPU for the whole [B,H,T] block in `dev`."""
    import sparse_memory_linear_sdm_amd as sdm

    widx, wsc, wk = sdm.select(dev["s1"], dev["s2"], cfg.W)
    ridx, rsc, rw = sdm.select(dev["q1"], dev["q2"], cfg.R)
    out = sdm.scan(M, widx, wk, ridx, rw, dev["v"], dev["alpha"], dev["beta"])
    return {"widx": widx, "wscore": wsc, "wk": wk, "ridx": ridx, "rscore": rsc, "rw": rw,
            "out": out}


def oracle_memory(cfg, host, b, h, M0h, dtype, cols=None, threads=1):
    """Oracle run of memory (b,h) (indices into the host block)."""
    M = oracle.state_init(M0h[None], 1, dtype)[0, 0].copy()
    r = oracle.run_memory(M, dtype, *(host[k][b, h] for k in NAMES), cfg.W, cfg.R, cols=cols,
                          threads=threads)
    r["M"] = M
    return r


def as_f32(M_np_or_bits, dtype):
    if dtype == oracle.BF16:
        return oracle.bf16_bits_to_f32(M_np_or_bits)
    return M_np_or_bits


def state_to_host(Mslice):
    """Device state slice -> numpy (float32 or uint16 bf16 bits)."""
    import torch

    if Mslice.dtype == torch.bfloat16:
        return Mslice.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return Mslice.contiguous().cpu().numpy()


def check_selection(g_idx, g_score, g_w, o_idx, o_score, o_w, what=""):
    assert np.array_equal(g_idx, o_idx), f"{what}: index mismatch at " \
        f"{np.argwhere(g_idx != o_idx)[:5].tolist()}"
    assert np.array_equal(g_score, o_score), f"{what}: score mismatch"
    err = np.abs(g_w.astype(np.float64) - o_w).max() if g_w.size else 0.0
    assert err <= WEIGHT_ATOL, f"{what}: weight error {err}"


def check_values(g, o, dtype, what=""):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if dtype == oracle.F32:
        err = np.abs(g - o).max() if g.size else 0.0
        assert err <= FP32_ATOL, f"{what}: max-abs error {err}"
        return err
    scale = np.abs(o).max()
    err = np.abs(g - o).max() if g.size else 0.0
    assert err <= BF16_REL * scale, f"{what}: normwise error {err} vs scale {scale}"
    return err / max(scale, 1e-30)
