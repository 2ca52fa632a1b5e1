"""GPU parity of the planned scan (sdm_scan_plan + sdm_scan_planned) against
the oracle's scan, and against sdm_scan.

Inputs are index lists built directly (the scan takes any rows: selected
ones, repeated ones across steps, rows outside [0, N)), so the cases can
force what the planned path handles specially: read-after-write hazards
inside the prefetch window (rows drawn from a small pool), lists longer
than the fast path's capacity (every row in one shard), skipped rows, and
the 1-, 2- and 4-shard launches (the shard count follows B*H and d_v).

Bars: M and out within FP32_ATOL of the oracle; M equal to sdm_scan's bit
for bit (the same fp32 update); out deterministic and equal across splits
of the sequence into calls."""
import numpy as np
import pytest

import oracle
import sdm_inputs as S
from gpu_util import FP32_ATOL, check_values

pytestmark = pytest.mark.gpu

F32 = oracle.F32


def _shard(rows, S):
    """Row shard of each row for S shards (the multiplicative hash the
    planned scan splits rows with); used only to build inputs that crowd
    one shard."""
    if S == 1:
        return np.zeros(rows.shape, np.int64)
    bits = S.bit_length() - 1
    return (((rows.astype(np.uint64) * 0xC2B2AE35) & 0xFFFFFFFF) >> (32 - bits)).astype(np.int64)


def _inputs(B, H, N, d_v, T, W, R, seed, pool=None, rows_from=None, skipped=False):
    rng = np.random.default_rng(seed)
    cand = np.arange(N) if rows_from is None else np.asarray(rows_from)
    if pool is not None:
        cand = rng.choice(cand, size=pool, replace=False)
    # distinct write rows per step (repeated ones are unspecified); reads may repeat
    keys = rng.random((B, H, T, cand.size))
    widx = cand[np.argsort(keys, axis=-1)[..., :W]].astype(np.int32)
    ridx = cand[rng.integers(0, cand.size, (B, H, T, R))].astype(np.int32)
    if skipped:  # rows outside [0, N): no access, a skipped read adds 0
        widx[..., 0, 1] = -1
        widx[..., 1::5, 0] = N + 3
        ridx[..., 2::3, R - 1] = -7
        ridx[..., 0, 0] = N
    wk = rng.random((B, H, T, W)).astype(np.float32)
    rw = (rng.random((B, H, T, R)) / R).astype(np.float32)
    v = rng.standard_normal((B, H, T, d_v)).astype(np.float32)
    alpha = rng.uniform(0.85, 1.0, (B, H, T)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (B, H, T)).astype(np.float32)
    M0 = rng.standard_normal((B, H, N, d_v)).astype(np.float32)
    return dict(widx=widx, wk=wk, ridx=ridx, rw=rw, v=v, alpha=alpha, beta=beta, M0=M0)


def _dev(h):
    import torch

    return {k: torch.from_numpy(np.ascontiguousarray(x)).cuda() for k, x in h.items()}


def _planned(d, M, d_v, splits=None):
    """Planned scan of the whole sequence, in calls over `splits` (a list of
    step counts) or one call."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    T = d["v"].shape[2]
    N = M.shape[2]
    splits = [T] if splits is None else splits
    outs, t0 = [], 0
    for n in splits:
        sl = {k: d[k][:, :, t0:t0 + n].contiguous() for k in
              ("widx", "wk", "ridx", "rw", "v", "alpha", "beta")}
        ws = sdm.scan_plan(sl["widx"], sl["wk"], sl["ridx"], sl["rw"], N, d_v)
        outs.append(sdm.scan_planned(M, sl["v"], sl["alpha"], sl["beta"], ws))
        t0 += n
    torch.cuda.synchronize()
    return torch.cat(outs, dim=2)


def _oracle(h, b, hh):
    """Oracle run of memory (b, hh).  The oracle takes rows in [0, N) only;
    rows outside are mapped onto a table extended past N: an invalid write
    slot j writes sink row N + j, an invalid read slot reads row N + W,
    which nothing writes and stays zero (the skipped rows' semantics)."""
    N = h["M0"].shape[2]
    wi, ri = h["widx"][b, hh].copy(), h["ridx"][b, hh].copy()
    W = wi.shape[1]
    wbad, rbad = (wi < 0) | (wi >= N), (ri < 0) | (ri >= N)
    Mo = h["M0"][b, hh]
    if wbad.any() or rbad.any():
        wi[wbad] = (N + np.broadcast_to(np.arange(W, dtype=np.int32), wi.shape))[wbad]
        ri[rbad] = N + W
        Mo = np.concatenate([Mo, np.zeros((W + 1, Mo.shape[1]), np.float32)])
    Mo = np.ascontiguousarray(Mo).copy()
    out = oracle.scan(Mo, F32, wi, h["wk"][b, hh], ri, h["rw"][b, hh], h["v"][b, hh],
                      h["alpha"][b, hh], h["beta"][b, hh])
    return Mo[:N], out


def _check_all(h, M, out, what):
    B, H = h["widx"].shape[:2]
    Mh, oh = M.cpu().numpy(), out.cpu().numpy()
    for b in range(B):
        for hh in range(H):
            Mo, oo = _oracle(h, b, hh)
            check_values(oh[b, hh], oo, F32, f"{what} out b={b} h={hh}")
            check_values(Mh[b, hh], Mo, F32, f"{what} M b={b} h={hh}")


def _shards(B, H, d_v):
    import sparse_memory_linear_sdm_amd as sdm

    # the workspace holds S * B*H*T*d_v partial floats when S > 1 (T = 64:
    # every section is a multiple of the 256-byte alignment)
    T = 64
    lists = (4 + 512 + 512 + 128 + 128) * B * H * T
    for S_ in (1, 2, 4, 8, 16):
        lay = lists * S_
        extra = S_ * B * H * T * d_v * 4 if S_ > 1 else 0
        if sdm.scan_plan_workspace_size(B, H, d_v, T) == lay + extra:
            return S_
    return None


@pytest.mark.parametrize("B,H,N,d_v,T,W,R,expect_S", [
    (1, 16, 4096, 128, 203, 64, 64, 8),   # the long-stream shape's launch: 8 shards
    (2, 2, 1024, 64, 77, 37, 50, 8),      # W, R below 64; T not a multiple of 8
    (4, 8, 2048, 128, 100, 64, 64, 2),    # 2 shards
    (8, 8, 4096, 128, 41, 64, 64, 1),     # one shard: every row of a step in one list
    (1, 4, 512, 256, 64, 16, 64, 8),
    (3, 1, 300, 32, 33, 64, 8, 8),
    (1, 1, 1000, 128, 1, 64, 64, 8),      # a single step
    (1, 2, 1000, 128, 3, 64, 64, 8),      # fewer steps than the prefetch depth
])
def test_planned_parity(B, H, N, d_v, T, W, R, expect_S):
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    assert _shards(B, H, d_v) == expect_S
    h = _inputs(B, H, N, d_v, T, W, R, seed=B * 100 + H * 10 + T)
    d = _dev(h)
    M = d["M0"].clone()
    out = _planned(d, M, d_v)
    _check_all(h, M, out, f"planned S={expect_S}")
    # sdm_scan on the same inputs: the same state bit for bit
    M2 = d["M0"].clone()
    out2 = sdm.scan(M2, d["widx"], d["wk"], d["ridx"], d["rw"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(M, M2)
    assert float((out - out2).abs().max()) <= 2 * FP32_ATOL


@pytest.mark.parametrize("pool,W,R", [(96, 32, 32), (70, 64, 64), (200, 64, 16)])
def test_planned_hazards(pool, W, R):
    # rows from a small pool: most steps read rows written one to a few steps
    # before (inside the prefetch window) or in the same step
    B, H, N, d_v, T = 1, 16, 4096, 128, 150
    h = _inputs(B, H, N, d_v, T, W, R, seed=pool + W, pool=pool)
    d = _dev(h)
    M = d["M0"].clone()
    out = _planned(d, M, d_v)
    _check_all(h, M, out, f"hazards pool={pool}")


def test_planned_read_rows_equal_write_rows():
    B, H, N, d_v, T, W = 1, 16, 2048, 64, 60, 64
    h = _inputs(B, H, N, d_v, T, W, W, seed=9)
    h["ridx"] = h["widx"].copy()  # every read row written by the same step
    h["ridx"][..., 1::2, :] = np.roll(h["widx"], 1, axis=2)[..., 1::2, :]  # or by the step before
    d = _dev(h)
    M = d["M0"].clone()
    out = _planned(d, M, d_v)
    _check_all(h, M, out, "read = write rows")


@pytest.mark.parametrize("pool", [None, 150])
@pytest.mark.parametrize("B,H", [(1, 16), (4, 8)])
def test_planned_one_shard_crowded(pool, B, H):
    # every row in shard 0: 64-row lists, past the fast path's capacity, so
    # every step takes the synchronous path (with hazards when pooled); with
    # pooled rows later steps also name writers at list positions the ring
    # does not hold
    N, d_v, T = 8192, 128, 90
    S_ = _shards(B, H, d_v)
    assert S_ > 1
    rows0 = np.nonzero(_shard(np.arange(N), S_) == 0)[0]
    h = _inputs(B, H, N, d_v, T, 64, 64, seed=31, pool=pool, rows_from=rows0)
    d = _dev(h)
    M = d["M0"].clone()
    out = _planned(d, M, d_v)
    _check_all(h, M, out, f"crowded shard pool={pool}")


def test_planned_skipped_rows():
    B, H, N, d_v, T = 2, 4, 1024, 128, 70
    h = _inputs(B, H, N, d_v, T, 64, 64, seed=77, skipped=True)
    d = _dev(h)
    M = d["M0"].clone()
    out = _planned(d, M, d_v)
    _check_all(h, M, out, "skipped rows")


def test_planned_chunked_equals_whole_and_deterministic():
    import torch

    B, H, N, d_v, T = 1, 16, 4096, 128, 120
    h = _inputs(B, H, N, d_v, T, 64, 64, seed=5, pool=300)
    d = _dev(h)
    M1 = d["M0"].clone()
    o1 = _planned(d, M1, d_v)
    M2 = d["M0"].clone()
    o2 = _planned(d, M2, d_v, splits=[1, 30, 7, 64, 18])
    M3 = d["M0"].clone()
    o3 = _planned(d, M3, d_v)
    assert torch.equal(M1, M2) and torch.equal(o1, o2)
    assert torch.equal(M1, M3) and torch.equal(o1, o3)


def test_planned_workspace_errors():
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    B, H, N, d_v, T = 1, 2, 256, 64, 10
    h = _inputs(B, H, N, d_v, T, 8, 8, seed=1)
    d = _dev(h)
    need = sdm.scan_plan_workspace_size(B, H, d_v, T)
    small = torch.empty((need - 256,), dtype=torch.uint8, device="cuda")
    with pytest.raises(sdm.SDMError, match="needed"):
        sdm.scan_plan(d["widx"], d["wk"], d["ridx"], d["rw"], N, d_v, workspace=small)
    assert sdm.scan_plan_workspace_size(B, H, 16, T) == 0
    with pytest.raises(sdm.SDMError, match="d_v"):
        sdm.scan_plan(d["widx"], d["wk"], d["ridx"], d["rw"], N, 16)


@pytest.mark.slow
def test_planned_long_shape_full_size():
    """The long-stream launch the bench times: 16 memories of 2^20 x 128
    fp32, 16384 steps per call, two consecutive calls, rows from the
    selections of the long workload's seeded scores.  The whole state and
    output against sdm_scan on a copy (state bit for bit, outputs within
    the bar), and head 7 against the oracle in one column of every 32-column
    tile (each column's recurrence involves that column alone)."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["long"]
    C, hc = 16384, 7
    cols = [32 * k + (9 * k) % 32 for k in range(cfg.d_v // 32)]
    M0 = torch.empty((cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, cfg.B)
    Mref = M.clone()
    Mo = S.host_block(cfg, "M0", h0=hc, nh=1)[0].copy()
    del M0
    for c in range(2):
        t0 = c * C
        d = {k: torch.empty(s, dtype=torch.float32, device="cuda") for k, s in (
            ("s1", (cfg.B, cfg.H, C, cfg.n)), ("s2", (cfg.B, cfg.H, C, cfg.n)),
            ("q1", (cfg.B, cfg.H, C, cfg.n)), ("q2", (cfg.B, cfg.H, C, cfg.n)),
            ("v", (cfg.B, cfg.H, C, cfg.d_v)), ("alpha", (cfg.B, cfg.H, C)),
            ("beta", (cfg.B, cfg.H, C)))}
        for k, t in d.items():
            S.device_block(cfg, k, t, t0=t0)
        widx, _, wk = sdm.select(d["s1"], d["s2"], cfg.W)
        ridx, _, rw = sdm.select(d["q1"], d["q2"], cfg.R)
        ws = sdm.scan_plan(widx, wk, ridx, rw, cfg.N, cfg.d_v)
        out = sdm.scan_planned(M, d["v"], d["alpha"], d["beta"], ws)
        out_ref = sdm.scan(Mref, widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"])
        torch.cuda.synchronize()
        err = float((out - out_ref).abs().max())
        assert err <= 2 * FP32_ATOL, f"chunk {c}: out differs from sdm_scan by {err:.3e}"
        assert torch.equal(M, Mref), f"chunk {c}: state differs from sdm_scan"
        g = {k: t[0, hc].cpu().numpy() for k, t in
             (("widx", widx), ("wk", wk), ("ridx", ridx), ("rw", rw), ("v", d["v"]),
              ("alpha", d["alpha"]), ("beta", d["beta"]))}
        oo = np.zeros((C, cfg.d_v), np.float32)
        for col in cols:
            oracle.scan(Mo, F32, g["widx"], g["wk"], g["ridx"], g["rw"], g["v"], g["alpha"],
                        g["beta"], cols=(col, col + 1), out=oo)
        gout = out[0, hc][:, cols].cpu().numpy()
        check_values(gout, oo[:, cols], F32, f"long planned chunk {c} out")
        print(f"long planned: chunk {c} checked (max |out - sdm_scan| {err:.2e})", flush=True)
        del d, widx, wk, ridx, rw, ws, out, out_ref
        torch.cuda.empty_cache()
    gm = M[0, hc][:, cols].cpu().numpy()
    check_values(gm, Mo[:, cols], F32, "long planned final M")
