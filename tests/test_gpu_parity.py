"""GPU parity of every call of the C ABI against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles, waves and blocks
and leave ragged tails.  Selected indices are compared bit for bit; memory
and outputs within the stated bars (tests/gpu_util.py)."""
import numpy as np
import pytest

import oracle
import sdm_inputs as S
from tests.gpu_util import (NAMES, check_selection, check_values, gpu_sequence, host_inputs,
                            oracle_memory, state_to_host, to_dev)

pytestmark = pytest.mark.gpu

F32, BF16 = oracle.F32, oracle.BF16


def _torch():
    import torch

    return torch


def _sel_case(x1, x2, K):
    import sparse_memory_linear_sdm_amd as sdm

    torch = _torch()
    gi, gs, gw = sdm.select(torch.from_numpy(x1).cuda(), torch.from_numpy(x2).cuda(), K)
    torch.cuda.synchronize()
    oi, os_, ow = oracle.select(x1, x2, K, threads=8)
    check_selection(gi.cpu().numpy(), gs.cpu().numpy(), gw.cpu().numpy(), oi, os_, ow,
                    f"n={x1.shape[-1]} K={K}")


@pytest.mark.parametrize("n,K,units", [(8, 8, 33), (16, 5, 70), (37, 9, 129), (64, 64, 257),
                                       (64, 8, 1000), (128, 32, 301), (256, 32, 515),
                                       (512, 17, 130), (1024, 64, 1027), (2048, 64, 64),
                                       (1024, 1, 50), (256, 2, 50)])
def test_select_random(n, K, units):
    cfg = S.CONFIGS["tiny"].with_(n=n, T=units, seed=1000 + n + K)
    x1 = S.host_block(cfg, "s1")[0, 0]
    x2 = S.host_block(cfg, "s2")[0, 0]
    _sel_case(x1, x2, K)


@pytest.mark.parametrize("n,K", [(8, 3), (64, 17), (256, 32), (1024, 64), (2048, 40)])
def test_select_integer_ties(n, K):
    # Small integers: many exactly equal halves and sums; the lower index
    # (stage 1) and the lower flat index (stage 2) must win every tie.
    rng = np.random.default_rng(n * 31 + K)
    x1 = rng.integers(-2, 3, (300, n)).astype(np.float32)
    x2 = rng.integers(-2, 3, (300, n)).astype(np.float32)
    _sel_case(x1, x2, K)


@pytest.mark.parametrize("n,K,spread", [(64, 64, 0.9), (256, 64, 3.0), (1024, 33, 0.9),
                                        (1024, 64, 5.0), (128, 7, 3.0)])
def test_select_rounding_ties(n, K, spread):
    # x1 on even integers near 2^24 (ulp 2) and x2 small: binary32 sums round
    # back onto the x1 grid, so whole rows of stage-2 pairs tie although the
    # x2 values differ; ties run far past any small candidate set and the
    # lower flat index must still win every one of them.
    rng = np.random.default_rng(n * 7 + K)
    x1 = (2.0 ** 24 + 2.0 * rng.integers(0, 6, (200, n))).astype(np.float32)
    x2 = rng.uniform(-spread, spread, (200, n)).astype(np.float32)
    _sel_case(x1, x2, K)
    _sel_case(x2, x1, K)


def test_select_degenerate_inputs():
    n = 256
    z = np.zeros((4, n), np.float32)
    _sel_case(z, z, 64)                       # everything ties
    neg = z.copy()
    neg[:, ::2] = -0.0                        # -0 and +0 must compare equal
    _sel_case(neg, z, 16)
    one = np.ones((3, 2), np.float32)
    one[:, 1] = 1.0 + 2.0 ** -23              # rounding tie of the sums
    two = np.tile(np.array([2.0, -5.0], np.float32), (3, 1))
    _sel_case(one, two, 1)
    _sel_case(one, two, 2)
    big = np.full((2, 64), -1.5e38, np.float32)
    big[:, 5] = 1.5e38
    _sel_case(big, big, 8)                    # sums near the binary32 limit
    ramp = np.tile(np.arange(1024, dtype=np.float32), (2, 1))
    _sel_case(ramp, ramp[:, ::-1].copy(), 64)


def test_state_init_bitwise():
    torch = _torch()
    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["small"].with_(B=3, H=2)
    M0 = S.host_block(cfg, "M0")
    for dtype, tdt in ((F32, torch.float32), (BF16, torch.bfloat16)):
        M = sdm.state_init(torch.from_numpy(M0).cuda(), cfg.B, tdt)
        ref = oracle.state_init(M0, cfg.B, dtype)
        assert np.array_equal(state_to_host(M), ref)


def _full_parity(cfg, dtype=F32, host=None, check_all=True):
    """Whole [B,H,T] block on the GPU; every memory against the oracle."""
    torch = _torch()
    import sparse_memory_linear_sdm_amd as sdm

    host = host or host_inputs(cfg)
    M0 = S.host_block(cfg, "M0")
    dev = to_dev(host)
    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    M = sdm.state_init(torch.from_numpy(M0).cuda(), cfg.B, tdt)
    g = gpu_sequence(cfg, dev, M)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items()}
    Mh = state_to_host(M)
    for b in range(cfg.B):
        for h in range(cfg.H):
            o = oracle_memory(cfg, host, b, h, M0[h], dtype, threads=8)
            tag = f"{cfg.name} b={b} h={h}"
            check_selection(g["widx"][b, h], g["wscore"][b, h], g["wk"][b, h], o["widx"],
                            o["wscore"], o["wk"], tag + " write")
            check_selection(g["ridx"][b, h], g["rscore"][b, h], g["rw"][b, h], o["ridx"],
                            o["rscore"], o["rw"], tag + " read")
            gm = Mh[b, h] if dtype == F32 else oracle.bf16_bits_to_f32(Mh[b, h])
            om = o["M"] if dtype == F32 else oracle.bf16_bits_to_f32(o["M"])
            check_values(gm, om, dtype, tag + " M")
            check_values(g["out"][b, h], o["out"], dtype, tag + " out")
    return g, Mh


def test_tiny_config_parity():
    _full_parity(S.CONFIGS["tiny"])


def test_small_config_parity_subset():
    # The small workload's shapes (n=256, d_v=64, W=R=32) on 2 of its 16
    # memories and its first 512 steps; the full config runs in the
    # full-size tests.  (An earlier scan producer faulted here: its per-chunk
    # value descriptor had a negative range past the end of the sequence for
    # column tiles > 0.  That loader is gone; every descriptor the kernels
    # build now comes from ranges.h, checked on the host before each launch
    # and for this shape by tests/test_buffer_ranges.py.)
    cfg = S.CONFIGS["small"].with_(B=1, H=2, T=512)
    _full_parity(cfg)


@pytest.mark.parametrize("d_v", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_scan_shapes(d_v, dtype):
    # Ragged: 3 memories (not a multiple of the 8-way XCD grouping), T not a
    # multiple of the 16-step LDS chunk, W and R not multiples of the rows
    # one wave instruction covers.
    cfg = S.CONFIGS["tiny"].with_(B=1, H=3, n=32, d_v=d_v, T=37, W=13, R=29,
                                  state="f32" if dtype == F32 else "bf16", seed=77 + d_v)
    _full_parity(cfg, dtype)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_scan_wide_tiles(dtype):
    # 96 memories x d_v 64: too many for 16-column tiles on one pass of the
    # chip, so the scan takes 32-column tiles with one step in flight (the
    # mid workload's configuration), here checked element by element.
    cfg = S.CONFIGS["tiny"].with_(B=2, H=48, n=32, d_v=64, T=45, W=13, R=29,
                                  state="f32" if dtype == F32 else "bf16", seed=991)
    _full_parity(cfg, dtype)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_scan_narrow_tiles_one_shard(dtype):
    # 20 memories x d_v 128 on 256 compute units: 16-column tiles fit (160
    # workgroups) but two row shards would not (320), so each (memory, tile)
    # is one workgroup handling every row.  The smaller configurations run
    # the two-shard path and the 96-memory case above the wide tiles.
    cfg = S.CONFIGS["tiny"].with_(B=2, H=10, n=32, d_v=128, T=45, W=13, R=29,
                                  state="f32" if dtype == F32 else "bf16", seed=992)
    _full_parity(cfg, dtype)


def _scan_row_shard(N):
    # The scan's row-shard hash, restated here only to build worst cases for
    # the two-shard path: row r belongs to shard (r * 0xC2B2AE35 mod 2^32) >> 31.
    r = np.arange(N, dtype=np.uint64)
    return ((r * 0xC2B2AE35) & 0xFFFFFFFF) >> 31


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_scan_row_shards_crowded_steps(dtype):
    # Two memories (so the rows are split between two workgroups), W = R = 64,
    # and index lists built so that one shard holds anywhere from 0 to all 64
    # of a step's rows, for writes and reads, in shuffled slot order.  The rows
    # come from pools of 72 per shard, so nearly every row recurs within the
    # prefetch window and many are read in the step that writes them.
    torch = _torch()
    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["tiny"].with_(B=1, H=2, n=32, d_v=32, T=70, W=64, R=64,
                                  state="f32" if dtype == F32 else "bf16", seed=993)
    H, T, N, d_v = cfg.H, cfg.T, cfg.N, cfg.d_v
    owner = _scan_row_shard(N)
    rng = np.random.default_rng(993)
    pools = [rng.choice(np.flatnonzero(owner == k), 72, replace=False) for k in (0, 1)]

    def lists(pattern, h):
        idx = np.empty((T, 64), np.int32)
        for t in range(T):
            k0 = pattern[(t + 3 * h) % len(pattern)]
            rows = np.concatenate([rng.choice(pools[0], k0, replace=False),
                                   rng.choice(pools[1], 64 - k0, replace=False)])
            idx[t] = rng.permutation(rows)
        return idx

    widx = np.stack([lists([64, 56, 49, 48, 40, 32, 16, 15, 8, 0], h) for h in range(H)])[None]
    ridx = np.stack([lists([0, 15, 33, 49, 64, 60, 20, 52, 48, 5], h) for h in range(H)])[None]
    counts = (owner[widx] == 0).sum(-1)
    assert counts.max() == 64 and counts.min() == 0  # each shard gets every row of some step
    wk = rng.uniform(0.0, 0.05, widx.shape).astype(np.float32)
    rw = rng.uniform(0.0, 0.05, ridx.shape).astype(np.float32)
    v = rng.standard_normal((1, H, T, d_v)).astype(np.float32)
    alpha = rng.uniform(0.9, 1.0, (1, H, T)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (1, H, T)).astype(np.float32)
    M0 = S.host_block(cfg, "M0")

    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    M = sdm.state_init(torch.from_numpy(M0).cuda(), 1, tdt)
    out = sdm.scan(M, *(torch.from_numpy(a).cuda() for a in (widx, wk, ridx, rw, v, alpha, beta)))
    torch.cuda.synchronize()
    gout = out.cpu().numpy()
    Mh = state_to_host(M)
    for h in range(H):
        Mo = oracle.state_init(M0[h:h + 1], 1, dtype)[0, 0]
        oo = oracle.scan(Mo, dtype, widx[0, h], wk[0, h], ridx[0, h], rw[0, h], v[0, h],
                         alpha[0, h], beta[0, h])
        gm = Mh[0, h] if dtype == F32 else oracle.bf16_bits_to_f32(Mh[0, h])
        om = Mo if dtype == F32 else oracle.bf16_bits_to_f32(Mo)
        check_values(gm, om, dtype, f"crowded shards h={h} M")
        check_values(gout[0, h], oo, dtype, f"crowded shards h={h} out")


@pytest.mark.parametrize("B,H,d_v", [(1, 3, 32), (2, 48, 64)])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_scan_skips_out_of_range_rows(B, H, d_v, dtype):
    """Row indices outside [0, N) given to sdm_scan are skipped: a write slot
    with such a row touches nothing, a read slot contributes 0.  Hand-built
    index lists hold -1, N, N + k, 2^31 - 1 and -2^31 among valid rows drawn
    from a small pool (so rows recur inside the prefetch window and are read
    in the step that writes them).  The oracle, which accepts valid rows only,
    runs the same steps on a table extended past N: each invalid write slot j
    writes sink row N + j (never compared), each invalid read slot reads row
    N + W, which nothing writes and stays zero.  (3 memories take the
    two-shard narrow-tile path, 96 memories the wide-tile path.)"""
    torch = _torch()
    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["tiny"].with_(B=B, H=H, n=32, d_v=d_v, T=60, W=16, R=16,
                                  state="f32" if dtype == F32 else "bf16", seed=995 + H)
    T, N, W, R = cfg.T, cfg.N, cfg.W, cfg.R
    rng = np.random.default_rng(995 + H + d_v)
    pool = rng.choice(N, 40, replace=False)
    bad_vals = np.array([-1, N, N + 7, N + 1000, 2 ** 31 - 1, -2 ** 31], np.int64)

    def lists(K):
        idx = np.empty((B, H, T, K), np.int32)
        for b in range(B):
            for h in range(H):
                for t in range(T):
                    row = rng.choice(pool, K, replace=False).astype(np.int64)
                    bad = rng.random(K) < 0.3
                    row[bad] = rng.choice(bad_vals, int(bad.sum()))
                    idx[b, h, t] = row.astype(np.int32)
        return idx

    widx, ridx = lists(W), lists(R)
    assert (widx < 0).any() and (widx >= N).any() and (ridx < 0).any() and (ridx >= N).any()
    wk = rng.uniform(0.0, 0.3, widx.shape).astype(np.float32)
    rw = rng.uniform(0.0, 0.3, ridx.shape).astype(np.float32)
    v = rng.standard_normal((B, H, T, d_v)).astype(np.float32)
    alpha = rng.uniform(0.9, 1.0, (B, H, T)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, H, T)).astype(np.float32)
    M0 = S.host_block(cfg, "M0")
    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    M = sdm.state_init(torch.from_numpy(M0).cuda(), B, tdt)
    out = sdm.scan(M, *(torch.from_numpy(a).cuda() for a in (widx, wk, ridx, rw, v, alpha, beta)))
    torch.cuda.synchronize()
    gout, Mh = out.cpu().numpy(), state_to_host(M)
    slot = np.arange(W, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            wi = widx[b, h].copy()
            ri = ridx[b, h].copy()
            wbad = (wi < 0) | (wi >= N)
            wi[wbad] = (N + np.broadcast_to(slot, wi.shape))[wbad]
            ri[(ri < 0) | (ri >= N)] = N + W
            ext = np.zeros((N + W + 1, d_v), np.float32)
            ext[:N] = M0[h]
            Mo = oracle.state_init(ext[None], 1, dtype)[0, 0].copy()
            oo = oracle.scan(Mo, dtype, wi, wk[b, h].astype(np.float64), ri,
                             rw[b, h].astype(np.float64), v[b, h], alpha[b, h], beta[b, h])
            assert not Mo[N + W].any()
            tag = f"invalid rows b={b} h={h}"
            gm = Mh[b, h] if dtype == F32 else oracle.bf16_bits_to_f32(Mh[b, h])
            om = Mo[:N] if dtype == F32 else oracle.bf16_bits_to_f32(Mo[:N])
            check_values(gm, om, dtype, tag + " M")
            check_values(gout[b, h], oo, dtype, tag + " out")


def test_hazard_same_rows_every_step():
    # Constant sub-scores: every step writes and reads the same slots, so
    # each step's loads depend on the previous step's stores.
    cfg = S.CONFIGS["tiny"].with_(B=1, H=2, T=70, d_v=32)
    host = host_inputs(cfg)
    for k in ("s1", "s2", "q1", "q2"):
        host[k][:] = host[k][:, :, :1]
    _full_parity(cfg, host=host)


def test_hazard_read_rows_equal_write_rows():
    cfg = S.CONFIGS["tiny"].with_(B=2, H=1, T=50, W=8, R=8)
    host = host_inputs(cfg)
    host["q1"], host["q2"] = host["s1"].copy(), host["s2"].copy()
    _full_parity(cfg, host=host)
    _full_parity(cfg, BF16, host=host)


def test_hazard_dense_reuse_small_table():
    # n = 8: N = 64 slots and W = R = 8 -- rows repeat constantly.
    cfg = S.CONFIGS["tiny"].with_(B=2, H=2, n=8, d_v=16, T=300, W=8, R=8)
    _full_parity(cfg)
    _full_parity(cfg.with_(state="bf16"), BF16)


def test_chunked_scan_bitwise_and_deterministic():
    torch = _torch()
    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["tiny"].with_(B=2, H=2, T=100, n=16, d_v=32)
    host = host_inputs(cfg)
    dev = to_dev(host)
    M0 = torch.from_numpy(S.host_block(cfg, "M0")).cuda()
    widx, _, wk = sdm.select(dev["s1"], dev["s2"], cfg.W)
    ridx, _, rw = sdm.select(dev["q1"], dev["q2"], cfg.R)
    args = (widx, wk, ridx, rw, dev["v"], dev["alpha"], dev["beta"])
    M1 = sdm.state_init(M0, cfg.B)
    o1 = sdm.scan(M1, *args)
    M2 = sdm.state_init(M0, cfg.B)
    o2 = sdm.scan(M2, *args)
    M3 = sdm.state_init(M0, cfg.B)
    parts = []
    for t0, t1 in ((0, 31), (31, 32), (32, 100)):
        parts.append(sdm.scan(M3, *(a[:, :, t0:t1].contiguous() for a in args)))
    torch.cuda.synchronize()
    assert torch.equal(M1, M2) and torch.equal(o1, o2)
    assert torch.equal(M1, M3) and torch.equal(o1, torch.cat(parts, dim=2))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_step_decode_parity(dtype):
    cfg = S.CONFIGS["decode"].with_(B=3, H=2, n=64, T=12, W=16, R=24,
                                    state="f32" if dtype == F32 else "bf16")
    _decode_parity(cfg, dtype)


@pytest.mark.parametrize("d_v", [128, 256])
@pytest.mark.parametrize("overlap", ["all", "part"])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_step_decode_reads_rows_it_writes(dtype, overlap, d_v):
    # Read sub-scores equal to the write ones ("all": every read row is a row
    # this step writes) or sharing one half ("part": some are).  With d_v 128
    # a step's rows fit one batch of loads and the read takes rows written in
    # the same step from the block's LDS copy; with d_v 256 the write and the
    # read run one after the other.
    cfg = S.CONFIGS["decode"].with_(B=2, H=2, n=64, T=6, W=64, R=64, d_v=d_v,
                                    state="f32" if dtype == F32 else "bf16", seed=405)
    host = host_inputs(cfg)
    host["q1"] = host["s1"].copy()
    if overlap == "all":
        host["q2"] = host["s2"].copy()
    _decode_parity(cfg, dtype, host)


@pytest.mark.parametrize("n,W,R,d_v,B,H", [
    (256, 64, 64, 128, 3, 2),   # the rows in one batch of loads per thread
    (256, 64, 64, 256, 2, 1),   # fp32: the write, then the read after a barrier
    (512, 17, 40, 64, 2, 2),
    (1024, 64, 64, 64, 1, 2),
    (2048, 33, 64, 16, 1, 1),
    (256, 1, 1, 16, 2, 2),
])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_step_decode_parity_large_n(dtype, n, W, R, d_v, B, H):
    # n = 256 .. 2048 (4 to 32 keys per lane in stage 1), random scores,
    # several consecutive tokens
    cfg = S.CONFIGS["decode"].with_(B=B, H=H, n=n, T=4, W=W, R=R, d_v=d_v,
                                    state="f32" if dtype == F32 else "bf16", seed=406 + n + W)
    _decode_parity(cfg, dtype)


@pytest.mark.parametrize("overlap", ["all", "part"])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_step_decode_reads_rows_it_writes_n256(dtype, overlap):
    cfg = S.CONFIGS["decode"].with_(B=2, H=2, n=256, T=4, W=64, R=64, d_v=128,
                                    state="f32" if dtype == F32 else "bf16", seed=407)
    host = host_inputs(cfg)
    host["q1"] = host["s1"].copy()
    if overlap == "all":
        host["q2"] = host["s2"].copy()
    _decode_parity(cfg, dtype, host)


def _decode_parity(cfg, dtype, host=None):
    torch = _torch()
    import sparse_memory_linear_sdm_amd as sdm

    host = host or host_inputs(cfg)
    dev = to_dev(host)
    M0 = S.host_block(cfg, "M0")
    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    M = sdm.state_init(torch.from_numpy(M0).cuda(), cfg.B, tdt)
    Mo = oracle.state_init(M0, cfg.B, dtype)
    for t in range(cfg.T):
        step = [dev[k][:, :, t].contiguous() for k in NAMES]
        out, wi, ri = sdm.step_decode(M, *step, cfg.W, cfg.R)
        oo, owi, ori = oracle.step_decode(Mo, dtype, *(host[k][:, :, t] for k in NAMES), cfg.W,
                                          cfg.R)
        torch.cuda.synchronize()
        assert np.array_equal(wi.cpu().numpy(), owi) and np.array_equal(ri.cpu().numpy(), ori)
        check_values(out.cpu().numpy(), oo, dtype, f"decode out t={t}")
    Mh = state_to_host(M)
    for b in range(cfg.B):
        for h in range(cfg.H):
            gm = Mh[b, h] if dtype == F32 else oracle.bf16_bits_to_f32(Mh[b, h])
            om = Mo[b, h] if dtype == F32 else oracle.bf16_bits_to_f32(Mo[b, h])
            check_values(gm, om, dtype, f"decode M b={b} h={h}")


@pytest.mark.parametrize("n", [32, 256])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_step_decode_equals_scan(dtype, n):
    torch = _torch()
    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["decode"].with_(B=2, H=2, n=n, T=20 if n == 32 else 8, W=12, R=12, d_v=64)
    dev = to_dev(host_inputs(cfg))
    M0 = torch.from_numpy(S.host_block(cfg, "M0")).cuda()
    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    Md = sdm.state_init(M0, cfg.B, tdt)
    outs = []
    for t in range(cfg.T):
        o, _, _ = sdm.step_decode(Md, *(dev[k][:, :, t].contiguous() for k in NAMES), cfg.W,
                                  cfg.R)
        outs.append(o)
    Ms = sdm.state_init(M0, cfg.B, tdt)
    g = gpu_sequence(cfg, dev, Ms)
    torch.cuda.synchronize()
    assert torch.equal(Md, Ms)
    # Same rows and weights, same per-element update; the read sums the same
    # products in a different order, so compare within the bar.
    check_values(torch.stack(outs, 2).cpu().numpy(), g["out"].cpu().numpy(), F32,
                 "decode vs scan out")


@pytest.mark.parametrize("n,W,R", [(64, 16, 64), (256, 64, 37), (1024, 64, 64), (512, 1, 5),
                                   (2048, 64, 64)])
def test_step_decode_selection_ties(n, W, R):
    # The fused decode step runs its own search variant; its write and read
    # indices must equal the oracle's selection bit for bit on inputs full of
    # exact ties (small integers) and binary32 rounding ties.
    import sparse_memory_linear_sdm_amd as sdm

    torch = _torch()
    rng = np.random.default_rng(n + W + R)
    B, H, d_v = 3, 4, 32
    for kind in ("integers", "rounding"):
        if kind == "integers":
            x = rng.integers(-2, 3, (4, B, H, n)).astype(np.float32)
        else:
            x = np.stack([(2.0 ** 24 + 2.0 * rng.integers(0, 6, (B, H, n))),
                          rng.uniform(-3, 3, (B, H, n)), (2.0 ** 24 + 2.0 * rng.integers(0, 6, (B, H, n))),
                          rng.uniform(-0.9, 0.9, (B, H, n))]).astype(np.float32)
        v = rng.standard_normal((B, H, d_v)).astype(np.float32)
        a = np.full((B, H), 0.9, np.float32)
        b = np.full((B, H), 0.5, np.float32)
        M = torch.zeros((B, H, n * n, d_v), dtype=torch.float32, device="cuda")
        dev = [torch.from_numpy(t.copy()).cuda() for t in (*x, v, a, b)]
        _, wi, ri = sdm.step_decode(M, *dev, W, R)
        torch.cuda.synchronize()
        ow, _, _ = oracle.select(x[0].reshape(-1, n), x[1].reshape(-1, n), W, threads=8)
        orr, _, _ = oracle.select(x[2].reshape(-1, n), x[3].reshape(-1, n), R, threads=8)
        assert np.array_equal(wi.cpu().numpy().reshape(-1, W), ow), f"{kind}: write indices"
        assert np.array_equal(ri.cpu().numpy().reshape(-1, R), orr), f"{kind}: read indices"


def test_step_decode_graph_replays_match_eager():
    # The decode calls of several tokens captured in a HIP graph and replayed
    # three times, with eager work and synchronisations in between; every
    # replay must equal the same calls run eagerly from the same state.
    import sparse_memory_linear_sdm_amd as sdm

    torch = _torch()
    cfg = S.CONFIGS["decode"].with_(B=4, H=2, n=64, T=6, W=16, R=16)
    dev = to_dev(host_inputs(cfg))
    steps = [[dev[k][:, :, t].contiguous() for k in NAMES] for t in range(cfg.T)]
    M0 = torch.from_numpy(S.host_block(cfg, "M0")).cuda()
    Mg = sdm.state_init(M0, cfg.B, torch.bfloat16)
    out_g = torch.empty((cfg.B, cfg.H, cfg.d_v), dtype=torch.float32, device="cuda")

    def calls(M, out):
        for st in steps:
            sdm.step_decode(M, *st, cfg.W, cfg.R, out=out, want_idx=False)

    calls(Mg, out_g)  # warm up outside the capture
    torch.cuda.synchronize()
    Mg.copy_(sdm.state_init(M0, cfg.B, torch.bfloat16))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(Mg, out_g)
    torch.cuda.synchronize()
    Mg.copy_(sdm.state_init(M0, cfg.B, torch.bfloat16))
    Me = sdm.state_init(M0, cfg.B, torch.bfloat16)
    out_e = torch.empty_like(out_g)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        calls(Me, out_e)
        torch.cuda.synchronize()
        assert torch.equal(Mg, Me), f"replay {rep}: state differs"
        assert torch.equal(out_g, out_e), f"replay {rep}: output differs"


# ---------------------------------------------------------------- fp8 E4M3 state

def _fp8_codes(t):
    return t.contiguous().view(_torch().uint8).cpu().numpy()


def test_state_init_fp8_bitwise_rounding():
    """Every finite E4M3 value, every midpoint between neighbours (exact ties),
    the binary32 neighbours of each midpoint, and random values at several
    scales: the GPU's E4M3 codes equal the oracle's, bit for bit."""
    import sparse_memory_linear_sdm_amd as sdm

    torch = _torch()
    t = np.array([oracle.fp8_to_double(c) for c in range(0x7F)])
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(5)
    vals = [t.astype(np.float32), mids, np.nextafter(mids, np.float32(1e9)),
            np.nextafter(mids, np.float32(-1e9))]
    vals += [(rng.standard_normal(4096) * s).astype(np.float32) for s in (1e-3, 0.02, 1.0, 50.0)]
    x = np.concatenate(vals)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448.0]
    d_v = 64
    x = np.concatenate([x, np.zeros((-x.size) % (2 * d_v), np.float32)]).reshape(2, -1, d_v)
    M = sdm.state_init(torch.from_numpy(x).cuda(), 3, torch.float8_e4m3fn)
    torch.cuda.synchronize()
    ref = oracle.state_init(x, 3, oracle.FP8)
    got = _fp8_codes(M)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, [(float(x[tuple(i[1:])]), int(got[tuple(i)]), int(ref[tuple(i)]))
                           for i in bad[:5]]


def _fp8_scan_case(cfg):
    """fp8 state: the GPU scan and the oracle scan on the same binary32
    selection weights (the oracle's, rounded to binary32), so the stored codes
    must agree bit for bit; outputs within the fp32 bar."""
    import sparse_memory_linear_sdm_amd as sdm

    torch = _torch()
    host = host_inputs(cfg)
    M0 = S.host_block(cfg, "M0")
    sel = {}
    for b in range(cfg.B):
        for h in range(cfg.H):
            wi, _, wk = oracle.select(host["s1"][b, h], host["s2"][b, h], cfg.W)
            ri, _, rw = oracle.select(host["q1"][b, h], host["q2"][b, h], cfg.R)
            sel[b, h] = (wi, wk.astype(np.float32), ri, rw.astype(np.float32))

    def stack(i, dt):
        return np.stack([np.stack([sel[b, h][i] for h in range(cfg.H)]) for b in range(cfg.B)]
                        ).astype(dt)

    widx, wk, ridx, rw = stack(0, np.int32), stack(1, np.float32), stack(2, np.int32), \
        stack(3, np.float32)
    dev = to_dev({k: host[k] for k in ("v", "alpha", "beta")})
    M = sdm.state_init(torch.from_numpy(M0).cuda(), cfg.B, torch.float8_e4m3fn)
    out = sdm.scan(M, *(torch.from_numpy(a).cuda() for a in (widx, wk, ridx, rw)), dev["v"],
                   dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    Mg, og = _fp8_codes(M), out.cpu().numpy()
    for b in range(cfg.B):
        for h in range(cfg.H):
            Mo = oracle.state_init(M0[h][None], 1, oracle.FP8)[0, 0].copy()
            oo = oracle.scan(Mo, oracle.FP8, widx[b, h], wk[b, h].astype(np.float64), ridx[b, h],
                             rw[b, h].astype(np.float64), host["v"][b, h], host["alpha"][b, h],
                             host["beta"][b, h])
            tag = f"fp8 {cfg.name} b={b} h={h}"
            nbad = int((Mg[b, h] != Mo).sum())
            assert nbad == 0, f"{tag}: {nbad} state codes differ"
            check_values(og[b, h], oo, F32, tag + " out")


@pytest.mark.parametrize("B,H,n,d_v,T,W,R", [
    (8, 36, 16, 32, 40, 8, 8),     # 288 memories x 1 tile: one step in flight
    (5, 16, 64, 128, 70, 64, 64),  # 80 memories x 4 tiles: one step in flight
    (1, 3, 32, 64, 101, 32, 17),   # few memories: three steps in flight, two row shards
    (2, 2, 8, 256, 150, 8, 8),     # 64-slot tables, W = R = 8: heavy reuse, forwarded rows
])
def test_scan_fp8_codes_bitwise(B, H, n, d_v, T, W, R):
    cfg = S.CONFIGS["tiny"].with_(B=B, H=H, n=n, d_v=d_v, T=T, W=W, R=R,
                                  seed=8100 + B + H + n + d_v)
    _fp8_scan_case(cfg)
