"""GPU parity of the training calls (sdm_scan_train, sdm_scan_backward,
sdm_select_backward, sdm_state_init_backward) against the CPU oracle.

Bars.  Indices: bit-exact (checked by the forward tests and again here).
Forward with tape: out and M bitwise equal to sdm_scan; tape (pre-write rows
and the rows each read used) within the fp32 bar of the oracle's.  The
reverse pass leaves the state as the forward left it (bitwise).  Gradients (fp32 on the GPU, float64 in the oracle):
normwise per memory, max|x - y| <= 1e-5 * max(1, max|y|).  Each gradient
element is a sum of at most a few hundred fp32 products per step, carried
over the steps by factors alpha*(1 - beta*k) <= 1, so its fp32 error stays
within a few hundred ulps of the tensor's largest element (~1e-5 relative);
the selection weights themselves differ by ~1e-7 between the sides.
"""
import numpy as np
import pytest

import oracle
import sdm_inputs as S
from tests.gpu_util import check_selection, host_inputs, to_dev

pytestmark = pytest.mark.gpu

GRAD_REL = 1e-5


def _close(g, o, what):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    scale = max(1.0, float(np.abs(o).max()) if o.size else 1.0)
    err = float(np.abs(g - o).max()) if o.size else 0.0
    assert err <= GRAD_REL * scale, f"{what}: error {err} vs scale {scale}"
    return err / scale


def _train_case(cfg, seed_g=None, check_mems=None):
    """Forward with tape, then the reverse pass, on the GPU; every checked
    memory against the oracle's backward on the oracle's own selections."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    host = host_inputs(cfg)
    dout = S.host_block(cfg, "dout")
    M0 = S.host_block(cfg, "M0")
    dev = to_dev(host)
    M = sdm.state_init(torch.from_numpy(M0).cuda(), cfg.B)
    M_start = M.clone()
    widx, wsc, wk = sdm.select(dev["s1"], dev["s2"], cfg.W)
    ridx, rsc, rw = sdm.select(dev["q1"], dev["q2"], cfg.R)
    out, tape = sdm.scan_train(M, widx, wk, ridx, rw, dev["v"], dev["alpha"], dev["beta"])
    # the same forward without a tape gives the same bits
    M2 = M_start.clone()
    out2 = sdm.scan(M2, widx, wk, ridx, rw, dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(M, M2)
    del M2, out2
    if seed_g is None:
        dMT = np.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v), np.float32)
    else:
        dMT = np.random.default_rng(seed_g).standard_normal(
            (cfg.B, cfg.H, cfg.N, cfg.d_v)).astype(np.float32)
    G = torch.from_numpy(dMT).cuda()
    M_end = M.clone()
    gr = sdm.scan_backward(widx, wk, ridx, rw, dev["v"], dev["alpha"], dev["beta"], tape,
                           torch.from_numpy(dout).cuda(), G)
    dM0 = sdm.state_init_backward(G)
    torch.cuda.synchronize()
    assert torch.equal(M, M_end), "the reverse pass must not touch the state"
    del M_start
    gr = {k: v.cpu().numpy() for k, v in gr.items()}
    Gh = G.cpu().numpy()
    tape_h = tape.cpu().numpy()
    gi, gw = widx.cpu().numpy(), wk.cpu().numpy()
    ri, rwh = ridx.cpu().numpy(), rw.cpu().numpy()
    mems = check_mems or [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    worst = 0.0
    for b, h in mems:
        tag = f"{cfg.name} b={b} h={h}"
        o_wi, o_ws, o_wk = oracle.select(host["s1"][b, h], host["s2"][b, h], cfg.W, threads=8)
        o_ri, o_rs, o_rw = oracle.select(host["q1"][b, h], host["q2"][b, h], cfg.R, threads=8)
        check_selection(gi[b, h], wsc[b, h].cpu().numpy(), gw[b, h], o_wi, o_ws, o_wk, tag + " w")
        check_selection(ri[b, h], rsc[b, h].cpu().numpy(), rwh[b, h], o_ri, o_rs, o_rw, tag + " r")
        o = oracle.scan_backward(M0[h], o_wi, o_wk, o_ri, o_rw, host["v"][b, h],
                                 host["alpha"][b, h], host["beta"][b, h], dout[b, h], dMT[b, h])
        worst = max(worst, _close(tape_h[b, h, :, :cfg.W], o["tape"], tag + " tape"))
        worst = max(worst, _close(tape_h[b, h, :, cfg.W:], o["rtape"], tag + " read tape"))
        for k in ("dv", "dwk", "drw", "dalpha", "dbeta"):
            worst = max(worst, _close(gr[k][b, h], o[k], f"{tag} {k}"))
        worst = max(worst, _close(Gh[b, h], o["dM0"], tag + " G"))
    # dM0 = sum over b of G: against the oracle's plain sum of the GPU's G
    want = oracle.state_init_backward(Gh)
    _close(dM0.cpu().numpy(), want, "dM0")
    return worst


# (B, H, n, d_v, T, W, R): each picks a different forward variant and tile
# shape -- 16-column tiles with two row shards (few memories), 16-column
# tiles unsharded, 32-column tiles (many memories), d_v = 16 (one tile) --
# with ragged T and W != R.
CASES = [
    (1, 2, 16, 16, 77, 8, 5),
    (2, 2, 32, 64, 130, 32, 32),
    (3, 7, 16, 128, 45, 16, 9),   # 21 memories: narrow tiles, one shard
    (5, 8, 64, 128, 33, 13, 64),  # 40 memories: 32-column tiles
    (1, 3, 64, 128, 60, 64, 64),  # two shards, full 64-row steps
]


@pytest.mark.parametrize("B,H,n,d_v,T,W,R", CASES)
def test_scan_backward_parity(B, H, n, d_v, T, W, R):
    cfg = S.CONFIGS["tiny"].with_(B=B, H=H, n=n, d_v=d_v, T=T, W=W, R=R,
                                  seed=7000 + B * 100 + H * 10 + W)
    _train_case(cfg, seed_g=B * 1000 + T)


def test_scan_backward_dense_reuse():
    """A tiny table (n = 8, 64 slots) with W = R = 8: rows are re-written and
    re-read at almost every step, read rows coincide with write rows, and the
    hashed match table sees collisions."""
    cfg = S.CONFIGS["tiny"].with_(B=2, H=3, n=8, d_v=32, T=200, W=8, R=8, seed=7777)
    _train_case(cfg, seed_g=5)


def test_scan_backward_small_config_subset():
    """The small workload's shapes (n = 256, d_v = 64, W = R = 32), all 16
    memories, first 512 steps, final-state gradient zero (loss on outputs)."""
    cfg = S.CONFIGS["small"].with_(T=512)
    _train_case(cfg, seed_g=None, check_mems=[(0, 0), (1, 2), (3, 3)])


@pytest.mark.parametrize("n,K,units", [(8, 8, 33), (64, 5, 70), (256, 32, 129), (1024, 64, 300),
                                       (37, 1, 20)])
def test_select_backward_parity(n, K, units):
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["tiny"].with_(n=n, T=units, seed=9100 + n + K)
    x1, x2 = S.host_block(cfg, "s1")[0, 0], S.host_block(cfg, "s2")[0, 0]
    dw = np.random.default_rng(n + K).standard_normal((units, K)).astype(np.float32)
    gi, _, gw = sdm.select(torch.from_numpy(x1).cuda(), torch.from_numpy(x2).cuda(), K)
    d1, d2 = sdm.select_backward(gi, gw, torch.from_numpy(dw).cuda(), n)
    torch.cuda.synchronize()
    oi, _, ow = oracle.select(x1, x2, K, threads=8)
    assert np.array_equal(gi.cpu().numpy(), oi)
    o1, o2 = oracle.select_backward(oi, ow, dw, n)
    _close(d1.cpu().numpy(), o1, "dx1")
    _close(d2.cpu().numpy(), o2, "dx2")
    # exact zeros at every half index no selected slot uses
    used1 = np.zeros((units, n), bool)
    np.put_along_axis(used1, oi // n, True, axis=1)
    assert np.all(d1.cpu().numpy()[~used1] == 0.0)


def test_chunked_training_bitwise():
    """Forward in two chunks (one tape each), then the reverse pass chunk by
    chunk in reverse order carrying G: every gradient is bitwise equal to the
    single-call forward and reverse pass, and the state keeps the forward's
    final value."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["tiny"].with_(B=2, H=3, n=32, d_v=64, T=150, W=32, R=16, seed=9300)
    host = host_inputs(cfg)
    dev = to_dev(host)
    dout = torch.from_numpy(S.host_block(cfg, "dout")).cuda()
    M0 = torch.from_numpy(S.host_block(cfg, "M0")).cuda()
    widx, _, wk = sdm.select(dev["s1"], dev["s2"], cfg.W)
    ridx, _, rw = sdm.select(dev["q1"], dev["q2"], cfg.R)
    names = ("v", "alpha", "beta")

    def sl(x, a, b):
        return x[:, :, a:b].contiguous()

    # whole
    M = sdm.state_init(M0, cfg.B)
    out, tape = sdm.scan_train(M, widx, wk, ridx, rw, *(dev[k] for k in names))
    G = torch.zeros_like(M)
    whole = sdm.scan_backward(widx, wk, ridx, rw, *(dev[k] for k in names), tape, dout, G)
    # two chunks
    T1 = 61
    spans = ((0, T1), (T1, cfg.T))
    M2 = sdm.state_init(M0, cfg.B)
    outs, tapes = [], []
    for a, b in spans:
        o, tp = sdm.scan_train(M2, sl(widx, a, b), sl(wk, a, b), sl(ridx, a, b), sl(rw, a, b),
                               *(sl(dev[k], a, b) for k in names))
        outs.append(o)
        tapes.append(tp)
    G2 = torch.zeros_like(M2)
    parts = {}
    for (a, b), tp in reversed(list(zip(spans, tapes))):
        parts[a] = sdm.scan_backward(sl(widx, a, b), sl(wk, a, b), sl(ridx, a, b),
                                     sl(rw, a, b), *(sl(dev[k], a, b) for k in names), tp,
                                     sl(dout, a, b), G2)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), out)
    assert torch.equal(G2, G)
    assert torch.equal(M2, M)
    assert torch.equal(torch.cat(tapes, dim=2), tape)
    for k in ("dv", "dwk", "drw", "dalpha", "dbeta"):
        assert torch.equal(torch.cat([parts[0][k], parts[T1][k]], dim=2), whole[k]), k


def _touch_reference(widx, ridx, N):
    """The sparse mode's bookkeeping from the index arrays on the host: the
    rows selected at all (as the packed bit table) and, per step, the slots
    whose row is selected for the last time (integer work, compared bit for
    bit)."""
    B, H, T, W = widx.shape
    R = ridx.shape[3]
    last = np.full((B, H, N), -1, np.int64)
    first = np.zeros((B, H, T, 2), np.uint64)
    steps = np.arange(T)
    for b in range(B):
        for h in range(H):
            rows = np.concatenate([widx[b, h], ridx[b, h]], axis=1).ravel()
            t_of = np.repeat(steps, W + R)
            ok = (rows >= 0) & (rows < N)  # indices outside [0, N) are ignored
            np.maximum.at(last[b, h], rows[ok], t_of[ok])
            for m, idx in enumerate((widx[b, h], ridx[b, h])):
                valid = (idx >= 0) & (idx < N)
                hit = valid & (last[b, h][np.where(valid, idx, 0)] == steps[:, None])
                bits = np.left_shift(np.uint64(1), np.arange(idx.shape[1], dtype=np.uint64))
                first[b, h, :, m] = np.bitwise_or.reduce(np.where(hit, bits, np.uint64(0)), axis=1)
    words = (N + 31) // 32
    sel = np.zeros((B, H, words * 32), bool)
    sel[:, :, :N] = last >= 0
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    seen = (sel.reshape(B, H, words, 32) * weights).sum(-1).astype(np.uint32)
    return seen, first


@pytest.mark.parametrize("B,H,n,d_v,T,W,R", CASES[:4] + [(2, 3, 8, 32, 200, 8, 8)])
def test_sparse_mode_matches_dense(B, H, n, d_v, T, W, R):
    """The sparse training mode (no zeroed G; each row's first touch in
    reverse starts from zero; the M0 gradient reads selected rows only) gives
    the dense mode's bits for every selected row of G and for dM0, and its
    per-step sums (dv, dk, dr, dalpha, dbeta; added over another tile width)
    meet the bar against the oracle.  G starts full of NaN, so reading any
    row the mode must not read shows."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["tiny"].with_(B=B, H=H, n=n, d_v=d_v, T=T, W=W, R=R,
                                  seed=9500 + B * 100 + H * 10 + W)
    host = host_inputs(cfg)
    dev = to_dev(host)
    dout_h = S.host_block(cfg, "dout")
    M0_h = S.host_block(cfg, "M0")
    dout = torch.from_numpy(dout_h).cuda()
    M = sdm.state_init(torch.from_numpy(S.host_block(cfg, "M0")).cuda(), cfg.B)
    widx, _, wk = sdm.select(dev["s1"], dev["s2"], cfg.W)
    ridx, _, rw = sdm.select(dev["q1"], dev["q2"], cfg.R)
    names = ("v", "alpha", "beta")
    _, tape = sdm.scan_train(M, widx, wk, ridx, rw, *(dev[k] for k in names))
    G = torch.zeros_like(M)
    gd = sdm.scan_backward(widx, wk, ridx, rw, *(dev[k] for k in names), tape, dout, G)
    dM0 = sdm.state_init_backward(G)
    seen, first = sdm.touch_prepare(widx, ridx, cfg.N)
    Gs = torch.full_like(M, float("nan"))
    gs = sdm.scan_backward(widx, wk, ridx, rw, *(dev[k] for k in names), tape, dout, Gs,
                           first=first)
    dM0s = sdm.state_init_backward(Gs, seen=seen)
    torch.cuda.synchronize()
    want_seen, want_first = _touch_reference(widx.cpu().numpy(), ridx.cpu().numpy(), cfg.N)
    assert np.array_equal(seen.cpu().numpy().view(np.uint32), want_seen)
    assert np.array_equal(first.cpu().numpy().view(np.uint64), want_first)
    touched = sdm.seen_rows(seen, cfg.N)
    assert torch.equal(G[touched], Gs[touched])
    assert torch.isnan(Gs[~touched]).all()  # never written
    assert torch.equal(dM0, dM0s)
    gs = {k: v.cpu().numpy() for k, v in gs.items()}
    for b in range(cfg.B):
        for h in range(cfg.H):
            o_wi, _, o_wk = oracle.select(host["s1"][b, h], host["s2"][b, h], cfg.W, threads=8)
            o_ri, _, o_rw = oracle.select(host["q1"][b, h], host["q2"][b, h], cfg.R, threads=8)
            o = oracle.scan_backward(M0_h[h], o_wi, o_wk, o_ri, o_rw, host["v"][b, h],
                                     host["alpha"][b, h], host["beta"][b, h], dout_h[b, h])
            for k in ("dv", "dwk", "drw", "dalpha", "dbeta"):
                _close(gs[k][b, h], o[k], f"sparse b={b} h={h} {k}")


def test_touch_prepare_ignores_out_of_range_rows():
    """Hand-built selections with indices outside [0, N) (ignored), W != R
    below 64, repeated rows across steps and a row both read and written in
    one step: the masks and the bitmap equal the host's bookkeeping bit for
    bit, over a ragged number of steps (not a multiple of the prefetch)."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    rng = np.random.default_rng(12)
    B, H, N, T, W, R = 2, 3, 300, 53, 7, 5
    widx = np.stack([[[rng.choice(N, W, replace=False) for _ in range(T)] for _ in range(H)]
                     for _ in range(B)]).astype(np.int32)
    ridx = np.stack([[[rng.choice(N, R, replace=False) for _ in range(T)] for _ in range(H)]
                     for _ in range(B)]).astype(np.int32)
    widx[0, 0, 3, 2] = -1
    widx[1, 2, 50, 0] = N + 5
    ridx[0, 1, 7, 4] = -7
    ridx[1, 0, 52, 1] = N
    ridx[0, 0, 10, 0] = widx[0, 0, 10, 1]  # read and written in one step
    seen, first = sdm.touch_prepare(torch.from_numpy(widx).cuda(), torch.from_numpy(ridx).cuda(), N)
    torch.cuda.synchronize()
    want_seen, want_first = _touch_reference(widx, ridx, N)
    assert np.array_equal(seen.cpu().numpy().view(np.uint32), want_seen)
    assert np.array_equal(first.cpu().numpy().view(np.uint64), want_first)
    f = first.cpu().numpy().view(np.uint64)
    one = np.uint64(1)
    assert (f[0, 0, 10, 0] >> one) & one == f[0, 0, 10, 1] & one  # the same row, the same flag


def test_training_degenerate_sizes():
    """T = 0 calls are no-ops that leave every buffer as it was; W = R = 1
    (single slot per step, weights exactly 1) matches the oracle; a selection
    gradient over zero units is a no-op."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["tiny"].with_(B=1, H=2, n=16, d_v=32, T=50, W=1, R=1, seed=9400)
    _train_case(cfg, seed_g=3)

    B, H, N, d_v, W, R = 1, 2, 256, 32, 4, 4
    M = torch.randn((B, H, N, d_v), device="cuda")
    G = torch.randn_like(M)
    M_before, G_before = M.clone(), G.clone()
    e = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device="cuda")  # noqa: E731
    widx, ridx = e(B, H, 0, W, dt=torch.int32), e(B, H, 0, R, dt=torch.int32)
    wk, rw = e(B, H, 0, W), e(B, H, 0, R)
    v, a, b = e(B, H, 0, d_v), e(B, H, 0), e(B, H, 0)
    out, tape = sdm.scan_train(M, widx, wk, ridx, rw, v, a, b)
    gr = sdm.scan_backward(widx, wk, ridx, rw, v, a, b, tape, e(B, H, 0, d_v), G)
    d1, d2 = sdm.select_backward(e(0, 8, dt=torch.int32), e(0, 8), e(0, 8), 16)
    torch.cuda.synchronize()
    seen, first = sdm.touch_prepare(widx, ridx, N)
    torch.cuda.synchronize()
    assert first.numel() == 0 and bool((seen == 0).all())
    assert out.numel() == 0 and tape.numel() == 0 and gr["dv"].numel() == 0
    assert d1.shape == (0, 16) and d2.shape == (0, 16)
    assert torch.equal(M, M_before) and torch.equal(G, G_before)
