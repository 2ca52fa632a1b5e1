"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses, against the CPU oracle on sampled memories (the oracle
recomputes those memories' whole sequences from the same seeded inputs,
regenerated on the host).  Indices bit-exact; values within the bars of
tests/gpu_util.py."""
import numpy as np
import pytest

import oracle
import sdm_inputs as S
from tests.gpu_util import (NAMES, check_selection, check_values, host_inputs, oracle_memory,
                            state_to_host)

pytestmark = pytest.mark.gpu

F32, BF16 = oracle.F32, oracle.BF16


def _dev_inputs(cfg, t0=0, nt=None, B=None):
    import torch

    nt = cfg.T - t0 if nt is None else nt
    B = cfg.B if B is None else B
    d = {}
    for k in NAMES:
        if k in ("alpha", "beta"):
            shape = (B, cfg.H, nt)
        elif k == "v":
            shape = (B, cfg.H, nt, cfg.d_v)
        else:
            shape = (B, cfg.H, nt, cfg.n)
        d[k] = torch.empty(shape, dtype=torch.float32, device="cuda")
        S.device_block(cfg, k, d[k], 0, 0, t0)
    return d


def _free():
    import gc

    import torch

    gc.collect()
    torch.cuda.empty_cache()


def _sampled_units(cfg, g, host_fn, rng, count=64):
    """Oracle selections of random single units (b,h,t), one by one, against
    the GPU selections in g (device tensors [B,H,T,K])."""
    for _ in range(count):
        b = int(rng.integers(cfg.B))
        h = int(rng.integers(cfg.H))
        t = int(rng.integers(g["widx"].shape[2]))
        blk = host_fn(b, h, t)
        wi, ws, wk = oracle.select(blk["s1"], blk["s2"], cfg.W)
        ri, rs, rw = oracle.select(blk["q1"], blk["q2"], cfg.R)
        u = {k: v[b, h, t].cpu().numpy() for k, v in g.items()}
        check_selection(u["widx"], u["wscore"], u["wk"], wi, ws, wk,
                        f"{cfg.name} unit b={b} h={h} t={t} write")
        check_selection(u["ridx"], u["rscore"], u["rw"], ri, rs, rw,
                        f"{cfg.name} unit b={b} h={h} t={t} read")


def test_device_generator_matches_host():
    import torch

    for cfg, name, blk in ((S.CONFIGS["mid"], "s1", (1, 2, 3, 17)),
                           (S.CONFIGS["long"], "q2", (0, 5, 1047976, 600)),
                           (S.CONFIGS["decode"], "alpha", (60, 1, 500, 12)),
                           (S.CONFIGS["small"], "v", (3, 3, 100, 9))):
        b0, h0, t0, nt = blk
        host = S.host_block(cfg, name, b0, 1, h0, 1, t0, nt)
        dev = torch.empty(host.shape, dtype=torch.float32, device="cuda")
        S.device_block(cfg, name, dev, b0, h0, t0)
        assert np.array_equal(dev.cpu().numpy().view(np.uint32), host.view(np.uint32)), name
    M0h = S.host_block(S.CONFIGS["mid"], "M0", h0=3, nh=1, t0=5000, nt=300)
    dev = torch.empty(M0h.shape, dtype=torch.float32, device="cuda")
    S.device_block(S.CONFIGS["mid"], "M0", dev, 0, 3, 5000)
    assert np.array_equal(dev.cpu().numpy().view(np.uint32), M0h.view(np.uint32))


def test_small_config_full():
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["small"]
    host = host_inputs(cfg)
    M0 = S.host_block(cfg, "M0")
    dev = {k: torch.from_numpy(v).cuda() for k, v in host.items()}
    M = sdm.state_init(torch.from_numpy(M0).cuda(), cfg.B)
    widx, wsc, wk = sdm.select(dev["s1"], dev["s2"], cfg.W)
    ridx, rsc, rw = sdm.select(dev["q1"], dev["q2"], cfg.R)
    out = sdm.scan(M, widx, wk, ridx, rw, dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    g = {"widx": widx.cpu().numpy(), "wscore": wsc.cpu().numpy(), "wk": wk.cpu().numpy(),
         "ridx": ridx.cpu().numpy(), "rscore": rsc.cpu().numpy(), "rw": rw.cpu().numpy(),
         "out": out.cpu().numpy()}
    Mh = M.cpu().numpy()
    for b in range(cfg.B):
        for h in range(cfg.H):
            o = oracle_memory(cfg, host, b, h, M0[h], F32, threads=16)
            tag = f"small b={b} h={h}"
            check_selection(g["widx"][b, h], g["wscore"][b, h], g["wk"][b, h], o["widx"],
                            o["wscore"], o["wk"], tag + " write")
            check_selection(g["ridx"][b, h], g["rscore"][b, h], g["rw"][b, h], o["ridx"],
                            o["rscore"], o["rw"], tag + " read")
            check_values(Mh[b, h], o["M"], F32, tag + " M")
            check_values(g["out"][b, h], o["out"], F32, tag + " out")


def test_mid_config_full_size():
    """The benchmark's workload and launch configuration: 64 memories of
    2^20 x 128 fp32 (32 GiB), T = 4096; two memories checked in full against
    the oracle, every memory's selections sampled."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["mid"]
    d = _dev_inputs(cfg)
    M0 = torch.empty((cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, cfg.B)
    widx, wsc, wk = sdm.select(d["s1"], d["s2"], cfg.W)
    ridx, rsc, rw = sdm.select(d["q1"], d["q2"], cfg.R)
    out = sdm.scan(M, widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    gd = {"widx": widx, "wscore": wsc, "wk": wk, "ridx": ridx, "rscore": rsc, "rw": rw}
    for b, h in ((0, 0), (7, 5)):
        g = {k: v[b:b + 1, h:h + 1].cpu().numpy() for k, v in gd.items()}
        host = host_inputs(cfg, b, 1, h, 1)
        M0h = S.host_block(cfg, "M0", h0=h, nh=1)[0]
        o = oracle_memory(cfg, host, 0, 0, M0h, F32, threads=16)
        tag = f"mid b={b} h={h}"
        check_selection(g["widx"][0, 0], g["wscore"][0, 0], g["wk"][0, 0], o["widx"],
                        o["wscore"], o["wk"], tag + " write")
        check_selection(g["ridx"][0, 0], g["rscore"][0, 0], g["rw"][0, 0], o["ridx"],
                        o["rscore"], o["rw"], tag + " read")
        check_values(M[b, h].cpu().numpy(), o["M"], F32, tag + " M")
        check_values(out[b, h].cpu().numpy(), o["out"], F32, tag + " out")
    rng = np.random.default_rng(11)

    def unit(b, h, t):
        return {k: S.host_block(cfg, k, b, 1, h, 1, t, 1)[0, 0, 0] for k in
                ("s1", "s2", "q1", "q2")}

    _sampled_units(cfg, gd, unit, rng, count=128)
    del d, M0, M, widx, wsc, wk, ridx, rsc, rw, out
    _free()


def test_mid_config_bf16_full_size():
    """The mid workload with bf16 state (bench.py --state bf16), all 64
    memories in that launch configuration; two memories checked in full
    against the oracle (indices bit-exact, state and outputs normwise 2e-2)."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["mid"]
    d = _dev_inputs(cfg)
    M0 = torch.empty((cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, cfg.B, torch.bfloat16)
    widx, wsc, wk = sdm.select(d["s1"], d["s2"], cfg.W)
    ridx, rsc, rw = sdm.select(d["q1"], d["q2"], cfg.R)
    out = sdm.scan(M, widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    for b, h in ((3, 1), (5, 6)):
        host = host_inputs(cfg, b, 1, h, 1)
        M0h = S.host_block(cfg, "M0", h0=h, nh=1)[0]
        o = oracle_memory(cfg, host, 0, 0, M0h, BF16, threads=16)
        tag = f"mid bf16 b={b} h={h}"
        check_selection(widx[b, h].cpu().numpy(), wsc[b, h].cpu().numpy(), wk[b, h].cpu().numpy(),
                        o["widx"], o["wscore"], o["wk"], tag + " write")
        check_selection(ridx[b, h].cpu().numpy(), rsc[b, h].cpu().numpy(), rw[b, h].cpu().numpy(),
                        o["ridx"], o["rscore"], o["rw"], tag + " read")
        gm = oracle.bf16_bits_to_f32(state_to_host(M[b, h]))
        check_values(gm, oracle.bf16_bits_to_f32(o["M"]), BF16, tag + " M")
        check_values(out[b, h].cpu().numpy(), o["out"], BF16, tag + " out")
    del d, M0, M, widx, wsc, wk, ridx, rsc, rw, out
    _free()


def test_mid_config_training_full_size():
    """The training step of the mid workload in the benchmark's launch
    configuration (64 memories of 2^20 x 128, T = 4096, gradient table
    zeroed, loss on the outputs): two memories' gradients checked in full
    against the oracle's reverse pass (their tapes and final states too),
    the state left bitwise as the forward ended it for every memory, and dM0
    against the plain sum of the GPU's G."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["mid"]
    B, H, T = cfg.B, cfg.H, cfg.T
    d = _dev_inputs(cfg)
    dout = torch.empty((B, H, T, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "dout", dout)
    M0 = torch.empty((H, cfg.N, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, B)
    widx, _, wk = sdm.select(d["s1"], d["s2"], cfg.W)
    ridx, _, rw = sdm.select(d["q1"], d["q2"], cfg.R)
    out, tape = sdm.scan_train(M, widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"])
    G = torch.zeros_like(M)
    M_end = M.clone()
    gr = sdm.scan_backward(widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"], tape, dout, G)
    dM0 = sdm.state_init_backward(G)
    torch.cuda.synchronize()
    assert torch.equal(M, M_end), "the reverse pass must not touch the state"
    del M_end
    for b, h in ((0, 0), (6, 3)):
        host = host_inputs(cfg, b, 1, h, 1)
        M0h = S.host_block(cfg, "M0", h0=h, nh=1)[0]
        wi, _, wkk = oracle.select(host["s1"][0, 0], host["s2"][0, 0], cfg.W, threads=16)
        ri, _, rww = oracle.select(host["q1"][0, 0], host["q2"][0, 0], cfg.R, threads=16)
        assert np.array_equal(widx[b, h].cpu().numpy(), wi)
        assert np.array_equal(ridx[b, h].cpu().numpy(), ri)
        o = oracle.scan_backward(M0h, wi, wkk, ri, rww, host["v"][0, 0], host["alpha"][0, 0],
                                 host["beta"][0, 0], S.host_block(cfg, "dout", b, 1, h, 1)[0, 0])
        tag = f"mid training b={b} h={h}"
        check_values(out[b, h].cpu().numpy(), oracle.scan(
            M0h.copy(), F32, wi, wkk, ri, rww, host["v"][0, 0], host["alpha"][0, 0],
            host["beta"][0, 0]), F32, tag + " out")
        for k in ("dv", "dwk", "drw", "dalpha", "dbeta"):
            _grad_close(gr[k][b, h].cpu().numpy(), o[k], f"{tag} {k}")
        _grad_close(G[b, h].cpu().numpy(), o["dM0"], tag + " G")
        check_values(M[b, h].cpu().numpy(), o["MT"], F32, tag + " final state")
        check_values(tape[b, h, :, :cfg.W].cpu().numpy(), o["tape"], F32, tag + " tape")
        check_values(tape[b, h, :, cfg.W:].cpu().numpy(), o["rtape"], F32, tag + " read tape")
        del o
    for h in (0, 5):
        want = oracle.state_init_backward(G[:, h:h + 1].cpu().numpy())[0]
        _grad_close(dM0[h].cpu().numpy(), want, f"dM0 h={h}")
    # the sparse mode, as the benchmark runs it, with G never cleared: the same bits for G and
    # dM0; its per-step sums use 16-column tiles (another order of the same additions)
    seen, first = sdm.touch_prepare(widx, ridx, cfg.N)
    Gs = torch.full_like(G, float("nan"))
    gs = sdm.scan_backward(widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"], tape, dout, Gs,
                           first=first)
    dM0s = sdm.state_init_backward(Gs, seen=seen)
    torch.cuda.synchronize()
    for k in gr:  # the same sums over another tile width: the bar against the dense ones
        for b, h in ((0, 0), (6, 3)):
            _grad_close(gs[k][b, h].cpu().numpy(), gr[k][b, h].cpu().numpy(),
                        f"sparse mode {k} b={b} h={h}")
    assert torch.equal(dM0, dM0s), "sparse mode dM0"
    touched = sdm.seen_rows(seen, cfg.N)
    for b in range(B):  # per sequence, to bound the temporaries
        assert torch.equal(G[b][touched[b]], Gs[b][touched[b]]), f"sparse mode G b={b}"
    del seen, first, Gs, gs, dM0s, touched
    del d, dout, M0, M, G, gr, dM0, widx, wk, ridx, rw, out, tape
    _free()


def test_mid_config_fp8_full_size():
    """The mid workload with fp8 E4M3 state, all 64 memories in the
    benchmark's launch configuration.  Memories are independent, so two
    sampled memories run on the oracle's own selections (weights rounded to
    binary32) while the rest keep the GPU's; the sampled memories' state codes
    must equal the oracle's bit for bit, and their outputs meet the fp32 bar."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["mid"]
    d = _dev_inputs(cfg)
    M0 = torch.empty((cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, cfg.B, torch.float8_e4m3fn)
    widx, _, wk = sdm.select(d["s1"], d["s2"], cfg.W)
    ridx, _, rw = sdm.select(d["q1"], d["q2"], cfg.R)
    torch.cuda.synchronize()
    picks = ((1, 2), (7, 7))
    ref = {}
    for b, h in picks:
        host = host_inputs(cfg, b, 1, h, 1)
        wi, _, wkk = oracle.select(host["s1"][0, 0], host["s2"][0, 0], cfg.W, threads=16)
        ri, _, rww = oracle.select(host["q1"][0, 0], host["q2"][0, 0], cfg.R, threads=16)
        wkk, rww = wkk.astype(np.float32), rww.astype(np.float32)
        widx[b, h] = torch.from_numpy(wi).cuda()
        wk[b, h] = torch.from_numpy(wkk).cuda()
        ridx[b, h] = torch.from_numpy(ri).cuda()
        rw[b, h] = torch.from_numpy(rww).cuda()
        ref[b, h] = (host, wi, wkk, ri, rww)
    out = sdm.scan(M, widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    for (b, h), (host, wi, wkk, ri, rww) in ref.items():
        M0h = S.host_block(cfg, "M0", h0=h, nh=1)
        Mo = oracle.state_init(M0h, 1, oracle.FP8)[0, 0].copy()
        oo = oracle.scan(Mo, oracle.FP8, wi, wkk.astype(np.float64), ri, rww.astype(np.float64),
                         host["v"][0, 0], host["alpha"][0, 0], host["beta"][0, 0])
        got = M[b, h].contiguous().view(torch.uint8).cpu().numpy()
        nbad = int((got != Mo).sum())
        assert nbad == 0, f"mid fp8 b={b} h={h}: {nbad} state codes differ"
        check_values(out[b, h].cpu().numpy(), oo, F32, f"mid fp8 b={b} h={h} out")
    del d, M0, M, widx, wk, ridx, rw, out
    _free()


def _grad_close(g, o, what):
    """Gradient bar: normwise per tensor, max|x - y| <= 1e-5 * max(1, max|y|)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    scale = max(1.0, float(np.abs(o).max()))
    err = float(np.abs(g - o).max())
    assert err <= 1e-5 * scale, f"{what}: error {err} vs scale {scale}"


def test_decode_config_full_size():
    """64 x 4 memories of 2^20 x 128 bf16 (64 GiB), 512 single-token calls;
    two memories checked against the oracle over all 512 steps."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["decode"]
    d = _dev_inputs(cfg)
    M0 = torch.empty((cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, cfg.B, torch.bfloat16)
    del M0
    _free()
    outs = torch.empty((cfg.B, cfg.H, cfg.T, cfg.d_v), dtype=torch.float32, device="cuda")
    wids = torch.empty((cfg.B, cfg.H, cfg.T, cfg.W), dtype=torch.int32, device="cuda")
    rids = torch.empty((cfg.B, cfg.H, cfg.T, cfg.R), dtype=torch.int32, device="cuda")
    for t in range(cfg.T):
        step = [d[k][:, :, t].contiguous() for k in NAMES]
        o, wi, ri = sdm.step_decode(M, *step, cfg.W, cfg.R)
        outs[:, :, t] = o
        wids[:, :, t] = wi
        rids[:, :, t] = ri
    torch.cuda.synchronize()
    for b, h in ((0, 0), (63, 3)):
        host = host_inputs(cfg, b, 1, h, 1)
        M0h = S.host_block(cfg, "M0", h0=h, nh=1)[0]
        o = oracle_memory(cfg, host, 0, 0, M0h, BF16, threads=16)
        tag = f"decode b={b} h={h}"
        assert np.array_equal(wids[b, h].cpu().numpy(), o["widx"]), tag + " write indices"
        assert np.array_equal(rids[b, h].cpu().numpy(), o["ridx"]), tag + " read indices"
        check_values(outs[b, h].cpu().numpy(), o["out"], BF16, tag + " out")
        gm = oracle.bf16_bits_to_f32(state_to_host(M[b, h]))
        check_values(gm, oracle.bf16_bits_to_f32(o["M"]), BF16, tag + " M")
    del d, M, outs, wids, rids
    _free()


def test_long_config_full_size():
    """16 memories of 2^20 x 128 fp32, T = 2^20 streamed in chunks of 16384
    steps (the state persists across calls).  Head 7 is checked over the whole
    stream: every selection bit-exact, and the outputs and the final state in
    columns 0..3 (column 0 carries the planted recall pattern) and in one
    column of every other 16-column tile, each at a different lane and
    element position, against the oracle (each column's recurrence involves
    that column alone, so the oracle computes just these).  Other heads'
    selections are sampled."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    cfg = S.CONFIGS["long"]
    C = 16384
    hc = 7
    # column ranges: [0, 4) in tile 0, then column 16k + (5k mod 16) of tile k
    ranges = [(0, 4)] + [(16 * k + (5 * k) % 16, 16 * k + (5 * k) % 16 + 1) for k in range(1, 8)]
    colsel = np.concatenate([np.arange(a, b) for a, b in ranges])
    M0 = torch.empty((cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device="cuda")
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, cfg.B)
    del M0
    _free()
    Mo = S.host_block(cfg, "M0", h0=hc, nh=1)[0].copy()
    rng = np.random.default_rng(12)
    i_s, j_s = S.planted_slot(cfg)
    f_star = i_s * cfg.n + j_s
    recall = None
    for c in range(cfg.T // C):
        t0 = c * C
        d = _dev_inputs(cfg, t0, C)
        widx, wsc, wk = sdm.select(d["s1"], d["s2"], cfg.W)
        ridx, rsc, rw = sdm.select(d["q1"], d["q2"], cfg.R)
        out = sdm.scan(M, widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"])
        torch.cuda.synchronize()
        gd = {"widx": widx, "wscore": wsc, "wk": wk, "ridx": ridx, "rscore": rsc, "rw": rw}
        g = {k: v[0, hc].cpu().numpy() for k, v in gd.items()}
        gout = out[0, hc][:, torch.from_numpy(colsel).cuda()].cpu().numpy()
        host = host_inputs(cfg, 0, 1, hc, 1, t0, C)
        wi, ws, wkk = oracle.select(host["s1"][0, 0], host["s2"][0, 0], cfg.W, threads=16)
        ri, rs, rwk = oracle.select(host["q1"][0, 0], host["q2"][0, 0], cfg.R, threads=16)
        tag = f"long h={hc} chunk {c}"
        check_selection(g["widx"], g["wscore"], g["wk"], wi, ws, wkk, tag + " write")
        check_selection(g["ridx"], g["rscore"], g["rw"], ri, rs, rwk, tag + " read")
        oo = np.zeros((C, cfg.d_v), np.float32)
        for cr in ranges:  # each call computes (and writes back) its columns only
            oracle.scan(Mo, F32, wi, wkk, ri, rwk, host["v"][0, 0], host["alpha"][0, 0],
                        host["beta"][0, 0], cols=cr, out=oo)
        check_values(gout, oo[:, colsel], F32, tag + " out")
        if t0 <= S.PLANT_WRITE_T < t0 + C:
            assert wi[S.PLANT_WRITE_T - t0, 0] == f_star, "planted slot not written"
        if c == cfg.T // C - 1:
            assert ri[-1, 0] == f_star, "planted slot not read back"
            recall = float(gout[-1, 0])

        def unit(b, h, t, t0=t0):
            return {k: S.host_block(cfg, k, b, 1, h, 1, t0 + t, 1)[0, 0, 0] for k in
                    ("s1", "s2", "q1", "q2")}

        _sampled_units(cfg, gd, unit, rng, count=4)
        del d, widx, wsc, wk, ridx, rsc, rw, out
        if c % 16 == 15:
            print(f"long: {c + 1} of {cfg.T // C} chunks checked", flush=True)
    gm = M[0, hc][:, torch.from_numpy(colsel).cuda()].cpu().numpy()
    check_values(gm, Mo[:, colsel], F32, "long final M")
    print(f"long: planted recall amplitude at t=T-1, column 0: {recall:.4f}", flush=True)
    del M
    _free()
