"""sdm_scan_backward_noalloc (the reverse pass on the library's per-GPU
static scratch buffer, for callers that cannot allocate) against
sdm_scan_backward with a caller workspace, through the C ABI: two calls in
a row, the second smaller than the first (the buffer keeps the first call's
contents), each compared bit for bit on every output, in the dense and the
sparse mode."""
import ctypes

import numpy as np
import pytest

import sdm_inputs as S

pytestmark = pytest.mark.gpu


def _case(cfg, sparse):
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    names = ("s1", "s2", "q1", "q2", "v", "alpha", "beta")
    d = {k: torch.from_numpy(np.ascontiguousarray(S.host_block(cfg, k))).cuda() for k in names}
    M0 = torch.from_numpy(S.host_block(cfg, "M0")).cuda()
    widx, _, wk = sdm.select(d["s1"], d["s2"], cfg.W)
    ridx, _, rw = sdm.select(d["q1"], d["q2"], cfg.R)
    M = sdm.state_init(M0, cfg.B)
    args = (widx, wk, ridx, rw, d["v"], d["alpha"], d["beta"])
    out, tape = sdm.scan_train(M, *args)
    g = torch.Generator().manual_seed(cfg.seed)
    dout = torch.randn(out.shape, generator=g).cuda()
    first = sdm.touch_prepare(widx, ridx, cfg.N)[1] if sparse else None
    G0 = torch.randn(M.shape, generator=g).cuda()  # dL/dM_T (dense mode), junk (sparse)
    return args, tape, dout, first, G0


def _outputs(shape_src, widx, ridx):
    import torch

    B, H, T, W = widx.shape
    R = ridx.shape[3]
    d_v = shape_src.shape[3]
    dev = widx.device
    shapes = {"dv": (B, H, T, d_v), "dwk": (B, H, T, W), "drw": (B, H, T, R),
              "dalpha": (B, H, T), "dbeta": (B, H, T)}
    return {k: torch.full(s, float("nan"), device=dev) for k, s in shapes.items()}


def _noalloc_call(args, tape, dout, G, o, first):
    """sdm_scan_backward_noalloc through the C ABI (ctypes)."""
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    widx, wk, ridx, rw, v, alpha, beta = args
    B, H, N, d_v = G.shape
    T, W, R = widx.shape[2], widx.shape[3], ridx.shape[3]
    ptr = [t.data_ptr() for t in (widx, wk, ridx, rw, v, alpha, beta, tape, dout, G, o["dv"],
                                  o["dwk"], o["drw"], o["dalpha"], o["dbeta"])]
    rc = sdm.lib().sdm_scan_backward_noalloc(
        B, H, N, d_v, T, W, R, *ptr, None if first is None else first.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, sdm.lib().sdm_last_error().decode()


def _compare(cfg, sparse):
    import torch

    import sparse_memory_linear_sdm_amd as sdm

    args, tape, dout, first, G0 = _case(cfg, sparse)
    G_ref, G_new = G0.clone(), G0.clone()
    ref = sdm.scan_backward(*args, tape, dout, G_ref, first=first)
    new = _outputs(G_new, args[0], args[2])
    _noalloc_call(args, tape, dout, G_new, new, first)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k].view(torch.int32), new[k].view(torch.int32)), \
            f"{cfg.name} {k} differs"
    assert torch.equal(G_ref.view(torch.int32), G_new.view(torch.int32)), f"{cfg.name} G differs"
    assert torch.isfinite(new["dv"]).all() and torch.isfinite(new["dalpha"]).all()


@pytest.mark.parametrize("sparse", [False, True])
def test_noalloc_backward_matches_workspace_backward_twice(sparse):
    big = S.CONFIGS["tiny"].with_(B=2, H=3, n=32, d_v=64, T=300, W=16, R=16, seed=41)
    small = S.CONFIGS["tiny"].with_(B=1, H=2, n=16, d_v=32, T=50, W=8, R=12, seed=42)
    _compare(big, sparse)    # first call on this GPU's buffer
    _compare(small, sparse)  # second call: a smaller input, the buffer holds the first's data


def test_noalloc_backward_rejects_sizes_above_its_buffer():
    import sparse_memory_linear_sdm_amd as sdm

    L = sdm.lib()
    # mid training sizes: 64 memories x 4096 steps x 8 tiles x 129 sums x 4 B > 64 MiB
    assert L.sdm_scan_backward_workspace_size(8, 8, 128, 4096, 64, 64) > (64 << 20)
    fake = 1 << 20  # never dereferenced: the call returns before any launch
    rc = L.sdm_scan_backward_noalloc(8, 8, 1 << 20, 128, 4096, 64, 64, *([fake] * 15), None,
                                     None)
    assert rc == 2 and b"static buffer" in L.sdm_last_error()
