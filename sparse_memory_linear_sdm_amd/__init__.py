"""Sparse Delta Memory (SDM) step on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of libsdm.so (include/sdm.h): it checks
tensor devices, dtypes and contiguity, passes raw device pointers and the
current HIP stream, and raises on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no CPU path and no
fallback -- importing works without the library, but every call raises if
libsdm.so is not built.  PyTorch is used only for device memory and streams.

Calls (same names as the C ABI without the "sdm_" prefix):
  project(X, Wt, n)                      -> (s1, s2, q1, q2, v, alpha, beta)
  select(x1, x2, K)                      -> (idx, score, weight)
  state_init(M0, B, dtype)               -> M
  scan(M, widx, wk, ridx, rw, v, alpha, beta) -> out      (M updated in place)
  step_decode(M, s1, s2, q1, q2, v, alpha, beta, W, R) -> (out, widx, ridx)
Training (fp32 state; selections held fixed):
  scan_train(M, widx, wk, ridx, rw, v, alpha, beta) -> (out, tape)
  scan_backward(widx, wk, ridx, rw, v, alpha, beta, tape, dout, G) -> dict
  scan_backward_noalloc(..., G, out) -> out   (no workspace, no allocation)
Planned scan (fp32 state; few memories, long sequences):
  scan_plan(widx, wk, ridx, rw, N, d_v) -> workspace
  scan_planned(M, v, alpha, beta, workspace) -> out       (M updated in place)
  touch_prepare(widx, ridx, N) -> (seen, first)
  select_backward(idx, weight, dweight, n) -> (dx1, dx2)
  state_init_backward(G) -> dM0
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdm.so")
ABI_VERSION = 6  # the library's sdm_abi_version() this binding is written for

SDM_F32 = 0
SDM_BF16 = 1
SDM_FP8 = 2
STATUS = {0: "SDM_OK", 1: "SDM_ERR_INVALID", 2: "SDM_ERR_UNSUPPORTED", 3: "SDM_ERR_HIP"}

# Every symbol include/sdm.h declares.
EXPORTS = ("sdm_project", "sdm_select", "sdm_state_init", "sdm_scan", "sdm_step_decode", "sdm_scan_train",
           "sdm_scan_backward_workspace_size", "sdm_scan_backward", "sdm_scan_backward_noalloc",
           "sdm_select_backward", "sdm_scan_plan_workspace_size", "sdm_scan_plan",
           "sdm_scan_planned", "sdm_state_init_backward", "sdm_touch_prepare", "sdm_status_string", "sdm_last_error",
           "sdm_abi_version")

_lib = None


class SDMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    """Load libsdm.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m sparse_memory_linear_sdm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.sdm_project.argtypes = [p, p, i32, i32, i32, i32, i32, i32] + [p] * 8
        L.sdm_select.argtypes = [p, p, i64, i32, i32, p, p, p, p]
        L.sdm_state_init.argtypes = [p, i32, p, i32, i32, i64, i32, p]
        L.sdm_scan.argtypes = [p, i32, i32, i32, i64, i32, i64, i32, i32] + [p] * 9
        L.sdm_step_decode.argtypes = [p, i32, i32, i32, i32, i32, i32, i32] + [p] * 11
        L.sdm_scan_train.argtypes = [p, i32, i32, i64, i32, i64, i32, i32] + [p] * 10
        L.sdm_scan_backward_workspace_size.argtypes = [i32, i32, i32, i64, i32, i32]
        L.sdm_scan_backward_workspace_size.restype = ctypes.c_size_t
        L.sdm_scan_backward.argtypes = ([i32, i32, i64, i32, i64, i32, i32] + [p] * 17 +
                                        [ctypes.c_size_t, p])
        L.sdm_scan_backward_noalloc.argtypes = [i32, i32, i64, i32, i64, i32, i32] + [p] * 17
        L.sdm_touch_prepare.argtypes = [i32, i32, i64, i64, i32, i32, p, p, p, p, p]
        L.sdm_scan_plan_workspace_size.argtypes = [i32, i32, i32, i64]
        L.sdm_scan_plan_workspace_size.restype = ctypes.c_size_t
        L.sdm_scan_plan.argtypes = [i32, i32, i64, i32, i64, i32, i32] + [p] * 5 + [ctypes.c_size_t, p]
        L.sdm_scan_planned.argtypes = [p, i32, i32, i64, i32, i64] + [p] * 5 + [ctypes.c_size_t, p]
        L.sdm_select_backward.argtypes = [p, p, p, i64, i32, i32, p, p, p]
        L.sdm_state_init_backward.argtypes = [p, i32, i32, i64, i32, p, p, p]
        for f in ("sdm_project", "sdm_select", "sdm_state_init", "sdm_scan", "sdm_step_decode",
                  "sdm_abi_version", "sdm_scan_train", "sdm_scan_backward",
                  "sdm_scan_backward_noalloc",
                  "sdm_select_backward", "sdm_state_init_backward", "sdm_touch_prepare",
                  "sdm_scan_plan", "sdm_scan_planned"):
            getattr(L, f).restype = ctypes.c_int
        L.sdm_status_string.argtypes = [i32]
        L.sdm_status_string.restype = ctypes.c_char_p
        L.sdm_last_error.argtypes = []
        L.sdm_last_error.restype = ctypes.c_char_p
        if L.sdm_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI {L.sdm_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise SDMError(rc, lib().sdm_last_error().decode())


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _arg(t, dtype, shape, name):
    """Check one tensor argument: type, exact shape (the one the call derives
    from its other arguments), dtype (one dtype or a tuple of allowed ones;
    None = any) and contiguity.  Returns (name, tensor) for _gpu().  A
    mismatch raises ValueError (TypeError for a non-tensor): the kernels
    index every buffer by sizes taken from other arguments, so a short or
    strided buffer must never reach them.  Every argument of a call passes
    these checks before any device check, so a call fails on the first bad
    shape whatever device its tensors are on."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if dtype is not None and t.dtype not in allowed:
        raise ValueError(f"{name} must be {' or '.join(map(str, allowed))}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return (name, t)


def _gpu(*args):
    """Device pointers of checked arguments ((name, tensor) pairs from _arg,
    or None for an absent optional one): every tensor must be on the GPU, all
    on the same device."""
    dev = None
    ptrs = []
    for a in args:
        if a is None:
            ptrs.append(None)
            continue
        name, t = a
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call's other tensors on {dev}")
        ptrs.append(t.data_ptr())
    return ptrs


def _state_dtype(M):
    import torch

    if M.dtype == torch.float32:
        return SDM_F32
    if M.dtype == torch.bfloat16:
        return SDM_BF16
    if M.dtype == torch.float8_e4m3fn:
        return SDM_FP8
    raise ValueError(f"state must be float32, bfloat16 or float8_e4m3fn, got {M.dtype}")


def _state_types():
    import torch

    return (torch.float32, torch.bfloat16, torch.float8_e4m3fn)


def _units(lead):
    units = 1
    for s in lead:
        units *= s
    return units


def project(X, Wt, n: int, out=None, stream=None):
    """Token projections on the matrix cores: X [B, T, d_model] bfloat16,
    Wt [H, P, d_model] bfloat16 with P = 4n + d_v + 2 (rows s1, s2, q1, q2,
    v, alpha, beta of each head).  Returns fp32 (s1, s2, q1, q2) [B, H, T, n],
    v [B, H, T, d_v], alpha, beta [B, H, T] (the gates through the logistic
    function).  out = that 7-tuple writes into caller tensors."""
    import torch

    bf16, f32 = torch.bfloat16, torch.float32
    if X.dim() != 3 or Wt.dim() != 3:
        raise ValueError("X must be [B, T, d_model] and Wt [H, P, d_model]")
    B, T, d_model = X.shape
    H, P = Wt.shape[0], Wt.shape[1]
    d_v = P - 4 * n - 2
    if n < 1 or d_v < 1:
        raise ValueError(f"Wt has P={P} rows per head: too few for n={n} (P = 4n + d_v + 2)")
    shapes = [(B, H, T, n)] * 4 + [(B, H, T, d_v), (B, H, T), (B, H, T)]
    names = ("s1", "s2", "q1", "q2", "v", "alpha", "beta")
    if out is None:
        out = tuple(torch.empty(sh, dtype=f32, device=X.device) for sh in shapes)
    if len(out) != 7:
        raise ValueError("out must hold 7 tensors (s1, s2, q1, q2, v, alpha, beta)")
    ptrs = _gpu(_arg(X, bf16, (B, T, d_model), "X"), _arg(Wt, bf16, (H, P, d_model), "Wt"),
                *(_arg(t, f32, sh, nm) for t, sh, nm in zip(out, shapes, names)))
    _check(lib().sdm_project(ptrs[0], ptrs[1], B, T, d_model, H, n, d_v, *ptrs[2:],
                             _stream(stream)))
    return tuple(out)


def select(x1, x2, K: int, out=None, stream=None):
    """Top-K slots of the product-key table for every leading index of
    x1, x2 [..., n]: returns idx int32, score fp32, weight fp32 [..., K].
    out = (idx, score, weight) writes into caller tensors (score may be
    None)."""
    import torch

    f32 = torch.float32
    shape = tuple(x1.shape)
    if len(shape) < 1:
        raise ValueError("x1 and x2 must have a last dimension n")
    n, lead = shape[-1], shape[:-1]
    if out is None:
        idx = torch.empty(lead + (K,), dtype=torch.int32, device=x1.device)
        score = torch.empty(lead + (K,), dtype=f32, device=x1.device)
        weight = torch.empty(lead + (K,), dtype=f32, device=x1.device)
    else:
        idx, score, weight = out
    p1, p2, pi, ps, pw = _gpu(
        _arg(x1, f32, shape, "x1"), _arg(x2, f32, shape, "x2"),
        _arg(idx, torch.int32, lead + (K,), "idx"),
        None if score is None else _arg(score, f32, lead + (K,), "score"),
        _arg(weight, f32, lead + (K,), "weight"))
    _check(lib().sdm_select(p1, p2, _units(lead), n, K, pi, ps, pw, _stream(stream)))
    return idx, score, weight


def state_init(M0, B: int, dtype=None, out=None, stream=None):
    """M [B,H,N,d_v] = M0 [H,N,d_v] for every b (fp32, bf16 or fp8 E4M3 state).
    out = an existing state tensor to fill (its dtype is the state type)."""
    import torch

    if M0.dim() != 3:
        raise ValueError(f"M0 must be [H, N, d_v], got {tuple(M0.shape)}")
    H, N, d_v = M0.shape
    a0 = _arg(M0, torch.float32, (H, N, d_v), "M0")
    if out is None:
        dtype = torch.float32 if dtype is None else dtype
        M = torch.empty((B, H, N, d_v), dtype=dtype, device=M0.device)
    else:
        M = out
    p0, pm = _gpu(a0, _arg(M, _state_types(), (B, H, N, d_v), "M"))
    _check(lib().sdm_state_init(pm, _state_dtype(M), p0, B, H, N, d_v, _stream(stream)))
    return M


def _scan_shapes(M, widx, ridx):
    if M.dim() != 4:
        raise ValueError(f"the state must be [B, H, N, d_v], got {tuple(M.shape)}")
    if widx.dim() != 4 or ridx.dim() != 4:
        raise ValueError("widx and ridx must be [B, H, T, W] and [B, H, T, R]")
    B, H, N, d_v = M.shape
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    return B, H, N, d_v, T, W, R


def _scan_args(B, H, T, W, R, d_v, widx, wk, ridx, rw, v, alpha, beta):
    import torch

    f32 = torch.float32
    return [_arg(widx, torch.int32, (B, H, T, W), "widx"), _arg(wk, f32, (B, H, T, W), "wk"),
            _arg(ridx, torch.int32, (B, H, T, R), "ridx"), _arg(rw, f32, (B, H, T, R), "rw"),
            _arg(v, f32, (B, H, T, d_v), "v"), _arg(alpha, f32, (B, H, T), "alpha"),
            _arg(beta, f32, (B, H, T), "beta")]


def scan(M, widx, wk, ridx, rw, v, alpha, beta, out=None, stream=None):
    """T steps of write + read on M [B,H,N,d_v] in place.  widx, wk
    [B,H,T,W]; ridx, rw [B,H,T,R]; v [B,H,T,d_v]; alpha, beta [B,H,T].
    Returns out [B,H,T,d_v] fp32."""
    import torch

    B, H, N, d_v, T, W, R = _scan_shapes(M, widx, ridx)
    am = _arg(M, _state_types(), (B, H, N, d_v), "M")
    ins = _scan_args(B, H, T, W, R, d_v, widx, wk, ridx, rw, v, alpha, beta)
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=torch.float32, device=M.device)
    pm, *ptrs = _gpu(am, *ins, _arg(out, torch.float32, (B, H, T, d_v), "out"))
    _check(lib().sdm_scan(pm, _state_dtype(M), B, H, N, d_v, T, W, R, *ptrs, _stream(stream)))
    return out


def step_decode(M, s1, s2, q1, q2, v, alpha, beta, W: int, R: int, out=None, want_idx=True,
                stream=None):
    """One token per (b,h): selections, write and read fused.  s1.. [B,H,n];
    v [B,H,d_v]; alpha, beta [B,H].  Returns (out [B,H,d_v], widx, ridx)."""
    import torch

    if M.dim() != 4:
        raise ValueError(f"the state must be [B, H, N, d_v], got {tuple(M.shape)}")
    B, H, N, d_v = M.shape
    n = s1.shape[-1]
    if n * n != N:
        raise ValueError(f"M has {N} rows but the halves give n*n = {n * n}")
    f32 = torch.float32
    ins = [_arg(M, _state_types(), (B, H, N, d_v), "M")]
    ins += [_arg(t, f32, (B, H, n), nm) for nm, t in
            (("s1", s1), ("s2", s2), ("q1", q1), ("q2", q2))]
    ins += [_arg(v, f32, (B, H, d_v), "v"), _arg(alpha, f32, (B, H), "alpha"),
            _arg(beta, f32, (B, H), "beta")]
    if out is None:
        out = torch.empty((B, H, d_v), dtype=f32, device=M.device)
    ins.append(_arg(out, f32, (B, H, d_v), "out"))
    widx = ridx = None
    if want_idx:
        widx = torch.empty((B, H, W), dtype=torch.int32, device=M.device)
        ridx = torch.empty((B, H, R), dtype=torch.int32, device=M.device)
    pm, *ptrs = _gpu(*ins)
    _check(lib().sdm_step_decode(pm, _state_dtype(M), B, H, n, d_v, W, R, *ptrs,
                                 widx.data_ptr() if widx is not None else None,
                                 ridx.data_ptr() if ridx is not None else None,
                                 _stream(stream)))
    return out, widx, ridx


def scan_train(M, widx, wk, ridx, rw, v, alpha, beta, out=None, tape=None, stream=None):
    """scan() on an fp32 state that also keeps, per step, the W pre-write rows
    and the R rows the read used: returns (out [B,H,T,d_v],
    tape [B,H,T,W+R,d_v])."""
    import torch

    f32 = torch.float32
    B, H, N, d_v, T, W, R = _scan_shapes(M, widx, ridx)
    am = _arg(M, f32, (B, H, N, d_v), "M")
    ins = _scan_args(B, H, T, W, R, d_v, widx, wk, ridx, rw, v, alpha, beta)
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=f32, device=M.device)
    if tape is None:
        tape = torch.empty((B, H, T, W + R, d_v), dtype=f32, device=M.device)
    pm, *ptrs = _gpu(am, *ins, _arg(out, f32, (B, H, T, d_v), "out"),
                     _arg(tape, f32, (B, H, T, W + R, d_v), "tape"))
    _check(lib().sdm_scan_train(pm, B, H, N, d_v, T, W, R, *ptrs, _stream(stream)))
    return out, tape


def scan_backward(widx, wk, ridx, rw, v, alpha, beta, tape, dout, G, workspace=None,
                  first=None, stream=None):
    """Reverse pass from the tape of scan_train (the state is not needed):
    G (dL/d final state, [B,H,N,d_v]) becomes dL/d initial state in place.
    With first (from touch_prepare) the final-state gradient is taken as
    zero and G need not be cleared; only the rows the steps select are
    written.  Returns dict dv [B,H,T,d_v], dwk [B,H,T,W], drw [B,H,T,R],
    dalpha, dbeta [B,H,T]."""
    import torch

    f32 = torch.float32
    B, H, N, d_v, T, W, R = _scan_shapes(G, widx, ridx)
    ins = _scan_args(B, H, T, W, R, d_v, widx, wk, ridx, rw, v, alpha, beta)
    ins += [_arg(tape, f32, (B, H, T, W + R, d_v), "tape"),
            _arg(dout, f32, (B, H, T, d_v), "dout"), _arg(G, f32, (B, H, N, d_v), "G")]
    af = None if first is None else _arg(first, torch.int64, (B, H, T, 2), "first")
    aw = None if workspace is None else _arg(workspace, None, None, "workspace")
    dev = G.device
    o = {"dv": torch.empty((B, H, T, d_v), dtype=f32, device=dev),
         "dwk": torch.empty((B, H, T, W), dtype=f32, device=dev),
         "drw": torch.empty((B, H, T, R), dtype=f32, device=dev),
         "dalpha": torch.empty((B, H, T), dtype=f32, device=dev),
         "dbeta": torch.empty((B, H, T), dtype=f32, device=dev)}
    ptrs = _gpu(*ins, *(_arg(o[k], f32, None, k) for k in ("dv", "dwk", "drw", "dalpha", "dbeta")),
                af, aw)
    need = int(lib().sdm_scan_backward_workspace_size(B, H, d_v, T, W, R))
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=f32, device=dev)
        ptrs[-1] = workspace.data_ptr()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().sdm_scan_backward(B, H, N, d_v, T, W, R, *ptrs, nbytes, _stream(stream)))
    return o


def scan_backward_noalloc(widx, wk, ridx, rw, v, alpha, beta, tape, dout, G, out, first=None,
                          stream=None):
    """scan_backward() without a workspace and without any allocation: the
    library's per-GPU static scratch buffer (64 MiB) holds the partial sums,
    and out is a dict of caller tensors dv [B,H,T,d_v], dwk [B,H,T,W],
    drw [B,H,T,R], dalpha, dbeta [B,H,T] (fp32).  Calls on one GPU share the
    buffer and must not overlap in time.  Returns out."""
    import torch

    f32 = torch.float32
    B, H, N, d_v, T, W, R = _scan_shapes(G, widx, ridx)
    ins = _scan_args(B, H, T, W, R, d_v, widx, wk, ridx, rw, v, alpha, beta)
    ins += [_arg(tape, f32, (B, H, T, W + R, d_v), "tape"),
            _arg(dout, f32, (B, H, T, d_v), "dout"), _arg(G, f32, (B, H, N, d_v), "G")]
    shapes = {"dv": (B, H, T, d_v), "dwk": (B, H, T, W), "drw": (B, H, T, R),
              "dalpha": (B, H, T), "dbeta": (B, H, T)}
    ins += [_arg(out[k], f32, shp, k) for k, shp in shapes.items()]
    af = None if first is None else _arg(first, torch.int64, (B, H, T, 2), "first")
    ptrs = _gpu(*ins, af)
    _check(lib().sdm_scan_backward_noalloc(B, H, N, d_v, T, W, R, *ptrs, _stream(stream)))
    return out


def touch_prepare(widx, ridx, N: int, seen=None, first=None, stream=None):
    """Bookkeeping of the sparse training mode: seen [B,H,ceil(N/32)] int32
    (the bits of the uint32 words: row r is selected at some step) and first
    [B,H,T,2] int64 (the bits of the uint64 masks of slots whose row is
    selected for the last time at that step).  N <= 2^20."""
    import torch

    if widx.dim() != 4 or ridx.dim() != 4:
        raise ValueError("widx and ridx must be [B, H, T, W] and [B, H, T, R]")
    B, H, T, W = widx.shape
    R = ridx.shape[3]
    ins = [_arg(widx, torch.int32, (B, H, T, W), "widx"),
           _arg(ridx, torch.int32, (B, H, T, R), "ridx")]
    if seen is None:
        seen = torch.empty((B, H, (N + 31) // 32), dtype=torch.int32, device=widx.device)
    if first is None:
        first = torch.empty((B, H, T, 2), dtype=torch.int64, device=widx.device)
    ptrs = _gpu(*ins, _arg(seen, torch.int32, (B, H, (N + 31) // 32), "seen"),
                _arg(first, torch.int64, (B, H, T, 2), "first"))
    _check(lib().sdm_touch_prepare(B, H, N, T, W, R, *ptrs, _stream(stream)))
    return seen, first


def seen_rows(seen, N: int):
    """The seen bitmap of touch_prepare as a [B,H,N] bool tensor."""
    import torch

    shifts = torch.arange(32, dtype=torch.int32, device=seen.device)
    bits = (seen.unsqueeze(-1) >> shifts) & 1
    return bits.reshape(seen.shape[0], seen.shape[1], -1)[:, :, :N].bool()


def select_backward(idx, weight, dweight, n: int, stream=None):
    """Gradient of the selection weights back to the halves: idx, weight,
    dweight [..., K] -> (dx1, dx2) [..., n] fp32."""
    import torch

    f32 = torch.float32
    shape = tuple(idx.shape)
    if len(shape) < 1:
        raise ValueError("idx must have a last dimension K")
    K, lead = shape[-1], shape[:-1]
    ins = [_arg(idx, torch.int32, shape, "idx"), _arg(weight, f32, shape, "weight"),
           _arg(dweight, f32, shape, "dweight")]
    dx1 = torch.empty(lead + (n,), dtype=f32, device=idx.device)
    dx2 = torch.empty(lead + (n,), dtype=f32, device=idx.device)
    ptrs = _gpu(*ins, _arg(dx1, f32, None, "dx1"), _arg(dx2, f32, None, "dx2"))
    _check(lib().sdm_select_backward(ptrs[0], ptrs[1], ptrs[2], _units(lead), n, K, ptrs[3],
                                     ptrs[4], _stream(stream)))
    return dx1, dx2


def state_init_backward(G, out=None, seen=None, stream=None):
    """dM0 [H,N,d_v] = sum over b of G [B,H,N,d_v]; with seen (from
    touch_prepare) only the rows each sequence selected count."""
    import torch

    f32 = torch.float32
    if G.dim() != 4:
        raise ValueError(f"G must be [B, H, N, d_v], got {tuple(G.shape)}")
    B, H, N, d_v = G.shape
    ag = _arg(G, f32, (B, H, N, d_v), "G")
    as_ = None if seen is None else _arg(seen, torch.int32, (B, H, (N + 31) // 32), "seen")
    dM0 = torch.empty((H, N, d_v), dtype=f32, device=G.device) if out is None else out
    pg, ps, po = _gpu(ag, as_, _arg(dM0, f32, (H, N, d_v), "dM0"))
    _check(lib().sdm_state_init_backward(pg, B, H, N, d_v, ps, po, _stream(stream)))
    return dM0


def scan_plan_workspace_size(B: int, H: int, d_v: int, T: int) -> int:
    """Bytes of workspace scan_plan / scan_planned need (0: unsupported)."""
    return int(lib().sdm_scan_plan_workspace_size(B, H, d_v, T))


def scan_plan(widx, wk, ridx, rw, N: int, d_v: int, workspace=None, stream=None):
    """Plan the steps of a planned scan on memories of N rows of d_v fp32
    columns: widx, wk [B,H,T,W]; ridx, rw [B,H,T,R].  Returns the workspace
    (a uint8 device tensor, allocated when None) for scan_planned."""
    import torch

    if widx.dim() != 4 or ridx.dim() != 4:
        raise ValueError("widx and ridx must be [B, H, T, W] and [B, H, T, R]")
    B, H, T, W = widx.shape
    R = ridx.shape[3]
    f32 = torch.float32
    ins = [_arg(widx, torch.int32, (B, H, T, W), "widx"), _arg(wk, f32, (B, H, T, W), "wk"),
           _arg(ridx, torch.int32, (B, H, T, R), "ridx"), _arg(rw, f32, (B, H, T, R), "rw")]
    need = scan_plan_workspace_size(B, H, d_v, T)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=widx.device)
    ptrs = _gpu(*ins, _arg(workspace, None, None, "workspace"))
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().sdm_scan_plan(B, H, N, d_v, T, W, R, *ptrs, nbytes, _stream(stream)))
    return workspace


def scan_planned(M, v, alpha, beta, workspace, out=None, stream=None):
    """Run the steps scan_plan wrote into workspace on the fp32 state M
    [B,H,N,d_v] in place; v [B,H,T,d_v]; alpha, beta [B,H,T].  Returns out
    [B,H,T,d_v] fp32."""
    import torch

    if M.dim() != 4 or v.dim() != 4:
        raise ValueError("M and v must be [B, H, N, d_v] and [B, H, T, d_v]")
    B, H, N, d_v = M.shape
    T = v.shape[2]
    f32 = torch.float32
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=f32, device=M.device)
    ptrs = _gpu(_arg(M, f32, (B, H, N, d_v), "M"), _arg(v, f32, (B, H, T, d_v), "v"),
                _arg(alpha, f32, (B, H, T), "alpha"), _arg(beta, f32, (B, H, T), "beta"),
                _arg(out, f32, (B, H, T, d_v), "out"), _arg(workspace, None, None, "workspace"))
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().sdm_scan_planned(ptrs[0], B, H, N, d_v, T, *ptrs[1:], nbytes, _stream(stream)))
    return out
