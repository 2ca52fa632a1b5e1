"""Sparse Delta Memory (SDM) step on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of libsdm.so (include/sdm.h): it checks
tensor devices, dtypes and contiguity, passes raw device pointers and the
current HIP stream, and raises on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no CPU path and no
fallback -- importing works without the library, but every call raises if
libsdm.so is not built.  PyTorch is used only for device memory and streams.

Calls (same names as the C ABI without the "sdm_" prefix):
  select(x1, x2, K)                      -> (idx, score, weight)
  state_init(M0, B, dtype)               -> M
  scan(M, widx, wk, ridx, rw, v, alpha, beta) -> out      (M updated in place)
  step_decode(M, s1, s2, q1, q2, v, alpha, beta, W, R) -> (out, widx, ridx)
Training (fp32 state; selections held fixed):
  scan_train(M, widx, wk, ridx, rw, v, alpha, beta) -> (out, tape)
  scan_backward(M, widx, wk, ridx, rw, v, alpha, beta, tape, dout, G) -> dict
  select_backward(idx, weight, dweight, n) -> (dx1, dx2)
  state_init_backward(G) -> dM0
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdm.so")
ABI_VERSION = 3  # the library's sdm_abi_version() this binding is written for

SDM_F32 = 0
SDM_BF16 = 1
SDM_FP8 = 2
STATUS = {0: "SDM_OK", 1: "SDM_ERR_INVALID", 2: "SDM_ERR_UNSUPPORTED", 3: "SDM_ERR_HIP"}

# Every symbol include/sdm.h declares.
EXPORTS = ("sdm_select", "sdm_state_init", "sdm_scan", "sdm_step_decode", "sdm_scan_train",
           "sdm_scan_backward_workspace_size", "sdm_scan_backward", "sdm_select_backward",
           "sdm_state_init_backward", "sdm_touch_prepare", "sdm_status_string", "sdm_last_error",
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
        L.sdm_select.argtypes = [p, p, i64, i32, i32, p, p, p, p]
        L.sdm_state_init.argtypes = [p, i32, p, i32, i32, i64, i32, p]
        L.sdm_scan.argtypes = [p, i32, i32, i32, i64, i32, i64, i32, i32] + [p] * 9
        L.sdm_step_decode.argtypes = [p, i32, i32, i32, i32, i32, i32, i32] + [p] * 11
        L.sdm_scan_train.argtypes = [p, i32, i32, i64, i32, i64, i32, i32] + [p] * 10
        L.sdm_scan_backward_workspace_size.argtypes = [i32, i32, i32, i64, i32, i32]
        L.sdm_scan_backward_workspace_size.restype = ctypes.c_size_t
        L.sdm_scan_backward.argtypes = ([i32, i32, i64, i32, i64, i32, i32] + [p] * 17 +
                                        [ctypes.c_size_t, p])
        L.sdm_touch_prepare.argtypes = [i32, i32, i64, i64, i32, i32, p, p, p, p, p]
        L.sdm_select_backward.argtypes = [p, p, p, i64, i32, i32, p, p, p]
        L.sdm_state_init_backward.argtypes = [p, i32, i32, i64, i32, p, p, p]
        for f in ("sdm_select", "sdm_state_init", "sdm_scan", "sdm_step_decode",
                  "sdm_abi_version", "sdm_scan_train", "sdm_scan_backward",
                  "sdm_select_backward", "sdm_state_init_backward", "sdm_touch_prepare"):
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


def _dev(t, dtype, name, ndim=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    return t.data_ptr()


def _state_dtype(M):
    import torch

    if M.dtype == torch.float32:
        return SDM_F32
    if M.dtype == torch.bfloat16:
        return SDM_BF16
    if M.dtype == torch.float8_e4m3fn:
        return SDM_FP8
    raise ValueError(f"state must be float32, bfloat16 or float8_e4m3fn, got {M.dtype}")


def select(x1, x2, K: int, out=None, stream=None):
    """Top-K slots of the product-key table for every leading index of
    x1, x2 [..., n]: returns idx int32, score fp32, weight fp32 [..., K]."""
    import torch

    if x1.shape != x2.shape:
        raise ValueError("x1 and x2 must have the same shape")
    n = x1.shape[-1]
    lead = tuple(x1.shape[:-1])
    units = 1
    for s in lead:
        units *= s
    if out is None:
        idx = torch.empty(lead + (K,), dtype=torch.int32, device=x1.device)
        score = torch.empty(lead + (K,), dtype=torch.float32, device=x1.device)
        weight = torch.empty(lead + (K,), dtype=torch.float32, device=x1.device)
    else:
        idx, score, weight = out
    sp = score.data_ptr() if score is not None else None
    _check(lib().sdm_select(_dev(x1, torch.float32, "x1"), _dev(x2, torch.float32, "x2"), units,
                            n, K, _dev(idx, torch.int32, "idx"), sp,
                            _dev(weight, torch.float32, "weight"), _stream(stream)))
    return idx, score, weight


def state_init(M0, B: int, dtype=None, out=None, stream=None):
    """M [B,H,N,d_v] = M0 [H,N,d_v] for every b (fp32, bf16 or fp8 E4M3 state)."""
    import torch

    dtype = torch.float32 if dtype is None else dtype
    H, N, d_v = M0.shape
    M = torch.empty((B, H, N, d_v), dtype=dtype, device=M0.device) if out is None else out
    _check(lib().sdm_state_init(M.data_ptr(), _state_dtype(M), _dev(M0, torch.float32, "M0", 3),
                                B, H, N, d_v, _stream(stream)))
    return M


def scan(M, widx, wk, ridx, rw, v, alpha, beta, out=None, stream=None):
    """T steps of write + read on M [B,H,N,d_v] in place.  widx, wk
    [B,H,T,W]; ridx, rw [B,H,T,R]; v [B,H,T,d_v]; alpha, beta [B,H,T].
    Returns out [B,H,T,d_v] fp32."""
    import torch

    B, H, N, d_v = M.shape
    if not M.is_contiguous():
        raise ValueError("M must be contiguous")
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    if tuple(v.shape) != (B, H, T, d_v):
        raise ValueError(f"v must be {(B, H, T, d_v)}, got {tuple(v.shape)}")
    for name, t, shp in (("widx", widx, (B, H, T, W)), ("wk", wk, (B, H, T, W)),
                         ("ridx", ridx, (B, H, T, R)), ("rw", rw, (B, H, T, R)),
                         ("alpha", alpha, (B, H, T)), ("beta", beta, (B, H, T))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {shp}, got {tuple(t.shape)}")
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=torch.float32, device=M.device)
    _check(lib().sdm_scan(M.data_ptr(), _state_dtype(M), B, H, N, d_v, T, W, R,
                          _dev(widx, torch.int32, "widx"), _dev(wk, torch.float32, "wk"),
                          _dev(ridx, torch.int32, "ridx"), _dev(rw, torch.float32, "rw"),
                          _dev(v, torch.float32, "v"), _dev(alpha, torch.float32, "alpha"),
                          _dev(beta, torch.float32, "beta"), _dev(out, torch.float32, "out"),
                          _stream(stream)))
    return out


def step_decode(M, s1, s2, q1, q2, v, alpha, beta, W: int, R: int, out=None, want_idx=True,
                stream=None):
    """One token per (b,h): selections, write and read fused.  s1.. [B,H,n];
    v [B,H,d_v]; alpha, beta [B,H].  Returns (out [B,H,d_v], widx, ridx)."""
    import torch

    B, H, N, d_v = M.shape
    n = s1.shape[-1]
    if n * n != N:
        raise ValueError(f"M has {N} rows but the halves give n*n = {n * n}")
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.float32, device=M.device)
    widx = ridx = None
    if want_idx:
        widx = torch.empty((B, H, W), dtype=torch.int32, device=M.device)
        ridx = torch.empty((B, H, R), dtype=torch.int32, device=M.device)
    ptrs = [_dev(t, torch.float32, nm) for nm, t in
            (("s1", s1), ("s2", s2), ("q1", q1), ("q2", q2), ("v", v), ("alpha", alpha),
             ("beta", beta), ("out", out))]
    _check(lib().sdm_step_decode(M.data_ptr(), _state_dtype(M), B, H, n, d_v, W, R, *ptrs,
                                 widx.data_ptr() if widx is not None else None,
                                 ridx.data_ptr() if ridx is not None else None,
                                 _stream(stream)))
    return out, widx, ridx


def _scan_shapes(M, widx, wk, ridx, rw, v, alpha, beta):
    B, H, N, d_v = M.shape
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    for name, t, shp in (("widx", widx, (B, H, T, W)), ("wk", wk, (B, H, T, W)),
                         ("ridx", ridx, (B, H, T, R)), ("rw", rw, (B, H, T, R)),
                         ("v", v, (B, H, T, d_v)), ("alpha", alpha, (B, H, T)),
                         ("beta", beta, (B, H, T))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {shp}, got {tuple(t.shape)}")
    return B, H, N, d_v, T, W, R


def _tape_shape(tape, shp):
    if tuple(tape.shape) != shp:
        raise ValueError(f"tape must be {shp}, got {tuple(tape.shape)}")


def _scan_ptrs(widx, wk, ridx, rw, v, alpha, beta):
    import torch

    return (_dev(widx, torch.int32, "widx"), _dev(wk, torch.float32, "wk"),
            _dev(ridx, torch.int32, "ridx"), _dev(rw, torch.float32, "rw"),
            _dev(v, torch.float32, "v"), _dev(alpha, torch.float32, "alpha"),
            _dev(beta, torch.float32, "beta"))


def scan_train(M, widx, wk, ridx, rw, v, alpha, beta, out=None, tape=None, stream=None):
    """scan() on an fp32 state that also keeps, per step, the W pre-write rows
    and the R rows the read used: returns (out [B,H,T,d_v],
    tape [B,H,T,W+R,d_v])."""
    import torch

    B, H, N, d_v, T, W, R = _scan_shapes(M, widx, wk, ridx, rw, v, alpha, beta)
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=torch.float32, device=M.device)
    if tape is None:
        tape = torch.empty((B, H, T, W + R, d_v), dtype=torch.float32, device=M.device)
    _tape_shape(tape, (B, H, T, W + R, d_v))
    _check(lib().sdm_scan_train(_dev(M, torch.float32, "M", 4), B, H, N, d_v, T, W, R,
                                *_scan_ptrs(widx, wk, ridx, rw, v, alpha, beta),
                                _dev(out, torch.float32, "out"),
                                _dev(tape, torch.float32, "tape"), _stream(stream)))
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

    B, H, N, d_v, T, W, R = _scan_shapes(G, widx, wk, ridx, rw, v, alpha, beta)
    _tape_shape(tape, (B, H, T, W + R, d_v))
    if first is not None and tuple(first.shape) != (B, H, T, 2):
        raise ValueError(f"first must be {(B, H, T, 2)}, got {tuple(first.shape)}")
    dev = G.device
    f32 = torch.float32
    o = {"dv": torch.empty((B, H, T, d_v), dtype=f32, device=dev),
         "dwk": torch.empty((B, H, T, W), dtype=f32, device=dev),
         "drw": torch.empty((B, H, T, R), dtype=f32, device=dev),
         "dalpha": torch.empty((B, H, T), dtype=f32, device=dev),
         "dbeta": torch.empty((B, H, T), dtype=f32, device=dev)}
    need = int(lib().sdm_scan_backward_workspace_size(B, H, d_v, T, W, R))
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=f32, device=dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().sdm_scan_backward(B, H, N, d_v, T, W, R,
                                   *_scan_ptrs(widx, wk, ridx, rw, v, alpha, beta),
                                   _dev(tape, f32, "tape"), _dev(dout, f32, "dout"),
                                   _dev(G, f32, "G", 4), o["dv"].data_ptr(), o["dwk"].data_ptr(),
                                   o["drw"].data_ptr(), o["dalpha"].data_ptr(),
                                   o["dbeta"].data_ptr(),
                                   None if first is None else _dev(first, torch.int64, "first"),
                                   _dev(workspace, workspace.dtype, "workspace"),
                                   nbytes, _stream(stream)))
    return o


def touch_prepare(widx, ridx, N: int, seen=None, first=None, stream=None):
    """Bookkeeping of the sparse training mode: seen [B,H,ceil(N/32)] int32
    (the bits of the uint32 words: row r is selected at some step) and first
    [B,H,T,2] int64 (the bits of the uint64 masks of slots whose row is
    selected for the last time at that step).  N <= 2^20."""
    import torch

    B, H, T, W = widx.shape
    R = ridx.shape[3]
    if tuple(ridx.shape) != (B, H, T, R):
        raise ValueError(f"ridx must be {(B, H, T, R)}, got {tuple(ridx.shape)}")
    dev = widx.device
    if seen is None:
        seen = torch.empty((B, H, (N + 31) // 32), dtype=torch.int32, device=dev)
    if first is None:
        first = torch.empty((B, H, T, 2), dtype=torch.int64, device=dev)
    _check(lib().sdm_touch_prepare(B, H, N, T, W, R, _dev(widx, torch.int32, "widx"),
                                   _dev(ridx, torch.int32, "ridx"),
                                   _dev(seen, torch.int32, "seen", 3),
                                   _dev(first, torch.int64, "first", 4), _stream(stream)))
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

    K = idx.shape[-1]
    lead = tuple(idx.shape[:-1])
    units = 1
    for s in lead:
        units *= s
    dx1 = torch.empty(lead + (n,), dtype=torch.float32, device=idx.device)
    dx2 = torch.empty(lead + (n,), dtype=torch.float32, device=idx.device)
    _check(lib().sdm_select_backward(_dev(idx, torch.int32, "idx"),
                                     _dev(weight, torch.float32, "weight"),
                                     _dev(dweight, torch.float32, "dweight"), units, n, K,
                                     dx1.data_ptr(), dx2.data_ptr(), _stream(stream)))
    return dx1, dx2


def state_init_backward(G, out=None, seen=None, stream=None):
    """dM0 [H,N,d_v] = sum over b of G [B,H,N,d_v]; with seen (from
    touch_prepare) only the rows each sequence selected count."""
    import torch

    B, H, N, d_v = G.shape
    dM0 = torch.empty((H, N, d_v), dtype=torch.float32, device=G.device) if out is None else out
    if seen is not None and tuple(seen.shape) != (B, H, (N + 31) // 32):
        raise ValueError(f"seen must be {(B, H, (N + 31) // 32)}, got {tuple(seen.shape)}")
    _check(lib().sdm_state_init_backward(_dev(G, torch.float32, "G", 4), B, H, N, d_v,
                                         None if seen is None else _dev(seen, torch.int32, "seen"),
                                         _dev(dM0, torch.float32, "dM0", 3), _stream(stream)))
    return dM0
