"""CPU oracle for the Sparse Delta Memory step -- TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU product path never imports it and has no CPU
fallback.  The arithmetic lives in sdm_oracle.c (plain C, gcc, no FMA
contraction, no fast-math); this file only builds it and marshals numpy
arrays.  See sdm_oracle.c for the definition it follows and its sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")
F32, BF16, FP8 = 0, 1, 2
_lib = None


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
           "-Wextra", "-o", LIB + ".tmp", os.path.join(_HERE, "sdm_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    global _lib
    _lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run oracle.build()")
        lib = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.oracle_select.argtypes = [p, p, i64, i32, i32, p, p, p]
        lib.oracle_state_init.argtypes = [p, i32, p, i32, i32, i64, i32]
        lib.oracle_scan.argtypes = [p, i32, i64, i32, i64, i32, i32, p, p, p, p, p, p, p, p,
                                    i32, i32]
        lib.oracle_step_decode.argtypes = [p, i32, i32, i32, i32, i32, i32, i32] + [p] * 10
        lib.oracle_scan_backward.argtypes = [p, i64, i32, i64, i32, i32] + [p] * 17
        lib.oracle_select_backward.argtypes = [p, p, p, i64, i32, i32, p, p]
        lib.oracle_project.argtypes = [p, p, i64, i32, i32, i32, p, p]
        lib.oracle_project.restype = ctypes.c_int
        lib.oracle_sigmoid.argtypes = [ctypes.c_double]
        lib.oracle_sigmoid.restype = ctypes.c_double
        lib.oracle_last_error.restype = ctypes.c_char_p
        lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        lib.oracle_bf16_from_double.restype = ctypes.c_uint16
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_fp8_from_float.argtypes = [ctypes.c_float]
        lib.oracle_fp8_from_float.restype = ctypes.c_uint8
        lib.oracle_fp8_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_to_double.restype = ctypes.c_double
        for f in ("oracle_select", "oracle_state_init", "oracle_scan", "oracle_step_decode",
                  "oracle_scan_backward", "oracle_select_backward"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc):
    if rc != 0:
        raise OracleError(_L().oracle_last_error().decode())


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return a.ctypes.data if a is not None else None


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def select(x1, x2, K: int, threads: int = 1):
    """Product-key top-K of halves x1, x2 [..., n] -> (idx int32, score f32,
    weight f64), each [..., K].  `threads` > 1 splits the independent units
    over several calls of the (single-threaded) oracle."""
    x1 = _c(x1, np.float32)
    x2 = _c(x2, np.float32)
    assert x1.shape == x2.shape
    n = x1.shape[-1]
    lead = x1.shape[:-1]
    units = int(np.prod(lead)) if lead else 1
    idx = np.empty(lead + (K,), np.int32)
    score = np.empty(lead + (K,), np.float32)
    weight = np.empty(lead + (K,), np.float64)
    f1, f2 = x1.reshape(units, n), x2.reshape(units, n)
    fi, fs, fw = idx.reshape(units, K), score.reshape(units, K), weight.reshape(units, K)
    L = _L()
    if threads <= 1 or units < 64:
        _check(L.oracle_select(_ptr(f1), _ptr(f2), units, n, K, _ptr(fi), _ptr(fs), _ptr(fw)))
    else:
        step = (units + threads - 1) // threads
        spans = [(s, min(units, s + step)) for s in range(0, units, step)]

        def run(sp):
            a, b = sp
            return L.oracle_select(_ptr(f1[a:b]), _ptr(f2[a:b]), b - a, n, K, _ptr(fi[a:b]),
                                   _ptr(fs[a:b]), _ptr(fw[a:b]))

        with ThreadPoolExecutor(threads) as ex:
            for rc in ex.map(run, spans):
                _check(rc)
    return idx, score, weight


_STATE_NP = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}


def state_init(M0, B: int, dtype: int = F32):
    """M [B,H,N,d_v] (float32, uint16 bf16 bits or uint8 fp8 codes) from
    M0 [H,N,d_v]."""
    M0 = _c(M0, np.float32)
    H, N, d_v = M0.shape
    M = np.empty((B, H, N, d_v), _STATE_NP[dtype])
    _check(_L().oracle_state_init(_ptr(M), dtype, _ptr(M0), B, H, N, d_v))
    return M


def scan(M, dtype, widx, wk, ridx, rw, v, alpha, beta, cols=None, out=None):
    """T steps on ONE memory M [N,d_v] in place; returns out [T,d_v] (float32).
    cols = (c0, c1) restricts the computed columns."""
    N, d_v = M.shape
    assert M.flags.c_contiguous
    assert M.dtype == _STATE_NP[dtype]
    widx, ridx = _c(widx, np.int32), _c(ridx, np.int32)
    wk, rw = _c(wk, np.float64), _c(rw, np.float64)
    v = _c(v, np.float32)
    alpha, beta = _c(alpha, np.float32), _c(beta, np.float32)
    T, W = widx.shape
    R = ridx.shape[1]
    assert v.shape == (T, d_v) and alpha.shape == (T,) and beta.shape == (T,)
    if out is None:
        out = np.zeros((T, d_v), np.float32)
    c0, c1 = (0, d_v) if cols is None else cols
    _check(_L().oracle_scan(_ptr(M), dtype, N, d_v, T, W, R, _ptr(widx), _ptr(wk), _ptr(ridx),
                            _ptr(rw), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(out), c0, c1))
    return out


def step_decode(M, dtype, s1, s2, q1, q2, v, alpha, beta, W: int, R: int):
    """One token for every (b,h) of M [B,H,N,d_v] in place.
    Returns (out [B,H,d_v], widx [B,H,W], ridx [B,H,R])."""
    B, H, N, d_v = M.shape
    n = s1.shape[-1]
    s1, s2, q1, q2 = (_c(a, np.float32) for a in (s1, s2, q1, q2))
    v, alpha, beta = _c(v, np.float32), _c(alpha, np.float32), _c(beta, np.float32)
    out = np.empty((B, H, d_v), np.float32)
    wi = np.empty((B, H, W), np.int32)
    ri = np.empty((B, H, R), np.int32)
    _check(_L().oracle_step_decode(_ptr(M), dtype, B, H, n, d_v, W, R, _ptr(s1), _ptr(s2),
                                   _ptr(q1), _ptr(q2), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(out), _ptr(wi), _ptr(ri)))
    return out, wi, ri


def scan_backward(M0, widx, wk, ridx, rw, v, alpha, beta, dout, dMT=None):
    """Gradients of T steps on ONE fp32 memory with the selections fixed.

    M0 [N,d_v]: the memory before step 0.  dout [T,d_v]: gradient of the loss
    with respect to the read outputs; dMT [N,d_v] (default zero): with respect
    to the memory after the last step.  Returns a dict with dM0 [N,d_v],
    dv [T,d_v], dwk [T,W], drw [T,R], dalpha [T], dbeta [T] (all float64),
    tape [T,W,d_v] (the pre-write rows, float32), rtape [T,R,d_v] (the rows
    each step's read saw, after its write, float32) and MT (the final memory)."""
    M0 = _c(M0, np.float32)
    N, d_v = M0.shape
    widx, ridx = _c(widx, np.int32), _c(ridx, np.int32)
    wk, rw = _c(wk, np.float64), _c(rw, np.float64)
    v, dout = _c(v, np.float32), _c(dout, np.float32)
    alpha, beta = _c(alpha, np.float32), _c(beta, np.float32)
    T, W = widx.shape
    R = ridx.shape[1]
    assert v.shape == (T, d_v) and dout.shape == (T, d_v)
    G = np.zeros((N, d_v), np.float64) if dMT is None else np.array(dMT, np.float64, order="C")
    dv = np.empty((T, d_v), np.float64)
    dwk = np.empty((T, W), np.float64)
    drw = np.empty((T, R), np.float64)
    da = np.empty((T,), np.float64)
    db = np.empty((T,), np.float64)
    tape = np.empty((T, W, d_v), np.float32)
    rtape = np.empty((T, R, d_v), np.float32)
    MT = np.empty((N, d_v), np.float32)
    _check(_L().oracle_scan_backward(_ptr(M0), N, d_v, T, W, R, _ptr(widx), _ptr(wk), _ptr(ridx),
                                     _ptr(rw), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(dout),
                                     _ptr(G), _ptr(dv), _ptr(dwk), _ptr(drw), _ptr(da), _ptr(db),
                                     _ptr(tape), _ptr(rtape), _ptr(MT)))
    return {"dM0": G, "dv": dv, "dwk": dwk, "drw": drw, "dalpha": da, "dbeta": db,
            "tape": tape, "rtape": rtape, "MT": MT}


def select_backward(idx, weight, dweight, n: int):
    """Gradient of the selection weights with respect to the halves x1, x2,
    with the selection held fixed.  idx, weight, dweight [..., K] ->
    (dx1, dx2) [..., n], float64."""
    idx = _c(idx, np.int32)
    w, dw = _c(weight, np.float64), _c(dweight, np.float64)
    K = idx.shape[-1]
    lead = idx.shape[:-1]
    units = int(np.prod(lead)) if lead else 1
    dx1 = np.empty(lead + (n,), np.float64)
    dx2 = np.empty(lead + (n,), np.float64)
    _check(_L().oracle_select_backward(_ptr(idx), _ptr(w), _ptr(dw), units, n, K, _ptr(dx1),
                                       _ptr(dx2)))
    return dx1, dx2


def state_init_backward(dM):
    """Gradient of the per-sequence copy M[b,h] = M0[h]: dM0[h] = sum over b
    of dM[b,h], summed in order b = 0, 1, ... in float64.  dM [B,H,N,d_v]."""
    dM = np.asarray(dM)
    acc = np.zeros(dM.shape[1:], np.float64)
    for b in range(dM.shape[0]):
        acc += dM[b]
    return acc


def bf16_from_double(x: float) -> int:
    return int(_L().oracle_bf16_from_double(float(x)))


def bf16_to_double(h: int) -> float:
    return float(_L().oracle_bf16_to_double(int(h)))


def fp8_from_float(x: float) -> int:
    return int(_L().oracle_fp8_from_float(float(x)))


def fp8_to_double(c: int) -> float:
    return float(_L().oracle_fp8_to_double(int(c)))


def fp8_codes_to_f32(a) -> np.ndarray:
    """Decode uint8 E4M3 codes to float32 (exact) with the oracle's decoder."""
    a = np.asarray(a, np.uint8)
    table = np.array([fp8_to_double(c) for c in range(256)], np.float64).astype(np.float32)
    return table[a]


def bf16_bits_to_f32(a) -> np.ndarray:
    """View uint16 bf16 bits as float32 values (exact widening)."""
    a = np.asarray(a, np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32)


def run_memory(M, dtype, s1, s2, q1, q2, v, alpha, beta, W, R, cols=None, threads=1):
    """Whole sequence on ONE memory: selections for all T steps, then the scan.
    s1.. [T,n]; v [T,d_v]; alpha, beta [T].  Returns dict of outputs."""
    widx, wsc, wk = select(s1, s2, W, threads=threads)
    ridx, rsc, rw = select(q1, q2, R, threads=threads)
    out = scan(M, dtype, widx, wk, ridx, rw, v, alpha, beta, cols=cols)
    return {"widx": widx, "wscore": wsc, "wk": wk, "ridx": ridx, "rscore": rsc, "rw": rw,
            "out": out}


def project(X_bits, Wt_bits, H: int, threads: int = 1):
    """Linear projections of the tokens (bf16 bits): X [M, d_model], Wt
    [H, P, d_model] -> (y, yabs), each [M, H, P] float64: the exact dot
    products and the sums of |x_k w_k| (see sdm_oracle.c).  `threads` > 1
    splits the tokens over several calls."""
    X = _c(X_bits, np.uint16)
    Wt = _c(Wt_bits, np.uint16)
    M, d_model = X.shape
    Hw, P, d2 = Wt.shape
    assert Hw == H and d2 == d_model
    y = np.empty((M, H, P), np.float64)
    ya = np.empty((M, H, P), np.float64)
    L = _L()
    if threads <= 1 or M < 2 * threads:
        _check(L.oracle_project(_ptr(X), _ptr(Wt), M, d_model, H, P, _ptr(y), _ptr(ya)))
        return y, ya
    step = (M + threads - 1) // threads
    spans = [(s, min(M, s + step)) for s in range(0, M, step)]

    def run(sp):
        a, b = sp
        return L.oracle_project(_ptr(X[a:b]), _ptr(Wt), b - a, d_model, H, P, _ptr(y[a:b]),
                                _ptr(ya[a:b]))

    with ThreadPoolExecutor(threads) as ex:
        for rc in ex.map(run, spans):
            _check(rc)
    return y, ya


def sigmoid(y):
    """The gates' logistic function, elementwise, float64 (the oracle's exp)."""
    L = _L()
    f = np.vectorize(lambda t: L.oracle_sigmoid(float(t)), otypes=[np.float64])
    return f(np.asarray(y, np.float64))
