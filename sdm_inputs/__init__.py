"""Seeded synthetic inputs for the Sparse Delta Memory step.

This package only generates inputs; it holds none of the method's arithmetic.
Both sides consume it: the CPU oracle through the host generator
(`host_block`), the GPU path through the device generator (`device_block`).
Both implement the same counter-based definition (Philox4x32-10 bits, a
uniform transform and a Box-Muller normal transform with fixed polynomials;
see gen_host.c) and produce identical bits, so any slice of any workload can
be regenerated on either side independently.

Workloads (the five configurations the step is measured and checked on):

  tiny    B1  H1  n64   (N=4096)   d_v16  T256     W=R=8   fp32 state
  small   B4  H4  n256  (N=65536)  d_v64  T2048    W=R=32  fp32 state
  mid     B8  H8  n1024 (N=2^20)   d_v128 T4096    W=R=64  fp32 state
  decode  B64 H4  n1024 (N=2^20)   d_v128 512 x T=1 W=R=64 bf16 state
  long    B1  H16 n1024 (N=2^20)   d_v128 T=2^20   W=R=64  fp32 state

Recipe (per element, all float32):
  s1, s2, q1, q2  N(0,1) sub-scores of length n per (b,h,t)
                  (mid: s = g[b,t,:] + 0.5*e[b,h,t,:], g shared across heads)
  v               N(0,1) of length d_v per (b,h,t)
  alpha           U(0.9, 1) per (b,h,t);  beta U(0, 1) per (b,h,t)
  M0              0.02 * N(0,1), one [N, d_v] table per head
  dout            N(0,1) of length d_v per (b,h,t): the output gradient fed to
                  the reverse pass (training)
  long: planted recall -- at t=1000 slot (i*, j*) gets s1[i*]=s2[j*]=16,
        v=e_0, alpha=beta=1; at t=T-1 the read halves get q1[i*]=q2[j*]=16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsdm_inputs_host.so")
DEV_LIB = os.path.join(_HERE, "libsdm_inputs_dev.so")

GEN_NORMAL = 0
GEN_UNIFORM = 1


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    n: int
    d_v: int
    T: int
    W: int
    R: int
    state: str  # "f32" or "bf16"
    seed: int
    mix: bool = False  # mid: sub-scores share a per-(b,t) component across heads
    planted: bool = False  # long: planted write at t=1000, read at t=T-1
    decode: bool = False  # T single-token calls instead of one T-step scan

    @property
    def N(self) -> int:
        return self.n * self.n

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS = {
    "tiny": Config("tiny", B=1, H=1, n=64, d_v=16, T=256, W=8, R=8, state="f32", seed=101),
    "small": Config("small", B=4, H=4, n=256, d_v=64, T=2048, W=32, R=32, state="f32", seed=202),
    "mid": Config("mid", B=8, H=8, n=1024, d_v=128, T=4096, W=64, R=64, state="f32", seed=303,
                  mix=True),
    "decode": Config("decode", B=64, H=4, n=1024, d_v=128, T=512, W=64, R=64, state="bf16",
                     seed=404, decode=True),
    "long": Config("long", B=1, H=16, n=1024, d_v=128, T=1 << 20, W=64, R=64, state="f32",
                   seed=505, planted=True),
}

# Stream tags (the Philox key's second word).
TAGS = {"s1": 0, "s2": 1, "q1": 2, "q2": 3, "v": 4, "alpha": 5, "beta": 6, "M0": 7,
        "g1": 8, "g2": 9, "planted": 10, "dout": 11}

PLANT_WRITE_T = 1000
PLANT_SCORE = 16.0


def _recipe(cfg: Config, name: str):
    """(tag, kind, scale, lo, hi, mix_tag, mixw, row_len) for tensor `name`."""
    if name in ("s1", "s2"):
        mix_tag = TAGS["g1" if name == "s1" else "g2"] if cfg.mix else -1
        return TAGS[name], GEN_NORMAL, 1.0, 0.0, 0.0, mix_tag, 0.5, cfg.n
    if name in ("q1", "q2"):
        return TAGS[name], GEN_NORMAL, 1.0, 0.0, 0.0, -1, 0.0, cfg.n
    if name == "v":
        return TAGS["v"], GEN_NORMAL, 1.0, 0.0, 0.0, -1, 0.0, cfg.d_v
    if name == "alpha":
        return TAGS["alpha"], GEN_UNIFORM, 1.0, 0.9, 1.0, -1, 0.0, 1
    if name == "beta":
        return TAGS["beta"], GEN_UNIFORM, 1.0, 0.0, 1.0, -1, 0.0, 1
    if name == "M0":
        return TAGS["M0"], GEN_NORMAL, 0.02, 0.0, 0.0, -1, 0.0, cfg.d_v
    if name == "dout":  # training: gradient of the loss with respect to the outputs
        return TAGS["dout"], GEN_NORMAL, 1.0, 0.0, 0.0, -1, 0.0, cfg.d_v
    raise KeyError(name)


def planted_slot(cfg: Config) -> tuple[int, int]:
    """(i*, j*) of the planted recall pattern: Philox call 0 of stream
    (seed, 'planted'), words 0 and 1 modulo n."""
    lib = _host()
    ctr = (ctypes.c_uint32 * 4)(0, 0, 0, 0)
    key = (ctypes.c_uint32 * 2)(cfg.seed, TAGS["planted"])
    out = (ctypes.c_uint32 * 4)()
    lib.sdm_gen_philox4x32_10(ctr, key, out)
    return int(out[0] % cfg.n), int(out[1] % cfg.n)


# --------------------------------------------------------------------------- build

def _cflags_host():
    return ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(verbose: bool = False) -> None:
    """Compile the host (gcc) and device (hipcc, gfx950) generators in-tree."""
    src_h = os.path.join(_HERE, "gen_host.c")
    src_d = os.path.join(_HERE, "gen_device.hip")
    cmds = [
        ["gcc", *_cflags_host(), "-o", HOST_LIB + ".tmp", src_h, "-lm"],
        ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC",
         "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", DEV_LIB + ".tmp", src_d],
    ]
    for cmd, out in zip(cmds, (HOST_LIB, DEV_LIB)):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE if not verbose else None,
                       stderr=subprocess.STDOUT if not verbose else None)
        os.replace(out + ".tmp", out)
    global _HOST, _DEV
    _HOST = None
    _DEV = None


_HOST = None
_DEV = None

_FILL_ARGS = [ctypes.c_void_p] + [ctypes.c_int64] * 10 + [
    ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_float, ctypes.c_float,
    ctypes.c_float, ctypes.c_int, ctypes.c_float]


def _host():
    global _HOST
    if _HOST is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run sdm_inputs.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.sdm_gen_fill_block.argtypes = _FILL_ARGS
        lib.sdm_gen_fill_block.restype = None
        lib.sdm_gen_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        lib.sdm_gen_value.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                                      ctypes.c_int]
        lib.sdm_gen_value.restype = ctypes.c_float
        _HOST = lib
    return _HOST


def _dev():
    global _DEV
    if _DEV is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run sdm_inputs.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.sdm_gen_fill_block_device.argtypes = _FILL_ARGS + [ctypes.c_void_p]
        lib.sdm_gen_fill_block_device.restype = ctypes.c_int
        _DEV = lib
    return _DEV


def philox4x32_10(ctr, key):
    """Raw Philox4x32-10 block (host implementation), for pinning the generator."""
    lib = _host()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib.sdm_gen_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def _logical_dims(cfg: Config, name: str):
    """(B, H, T, len) of the logical tensor the flat element number runs over."""
    tag, kind, scale, lo, hi, mix_tag, mixw, ln = _recipe(cfg, name)
    if name == "M0":
        return 1, cfg.H, cfg.N, ln
    return cfg.B, cfg.H, cfg.T, ln


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def host_block(cfg: Config, name: str, b0: int = 0, nb: int | None = None, h0: int = 0,
               nh: int | None = None, t0: int = 0, nt: int | None = None) -> np.ndarray:
    """Host copy of block [b0:b0+nb, h0:h0+nh, t0:t0+nt, :] of tensor `name`.

    Shapes: s1/s2/q1/q2 [nb,nh,nt,n]; v [nb,nh,nt,d_v]; alpha/beta [nb,nh,nt];
    M0 [nh, nt, d_v] where the t-range runs over the N rows (b is ignored)."""
    Bl, Hl, Tl, ln = _logical_dims(cfg, name)
    if name == "M0":
        b0, nb = 0, 1
    nb = Bl - b0 if nb is None else nb
    nh = Hl - h0 if nh is None else nh
    nt = Tl - t0 if nt is None else nt
    assert 0 <= b0 and b0 + nb <= Bl and 0 <= h0 and h0 + nh <= Hl and 0 <= t0 and t0 + nt <= Tl
    out = np.empty((nb, nh, nt, ln), dtype=np.float32)
    tag, kind, scale, lo, hi, mix_tag, mixw, _ = _recipe(cfg, name)
    lib = _host()
    rows = nb * nh * nt
    # Split over t (then over (b,h)) so large blocks fill on several threads.
    jobs = []
    tchunk = max(1, min(nt, (1 << 22) // max(1, ln)))
    for bb in range(nb):
        for hh in range(nh):
            for ts in range(0, nt, tchunk):
                jobs.append((bb, hh, ts, min(tchunk, nt - ts)))

    def run(job):
        bb, hh, ts, cnt = job
        view = out[bb, hh, ts:ts + cnt]
        lib.sdm_gen_fill_block(view.ctypes.data, 1, 1, cnt, ln, Bl, Hl, Tl, b0 + bb, h0 + hh,
                               t0 + ts, cfg.seed, tag, kind, scale, lo, hi, mix_tag, mixw)

    if rows * ln < (1 << 18) or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(run, jobs))
    _plant_host(cfg, name, out, b0, h0, t0)
    if name in ("alpha", "beta"):
        return out[..., 0]
    if name == "M0":
        return out[0]
    return out


def _plant_points(cfg: Config, name: str):
    """List of (t, column, value) overrides of the planted recall pattern."""
    if not cfg.planted:
        return []
    i_s, j_s = planted_slot(cfg)
    tw, tr = PLANT_WRITE_T, cfg.T - 1
    pts = []
    if tw < cfg.T:
        if name == "s1":
            pts.append((tw, i_s, PLANT_SCORE))
        elif name == "s2":
            pts.append((tw, j_s, PLANT_SCORE))
        elif name in ("alpha", "beta"):
            pts.append((tw, 0, 1.0))
        elif name == "v":
            pts.append((tw, None, None))  # whole row becomes e_0
    if name == "q1":
        pts.append((tr, i_s, PLANT_SCORE))
    elif name == "q2":
        pts.append((tr, j_s, PLANT_SCORE))
    return pts


def _plant_host(cfg, name, out, b0, h0, t0):
    if name == "M0":
        return
    nt = out.shape[2]
    for t, col, val in _plant_points(cfg, name):
        if t0 <= t < t0 + nt:
            if col is None:
                out[:, :, t - t0, :] = 0.0
                out[:, :, t - t0, 0] = 1.0
            else:
                out[:, :, t - t0, col] = val


def device_block(cfg: Config, name: str, dst, b0: int = 0, h0: int = 0, t0: int = 0,
                 stream=None) -> None:
    """Fill the contiguous device tensor `dst` with block (b0.., h0.., t0..) of
    `name`; dst's shape gives the block extent (same layouts as host_block)."""
    import torch

    Bl, Hl, Tl, ln = _logical_dims(cfg, name)
    if not (dst.is_cuda and dst.dtype == torch.float32 and dst.is_contiguous()):
        raise ValueError("dst must be a contiguous float32 device tensor")
    shp = list(dst.shape)
    if name == "M0":
        nh, nt = shp[0], shp[1]
        nb, b0 = 1, 0
        assert shp[2] == ln
    elif name in ("alpha", "beta"):
        nb, nh, nt = shp
    else:
        nb, nh, nt, l2 = shp
        assert l2 == ln
    assert b0 + nb <= Bl and h0 + nh <= Hl and t0 + nt <= Tl
    tag, kind, scale, lo, hi, mix_tag, mixw, _ = _recipe(cfg, name)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = _dev().sdm_gen_fill_block_device(dst.data_ptr(), nb, nh, nt, ln, Bl, Hl, Tl, b0, h0, t0,
                                         cfg.seed, tag, kind, scale, lo, hi, mix_tag, mixw,
                                         stream)
    if rc != 0:
        raise RuntimeError(f"sdm_gen_fill_block_device failed with hipError {rc}")
    if name == "M0":
        return
    view = dst.view(nb, nh, nt, ln)
    for t, col, val in _plant_points(cfg, name):
        if t0 <= t < t0 + nt:
            if col is None:
                view[:, :, t - t0, :] = 0.0
                view[:, :, t - t0, 0] = 1.0
            else:
                view[:, :, t - t0, col] = val


def _bf16_bits_rne(a: np.ndarray) -> np.ndarray:
    """float32 array (finite) -> bf16 bit patterns (uint16), round to nearest
    even: add 0x7FFF plus the lowest kept bit, then drop the low 16 bits."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >>
            np.uint32(16)).astype(np.uint16)


def projection_inputs(B: int, T: int, d_model: int, H: int, P: int, seed: int = 0):
    """Seeded inputs of the token projections, as bf16 bit patterns (uint16):
    X [B, T, d_model] ~ N(0, 1) and Wt [H, P, d_model] ~ N(0, 1/d_model), so
    that each projected value is about N(0, 1), the distribution the
    workloads above give the sub-scores and values.  float32 draws from
    numpy's PCG64 seeded with `seed` (X first, then Wt), each rounded once to
    bf16 to nearest even.  The pages train these weights; random ones of the
    same shape stand in for them."""
    rng = np.random.default_rng(seed)
    X = _bf16_bits_rne(rng.standard_normal((B, T, d_model), dtype=np.float32))
    w = rng.standard_normal((H, P, d_model), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(d_model))
    return X, _bf16_bits_rne(w)
