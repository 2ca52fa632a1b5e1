"""The Python binding rejects every mis-shaped, mistyped or strided tensor,
caller-supplied outputs included, before it calls the library: the kernels
index each buffer by sizes taken from other arguments, so a short buffer
would be read or written out of bounds.  Shapes are checked before the
device, so these run on CPU tensors and no kernel is ever reached."""
import pytest
import torch

import sparse_memory_linear_sdm_amd as sdm

f32, i32, i64 = torch.float32, torch.int32, torch.int64
B, H, N, n, d_v, T, W, R = 2, 3, 64, 8, 16, 5, 4, 3


def z(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def scan_args():
    return dict(M=z(B, H, N, d_v), widx=z(B, H, T, W, dtype=i32), wk=z(B, H, T, W),
                ridx=z(B, H, T, R, dtype=i32), rw=z(B, H, T, R), v=z(B, H, T, d_v),
                alpha=z(B, H, T), beta=z(B, H, T))


def expect(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_well_formed_cpu_tensors_stop_at_the_device_check():
    a = scan_args()
    expect("on the GPU", sdm.scan, **a)
    expect("on the GPU", sdm.select, z(4, n), z(4, n), 3)
    expect("on the GPU", sdm.state_init, z(H, N, d_v), B)


@pytest.mark.parametrize("name,bad", [
    ("widx", z(B, H, T, W)), ("wk", z(B, H, T, W - 1)), ("rw", z(B, H, T, R + 1)),
    ("v", z(B, H, T, d_v - 4)), ("v", z(B, H, T + 1, d_v)), ("alpha", z(B, H, T + 1)),
    ("beta", z(B, H)), ("M", z(B, H, N, d_v, dtype=i32)), ("wk", z(B, H, T, W, dtype=torch.float64))])
def test_scan_rejects_bad_inputs(name, bad):
    a = scan_args()
    a[name] = bad
    expect(name, sdm.scan, **a)


def test_scan_rejects_bad_out_and_strided_inputs():
    a = scan_args()
    expect("out", sdm.scan, **a, out=z(B, H, T - 1, d_v))
    expect("out", sdm.scan, **a, out=z(B, H, T, d_v, dtype=torch.bfloat16))
    a["v"] = z(B, H, d_v, T).transpose(2, 3)  # right shape, strided
    expect("v must be contiguous", sdm.scan, **a)


def test_state_init_rejects_bad_out():
    expect("M must have shape", sdm.state_init, z(H, N, d_v), B, out=z(B, H, N - 1, d_v))
    expect("M must have shape", sdm.state_init, z(H, N, d_v), B, out=z(B + 1, H, N, d_v))
    expect("M must be", sdm.state_init, z(H, N, d_v), B, out=z(B, H, N, d_v, dtype=i32))
    expect("M must be contiguous", sdm.state_init, z(H, N, d_v), B,
           out=z(B, H, d_v, N).transpose(2, 3))


def test_select_rejects_bad_out():
    x = z(2, 7, n)
    expect("idx", sdm.select, x, x, 3, out=(z(2, 7, 2, dtype=i32), None, z(2, 7, 3)))
    expect("idx", sdm.select, x, x, 3, out=(z(2, 7, 3), None, z(2, 7, 3)))  # wrong dtype
    expect("weight", sdm.select, x, x, 3, out=(z(2, 7, 3, dtype=i32), None, z(14, 3)))
    expect("score", sdm.select, x, x, 3, out=(z(2, 7, 3, dtype=i32), z(2, 7, 4), z(2, 7, 3)))
    expect("x2", sdm.select, x, z(2, 7, n + 1), 3)


def decode_args():
    return dict(M=z(B, H, n * n, d_v), s1=z(B, H, n), s2=z(B, H, n), q1=z(B, H, n),
                q2=z(B, H, n), v=z(B, H, d_v), alpha=z(B, H), beta=z(B, H), W=W, R=R)


@pytest.mark.parametrize("name,bad", [
    ("s2", z(B, H, n - 1)), ("q1", z(B, 1, n)), ("q2", z(B * H, n)), ("v", z(B, H, d_v + 1)),
    ("alpha", z(B, H, 1)), ("beta", z(B)), ("s1", z(B, H, n, dtype=torch.float16))])
def test_step_decode_rejects_bad_inputs(name, bad):
    a = decode_args()
    a[name] = bad
    expect(name, sdm.step_decode, **a)


def test_step_decode_rejects_bad_out():
    expect("out", sdm.step_decode, **decode_args(), out=z(B, H, d_v - 1))
    expect("out", sdm.step_decode, **decode_args(), out=z(B, H, d_v, dtype=i32))


def train_args():
    a = scan_args()
    a["tape"] = z(B, H, T, W + R, d_v)
    a["dout"] = z(B, H, T, d_v)
    a["G"] = a.pop("M")
    return a


def test_scan_backward_rejects_bad_inputs():
    for name, bad in (("dout", z(B, H, T, d_v + 1)), ("dout", z(B, H, T - 1, d_v)),
                      ("tape", z(B, H, T, W, d_v)), ("G", z(B, H, N, d_v, dtype=torch.float64))):
        a = train_args()
        a[name] = bad
        expect(name, sdm.scan_backward, **a)
    expect("first", sdm.scan_backward, **train_args(), first=z(B, H, T, 1, dtype=i64))
    expect("first", sdm.scan_backward, **train_args(), first=z(B, H, T, 2, dtype=i32))
    expect("on the GPU", sdm.scan_backward, **train_args())


def test_scan_train_rejects_bad_out_and_tape():
    a = scan_args()
    expect("tape", sdm.scan_train, **a, tape=z(B, H, T, W + R - 1, d_v))
    expect("out", sdm.scan_train, **a, out=z(B, H, T, d_v + 16))
    a["M"] = z(B, H, N, d_v, dtype=torch.bfloat16)
    expect("M must be", sdm.scan_train, **a)


def test_training_helpers_reject_bad_tensors():
    wi, ri = z(B, H, T, W, dtype=i32), z(B, H, T, R, dtype=i32)
    expect("seen", sdm.touch_prepare, wi, ri, N, seen=z(B, H, N // 32 + 1, dtype=i32))
    expect("first", sdm.touch_prepare, wi, ri, N, first=z(B, H, T, 2, dtype=f32))
    expect("ridx", sdm.touch_prepare, wi, z(B, H, T + 1, R, dtype=i32), N)
    expect("dweight", sdm.select_backward, z(4, W, dtype=i32), z(4, W), z(4, W + 1), n)
    expect("weight", sdm.select_backward, z(4, W, dtype=i32), z(4, W + 2), z(4, W), n)
    G = z(B, H, N, d_v)
    expect("dM0", sdm.state_init_backward, G, out=z(H, N, d_v - 1))
    expect("seen", sdm.state_init_backward, G, seen=z(B, H, N // 32 - 1, dtype=i32))


def test_project_rejects_bad_inputs_and_outputs():
    bf = torch.bfloat16
    d_model, P = 64, 4 * n + d_v + 2
    X, Wt = z(B, T, d_model, dtype=bf), z(H, P, d_model, dtype=bf)
    expect("on the GPU", sdm.project, X, Wt, n)
    expect("X must be", sdm.project, z(B, T, d_model), Wt, n)          # fp32 X
    expect("X must be", sdm.project, z(B * T, d_model, dtype=bf), Wt, n)
    expect("too few", sdm.project, X, Wt, P)                            # n too large for P
    expect("Wt must have shape", sdm.project, X, z(H, P, d_model + 64, dtype=bf), n)
    outs = [z(B, H, T, n)] * 4 + [z(B, H, T, d_v), z(B, H, T), z(B, H, T)]
    expect("on the GPU", sdm.project, X, Wt, n, out=tuple(outs))
    bad = list(outs)
    bad[4] = z(B, H, T, d_v + 1)
    expect("v must have shape", sdm.project, X, Wt, n, out=tuple(bad))
    bad = list(outs)
    bad[6] = z(B, T, H)
    expect("beta", sdm.project, X, Wt, n, out=tuple(bad))
    expect("7 tensors", sdm.project, X, Wt, n, out=tuple(outs[:6]))
