"""The C-ABI library loads, exports every function include/sdm.h declares,
and rejects bad arguments before any launch (these calls never reach the GPU,
so they run without one)."""
import ctypes
import os
import re

import pytest

import sparse_memory_linear_sdm_amd as sdm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")

FAKE = 1 << 20  # a non-null, 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(sdm.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = sdm.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.sdm_abi_version() == 6
    assert L.sdm_status_string(0) == b"SDM_OK"
    assert L.sdm_status_string(2) == b"SDM_ERR_UNSUPPORTED"


def _err():
    return sdm.lib().sdm_last_error().decode()


def test_select_validation():
    L = sdm.lib()
    ok = (FAKE, FAKE, 10, 64, 8, FAKE, FAKE, FAKE, None)
    bad = [
        ((None,) + ok[1:], 1, "x1"),
        (ok[:5] + (None,) + ok[6:], 1, "idx"),
        (ok[:2] + (-1,) + ok[3:], 1, "units"),
        (ok[:4] + (0,) + ok[5:], 1, "K"),
        (ok[:4] + (65,) + ok[5:], 1, "K"),
        (ok[:3] + (100,) + ok[4:], 2, "n=100"),
        (ok[:3] + (4096, 64) + ok[5:], 2, "n=4096"),
        (ok[:3] + (128, 96) + ok[5:], 2, "K=96"),
        ((FAKE + 4,) + ok[1:3] + (256,) + ok[4:], 1, "aligned"),
    ]
    for args, status, word in bad:
        rc = L.sdm_select(*args)
        assert rc == status, (args, rc, _err())
        assert word in _err()


def test_project_validation():
    L = sdm.lib()
    ok = (FAKE, FAKE, 2, 100, 256, 2, 64, 16) + (FAKE,) * 7 + (None,)
    bad = [
        ((None,) + ok[1:], 1, "NULL"),
        (ok[:4] + (96,) + ok[5:], 2, "multiple of 64"),
        (ok[:4] + (0,) + ok[5:], 2, "multiple of 64"),
        (ok[:4] + (65600,) + ok[5:], 2, "multiple of 64"),
        (ok[:2] + (-1,) + ok[3:], 1, "B and T"),
        (ok[:6] + (0,) + ok[7:], 1, "n and d_v"),
        (ok[:5] + (1 << 20, 1 << 20) + ok[7:], 2, "2^31"),
        (ok[:2] + (1 << 30, 1 << 30) + ok[4:], 2, "tiles"),
        (ok[:12] + (None,) + ok[13:], 1, "v is NULL"),
        (ok[:8] + (FAKE + 2,) + ok[9:], 1, "s1 must be 4-byte aligned"),
        ((FAKE + 8,) + ok[1:], 1, "16-byte aligned"),
    ]
    for args, status, word in bad:
        rc = L.sdm_project(*args)
        assert rc == status, (args, rc, _err())
        assert word in _err(), _err()
    assert L.sdm_project(None, None, 0, 100, 256, 2, 64, 16, *([None] * 7), None) == 0


def test_state_init_validation():
    L = sdm.lib()
    assert L.sdm_state_init(None, 0, FAKE, 1, 1, 16, 16, None) == 1
    assert L.sdm_state_init(FAKE, 7, FAKE, 1, 1, 16, 16, None) == 1
    assert L.sdm_state_init(FAKE, 0, FAKE, 1, 1, 16, 24, None) == 2
    assert L.sdm_state_init(FAKE, 0, FAKE, 0, 1, 16, 16, None) == 1
    assert L.sdm_state_init(FAKE + 8, 0, FAKE, 1, 1, 16, 16, None) == 1
    assert L.sdm_state_init(FAKE, 0, FAKE, 1, 1, 1 << 31, 16, None) == 1


def test_scan_validation():
    L = sdm.lib()
    ok = [FAKE, 0, 1, 1, 4096, 16, 8, 8, 8] + [FAKE] * 9 + [None]
    assert len(ok) == 19

    def call(**kw):
        a = list(ok)
        pos = {"M": 0, "dtype": 1, "B": 2, "H": 3, "N": 4, "d_v": 5, "T": 6, "W": 7, "R": 8,
               "widx": 9, "v": 13, "out": 16}
        for k, v in kw.items():
            a[pos[k]] = v
        return L.sdm_scan(*a)

    assert call(M=None) == 1
    assert call(dtype=3) == 1
    assert call(dtype=2) == 2  # fp8 state needs d_v >= 32
    assert call(B=0) == 1
    assert call(T=-1) == 1
    assert call(W=0) == 1
    assert call(W=65) == 2
    assert call(R=100) == 2
    assert call(d_v=48) == 2
    assert call(N=4, W=8) == 1
    assert call(widx=None) == 1
    assert call(v=FAKE + 4) == 1
    assert call(out=FAKE + 8) == 1


def test_step_decode_validation():
    L = sdm.lib()
    ok = [FAKE, 1, 2, 2, 64, 128, 8, 8] + [FAKE] * 8 + [None, None, None]
    assert L.sdm_step_decode(*([None] + ok[1:])) == 1
    a = list(ok); a[4] = 100
    assert L.sdm_step_decode(*a) == 2
    a = list(ok); a[6] = 65
    assert L.sdm_step_decode(*a) == 1
    a = list(ok); a[5] = 100
    assert L.sdm_step_decode(*a) == 2
    a = list(ok); a[8] = None
    assert L.sdm_step_decode(*a) == 1
    a = list(ok); a[1] = 5
    assert L.sdm_step_decode(*a) == 1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sdm, "_lib", None)
    monkeypatch.setattr(sdm, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        sdm.lib()


def test_training_calls_validation():
    L = sdm.lib()
    # sdm_scan_train: M, B, H, N, d_v, T, W, R, 7 inputs, out, tape, stream
    ok = [FAKE, 1, 1, 4096, 16, 8, 8, 8] + [FAKE] * 9 + [None]
    assert L.sdm_scan_train(*ok[:16] + [None, None]) == 1  # tape NULL
    a = list(ok); a[16] = FAKE + 4
    assert L.sdm_scan_train(*a) == 1  # tape misaligned
    a = list(ok); a[5] = 1 << 22; a[4] = 256; a[6] = 64
    assert L.sdm_scan_train(*a) == 2 and "tape" in _err()  # one memory's tape above 2 GiB
    a = list(ok); a[4] = 128; a[5] = 40000; a[6] = 64; a[7] = 64
    assert L.sdm_scan_train(*a) == 2 and "W+R" in _err()  # the read rows count too
    need = L.sdm_scan_backward_workspace_size(2, 4, 128, 100, 64, 32)
    assert need == 2 * 4 * 100 * 8 * (64 + 32 + 1) * 4  # 8 column tiles of 16 (the narrowest)
    assert L.sdm_scan_backward_workspace_size(1, 1, 16, 10, 8, 8) == 10 * 1 * 17 * 4
    assert L.sdm_scan_backward_workspace_size(1, 1, 48, 10, 8, 8) == 0
    # sdm_scan_backward: B, H, N, d_v, T, W, R, 7 inputs, tape, dout, G, dv, dwk, drw,
    # dalpha, dbeta, first, workspace, bytes, stream (the state is not an argument)
    wsb = L.sdm_scan_backward_workspace_size(1, 1, 16, 8, 8, 8)
    ok = [1, 1, 4096, 16, 8, 8, 8] + [FAKE] * 17 + [wsb, None]
    assert len(ok) == 26
    a = list(ok); a[22] = FAKE + 4  # first misaligned
    assert L.sdm_scan_backward(*a) == 1 and "first" in _err()
    a = list(ok); a[24] = wsb - 4
    assert L.sdm_scan_backward(*a) == 1 and "workspace" in _err()
    a = list(ok); a[16] = None  # G
    assert L.sdm_scan_backward(*a) == 1
    a = list(ok); a[14] = FAKE + 4  # tape misaligned
    assert L.sdm_scan_backward(*a) == 1
    a = list(ok); a[4] = 1 << 26
    assert L.sdm_scan_backward(*a) == 2
    # one finishing wavefront per memory and step: B*H*T of 2^26 would need
    # 2^32 work-items in one launch
    a = list(ok); a[0] = 1 << 8; a[1] = 1 << 8; a[4] = 1 << 10
    assert L.sdm_scan_backward(*a) == 2 and "2^26 - 4" in _err()
    a = list(ok); a[0] = 1 << 11; a[1] = 1 << 10  # 2^21 memories
    assert L.sdm_scan_backward(*a) == 2 and "2^20" in _err()
    a = list(ok); a[3] = 24
    assert L.sdm_scan_backward(*a) == 2
    a = list(ok); a[3] = 128; a[4] = 40000; a[5] = 64; a[6] = 64
    assert L.sdm_scan_backward(*a) == 2 and "W+R" in _err()
    # sdm_select_backward: idx, w, dw, units, n, K, dx1, dx2, stream
    ok = [FAKE, FAKE, FAKE, 10, 64, 8, FAKE, FAKE, None]
    a = list(ok); a[6] = None
    assert L.sdm_select_backward(*a) == 1
    a = list(ok); a[5] = 65
    assert L.sdm_select_backward(*a) == 1
    a = list(ok); a[4] = 100
    assert L.sdm_select_backward(*a) == 2
    # sdm_state_init_backward: G, B, H, N, d_v, last, dM0, stream
    assert L.sdm_state_init_backward(FAKE, 1, 1, 16, 16, None, None, None) == 1
    assert L.sdm_state_init_backward(FAKE, 0, 1, 16, 16, None, FAKE, None) == 1
    assert L.sdm_state_init_backward(FAKE, 1, 1, 16, 20, None, FAKE, None) == 2
    assert L.sdm_state_init_backward(FAKE, 1, 1, 16, 16, FAKE + 2, FAKE, None) == 1
    # sdm_touch_prepare: B, H, N, T, W, R, widx, ridx, last, first, stream
    ok = [1, 1, 4096, 8, 8, 8, FAKE, FAKE, FAKE, FAKE, None]
    for i, bad, want in ((4, 65, 1), (5, 0, 1), (2, 0, 1), (8, None, 1), (9, FAKE + 4, 1),
                         (3, 1 << 26, 2), (3, -1, 1), (0, 0, 1), (2, (1 << 20) + 1, 2)):
        a = list(ok); a[i] = bad
        assert L.sdm_touch_prepare(*a) == want, (i, bad)
    a = list(ok); a[3] = 1 << 23; a[4] = 64  # T * W * 4 = 2^31: index arrays too large
    assert L.sdm_touch_prepare(*a) == 2 and "2 GiB" in _err()
    a = list(ok); a[6] = None
    assert L.sdm_touch_prepare(*a) == 1  # widx NULL with T > 0
    a = list(ok); a[0] = 1 << 11; a[1] = 1 << 10
    assert L.sdm_touch_prepare(*a) == 2 and "2^20" in _err()
    # sdm_select_backward: units at the launch limit (ceil(units/4) blocks of 256 threads)
    assert L.sdm_select_backward(FAKE, FAKE, FAKE, (1 << 26) - 3, 64, 8, FAKE, FAKE, None) == 2


def test_launch_size_limits():
    """Every call that launches one wavefront per unit, or walks memories,
    rejects sizes whose grid would need 2^32 work-items, before any launch."""
    L = sdm.lib()
    # select: (units + 3) / 4 blocks of 256 threads; 2^26 - 4 units is the largest grid
    assert L.sdm_select(FAKE, FAKE, (1 << 26) - 3, 64, 8, FAKE, FAKE, FAKE, None) == 2
    assert "2^26 - 4" in _err()
    assert L.sdm_select(FAKE, FAKE, 1 << 32, 64, 8, FAKE, FAKE, FAKE, None) == 2
    # scan / scan_train: at most 2^20 memories
    assert L.sdm_scan(FAKE, 0, 1 << 11, 1 << 10, 4096, 16, 8, 8, 8, *[FAKE] * 9, None) == 2
    assert "2^20" in _err()
    assert L.sdm_scan_train(FAKE, 1 << 11, 1 << 10, 4096, 16, 8, 8, 8, *[FAKE] * 9,
                            FAKE, None) == 2
    # decode
    ok = [FAKE, 1, 1 << 11, 1 << 10, 64, 128, 8, 8] + [FAKE] * 8 + [None, None, None]
    assert L.sdm_step_decode(*ok) == 2 and "2^20" in _err()


def test_fp8_state_validation():
    L = sdm.lib()
    assert L.sdm_state_init(FAKE, 2, FAKE, 1, 1, 16, 16, None) == 2  # fp8 needs d_v >= 32
    assert L.sdm_state_init(FAKE, 3, FAKE, 1, 1, 16, 32, None) == 1
    ok = [FAKE, 1, 1, 1, 64, 128, 8, 8] + [FAKE] * 8 + [None, None, None]
    ok[1] = 2
    assert L.sdm_step_decode(*ok) == 2 and "decode" in _err()


def test_zero_length_calls_accept_null_arrays():
    """T = 0 and units = 0 are no-ops whose empty arrays may be NULL (what an
    empty tensor hands over); sizes and the state pointer are still checked."""
    L = sdm.lib()
    assert L.sdm_select(None, None, 0, 64, 8, None, None, None, None) == 0
    assert L.sdm_select(None, None, 0, 64, 65, None, None, None, None) == 1  # K still checked
    assert L.sdm_select_backward(None, None, None, 0, 64, 8, None, None, None) == 0
    null9 = [None] * 8
    assert L.sdm_scan(FAKE, 0, 1, 1, 4096, 16, 0, 8, 8, *null9, None) == 0
    assert L.sdm_scan(None, 0, 1, 1, 4096, 16, 0, 8, 8, *null9, None) == 1  # M still required
    assert L.sdm_scan_train(FAKE, 1, 1, 4096, 16, 0, 8, 8, *null9, None, None) == 0
    args = [1, 1, 4096, 16, 0, 8, 8] + [None] * 9 + [FAKE] + [None] * 7 + [0, None]
    assert L.sdm_scan_backward(*args) == 0
    args[16] = None  # G is state-sized and still required
    assert L.sdm_scan_backward(*args) == 1
