"""Host check of every raw buffer descriptor the scan, training-forward,
reverse-scan and bookkeeping kernels build (sparse_memory_linear_sdm_amd/
csrc/ranges.h, compiled here with g++ alone): for every shape the GPU tests
and the workloads use, and a sweep around them, each descriptor's range is in
[0, 2^31), the last valid access of every column tile lies inside it, and the
"no access" offset 2^31 lies past it.  The C-ABI layer runs the same check
before every launch.

It also shows, on the CPU, how the GPU fault recorded for the small
workload's parity test arose: an earlier scan producer built its per-chunk
value descriptor with the range steps * d_v * 4 - tile * 128, which is
negative for a chunk past the end of the sequence (steps = 0) and any column
tile > 0 -- for d_v = 64 (the first tested shape with two tiles), -128, i.e.
a 32-bit record count of 2^32 - 128 that switched range checking off."""
import itertools
import os
import shutil
import subprocess

import pytest

import sdm_inputs as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIMIT = 1 << 31


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("ranges") / "ranges_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                    os.path.join(ROOT, "tests", "native", "ranges_check.cpp"), "-o", exe],
                   check=True)

    def run(lines):
        r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                           timeout=120, check=True)
        return r.stdout.split("\n")[:len(lines)]

    return run


def _accepted(N, d_v, es, T, W, R, tape):
    """Sizes the C-ABI layer's other checks accept (tables and tapes below 2 GiB)."""
    if N * d_v * es >= LIMIT:
        return False
    return not tape or T * (W + R) * d_v * 4 < LIMIT


def _shapes():
    cfgs = [S.CONFIGS[k] for k in ("tiny", "small", "mid", "decode", "long")]
    cfgs.append(S.CONFIGS["small"].with_(B=1, H=2, T=512))  # the parity subset that faulted
    named = {(c.N, c.d_v, c.T, c.W, c.R) for c in cfgs}
    named.add((S.CONFIGS["long"].N, 128, 16384, 64, 64))      # one long-stream chunk
    sweep = set(itertools.product(
        [64, 1024, 1369, 4096, 65536, 1 << 20],                # n = 8, 32, 37, 64, 256, 1024
        [16, 32, 64, 128, 256],
        [1, 7, 8, 9, 12, 37, 45, 70, 100, 300, 512, 4096],
        [(1, 1), (8, 8), (13, 29), (16, 24), (32, 32), (64, 64)]))
    sweep = {(N, d, T, W, R) for N, d, T, (W, R) in sweep if max(W, R) <= N}
    return sorted(named | sweep)


def test_every_descriptor_of_every_tested_shape_is_in_range(checker):
    lines, want = [], []
    for N, d_v, T, W, R in _shapes():
        for es in (4, 2, 1):
            if es == 1 and d_v < 32:
                continue  # fp8 state needs d_v >= 32
            if _accepted(N, d_v, es, T, W, R, False):
                lines.append(f"scan {N} {d_v} {es} {T} {W} {R}")
        if _accepted(N, d_v, 4, T, W, R, True):
            lines.append(f"train {N} {d_v} 4 {T} {W} {R}")
            lines.append(f"bwd {N} {d_v} 4 {T} {W} {R}")
        lines.append(f"touch {N} {d_v} 4 {T} {W} {R}")
    got = checker(lines)
    bad = [l for l, g in zip(lines, got) if g != "1"]
    assert not bad, bad[:10]
    assert len(lines) > 5000


def test_oversized_tables_are_caught(checker):
    # the checks are not vacuous: a table or tape of 2 GiB fails them
    got = checker([f"scan {1 << 22} 128 4 8 8 8",          # 2 GiB state table
                   f"train {1 << 10} 128 4 {1 << 15} 64 64",  # 2 GiB tape
                   f"bwd {1 << 22} 128 4 8 8 8",
                   f"touch 4096 16 4 {1 << 27} 8 8",          # 2 GiB of masks
                   f"scan {(1 << 21) - 1} 256 4 8 8 8"])     # just below 2 GiB: fine
    assert got == ["0", "0", "0", "0", "1"]


def test_old_metadata_range_shows_the_recorded_fault(checker):
    # small workload subset: d_v = 64 -> two 32-column tiles.  In range for the
    # chunks inside the sequence, negative past its end for tile 1.
    got = checker(["oldmeta 8 64 1", "oldmeta 8 64 0", "oldmeta 0 64 0", "oldmeta 0 64 1"])
    vals = [tuple(int(x) for x in g.split()) for g in got]
    assert vals[0] == (8 * 64 * 4 - 128, 8 * 64 * 4 - 128)
    assert vals[2] == (0, 0)
    assert vals[3] == (-128, (1 << 32) - 128)  # record count ~4 G: range checking off
