"""Host check of the persistent kernels' work queues (the LM-head kernel and the backward GEMMs):
the kernels' own queue code (csrc/rlk_queue.h, compiled for the host) must hand out every item of
a launch exactly once, whatever the launch geometry. No GPU is needed.

A dropped item would leave a tile's partials unwritten and a repeated one would only cost time,
so coverage is what makes a schedule-independent result possible (RL-Kernel v0.1.0 summary,
"Numeric execution contract": the result may not depend on how the work is split).
"""

import os
import random
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("queue") / "queue_check")
    csrc = os.path.join(ROOT, "invariant_lm_head_deterministic_amd", "csrc")
    subprocess.run([HIPCC, "-std=c++17", "-O1", f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
                    os.path.join(ROOT, "tests", "queue_check.cpp"), "-o", exe], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return exe


def _launch(rows: int, H: int, V: int, segments: int = 4, bt: int = 256):
    """(n_vb, n_tt, rb) of a one-pass launch: 4-tile vocab blocks of 64-column tiles per segment,
    row tiles of bt rows, bands whose hidden rows stay under 64 MB."""
    tiles = -(-(V // segments) // 64)
    n_vb = segments * (-(-tiles // 4))
    n_tt = -(-rows // bt)
    rb = max(1, (64 << 20) // (bt * H * 2))
    return n_vb, n_tt, rb


def _run(exe, geoms):
    args = [str(v) for g in geoms for v in g]
    r = subprocess.run([exe, *args], capture_output=True, text=True)
    lines = r.stdout.strip().splitlines()
    assert len(lines) == len(geoms), r.stdout + r.stderr
    bad = [ln for ln in lines if not ln.startswith("OK")]
    assert r.returncode == 0 and not bad, "\n".join(bad)


def test_workload_launches(checker):
    _run(checker, [
        _launch(4096, 4096, 151936),            # Qwen3-8B head, one pass
        _launch(4096, 4096, 151936, 1),         # one segment
        _launch(4096, 4096, 37984, 1),          # one TP4 shard
        _launch(55296, 4096, 151936),           # long GRPO batch, one pass (7 bands)
        _launch(8192, 4096, 151936),            # one 8192-row chunk
        _launch(6144, 4096, 151936),            # the batch's last chunk
        _launch(8192, 5120, 151936),            # fused-norm head (bands of 25 row tiles)
        _launch(600, 65536, 256),               # largest hidden size (bands of 2)
        _launch(257, 256, 1000),                # one row past a row tile
        _launch((1 << 21) + 3, 1024, 1000),     # the 2^21 + 3 row test
    ])


def _gemm(M: int, N: int, batches: int = 1):
    """(n_vb, n_tt, rb) of a backward GEMM launch: 256 x 256 tiles, the items A tiles x (batch,
    B tile), one band per batch."""
    n_mt, n_nt = -(-M // 256), -(-N // 256)
    return n_mt, n_nt * batches, n_nt


def test_backward_gemm_launches(checker):
    J = 4 * 38016  # Qwen3-8B head: 4 segments of 37984 positions padded to 128
    _run(checker, [
        _gemm(J, 4096),            # dz: padded positions x rows
        _gemm(4096, 4096, 4),      # dh: hidden columns x rows, one batch per segment
        _gemm(4096, J),            # dW: hidden columns x padded positions
        _gemm(J // 4, 4096),       # dz of one TP4 shard
        _gemm(128, 1, 8),          # tiny: 8 segments of one row
        _gemm(5120, 8192, 4),      # fused-norm head's dh
        _gemm(300, 77, 2),
    ])


def test_random_geometries(checker):
    rng = random.Random(1234)
    geoms = [(rng.randint(1, 700), rng.randint(1, 300), rng.randint(1, 40)) for _ in range(300)]
    geoms += [(n_vb, n_tt, rb) for n_vb in (1, 7, 8, 9, 16, 17) for n_tt in (1, 2, 3, 31, 32, 33)
              for rb in (1, 4, 32)]
    _run(checker, geoms)
