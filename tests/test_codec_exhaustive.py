"""The library's fp32 -> E4M3 encoder (csrc/fp8_codec.h; it quantises x / s and h / s on the GPU)
against the oracle's codec on every finite float32 bit pattern, 2^32 - 2^24 of them, on the CPU.

The encoder source is compiled for the host into a small harness (tests/e4m3_encode_harness.cpp);
the oracle codec (oracle/fp8_e4m3.py) is written from the format definition and shares nothing
with it.  The patterns are split into chunks spread over worker processes."""
import ctypes
import os
import subprocess
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_top_amd", "csrc")
HARNESS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "e4m3_encode_harness.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CHUNK = 1 << 22

_lib = None


def _worker_init(path):
    global _lib
    _lib = ctypes.CDLL(path)
    _lib.e4m3_encode_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]


def _compare(start):
    from oracle import fp8_e4m3
    out = np.empty(CHUNK, np.uint8)
    _lib.e4m3_encode_range(start, CHUNK, out.ctypes.data)
    v = (np.arange(CHUNK, dtype=np.uint32) + np.uint32(start)).view(np.float32)
    want = fp8_e4m3.encode(v.astype(np.float64))
    bad = np.nonzero(out != want)[0]
    if bad.size:
        i = int(bad[0])
        return int(bad.size), (start + i, int(out[i]), int(want[i]))
    return 0, None


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    so = str(tmp_path_factory.mktemp("codec") / "e4m3_harness.so")
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-fPIC", "-shared", f"-I{CSRC}",
                    HARNESS, "-o", so], check=True, capture_output=True)
    return so


def test_harness_spot_values(harness):
    _worker_init(harness)
    vals = np.array([0.0, -0.0, 1.0, 448.0, 464.0, 1e9, -1.0, 2.0 ** -9, 2.0 ** -10, 1.0625, 1.1875],
                    np.float32)
    want = [0x00, 0x80, 0x38, 0x7E, 0x7E, 0x7E, 0xB8, 0x01, 0x00, 0x38, 0x3A]
    got = []
    for v in vals:
        out = np.empty(1, np.uint8)
        _lib.e4m3_encode_range(int(v.view(np.uint32)), 1, out.ctypes.data)
        got.append(int(out[0]))
    assert got == want


@pytest.mark.slow
@pytest.mark.timeout(1800)
def test_encoder_matches_oracle_on_every_finite_fp32(harness):
    # finite patterns: exponent field below 255, both signs
    starts = [s for base in (0, 0x80000000) for s in range(base, base + 0x7F800000, CHUNK)]
    workers = max(1, min(len(os.sched_getaffinity(0)), 16))
    ctx = mp.get_context("fork")
    mismatches, first = 0, None
    with ProcessPoolExecutor(workers, mp_context=ctx, initializer=_worker_init,
                             initargs=(harness,)) as ex:
        for n, f in ex.map(_compare, starts, chunksize=4):
            mismatches += n
            first = first or f
    assert len(starts) * CHUNK == 2 ** 32 - 2 ** 24
    assert mismatches == 0, f"{mismatches} mismatches; first (pattern, got, want): {first}"
