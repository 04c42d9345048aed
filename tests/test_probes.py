"""The HBM probe library that `bench.py --workload ceiling` times: it loads,
exports its two calls, reports the bytes one chunk of each access mix moves,
and rejects bad arguments before it launches anything (no GPU needed: every
lap_stream call here fails validation, so no HIP call is made)."""

import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE_LIB = os.path.join(ROOT, "block_causal_linear_amd", "libla_probes.so")

pytestmark = pytest.mark.skipif(not os.path.exists(PROBE_LIB), reason="libla_probes.so not built")

READ, WRITE, COPY, WIDEN = 0, 1, 2, 3
SWEEP, RANGE, ONESHOT = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    pl = ctypes.CDLL(PROBE_LIB)
    pl.lap_chunk_bytes.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_longlong),
                                   ctypes.POINTER(ctypes.c_longlong)]
    pl.lap_chunk_bytes.restype = ctypes.c_int
    pl.lap_stream.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_longlong, ctypes.c_void_p,
                                                   ctypes.c_void_p]
    pl.lap_stream.restype = ctypes.c_int
    return pl


def chunk_bytes(lib, mode):
    r, w = ctypes.c_longlong(-1), ctypes.c_longlong(-1)
    rc = lib.lap_chunk_bytes(mode, ctypes.byref(r), ctypes.byref(w))
    return rc, r.value, w.value


def test_chunk_bytes_of_each_mix(lib):
    rc, r, w = chunk_bytes(lib, READ)
    assert rc == 0 and r > 0 and w == 0 and r % 16 == 0
    rc, r2, w2 = chunk_bytes(lib, WRITE)
    assert rc == 0 and r2 == 0 and w2 == r
    rc, r3, w3 = chunk_bytes(lib, COPY)
    assert rc == 0 and r3 == w3 == r
    # the readout's mix: bfloat16 in, float32 out, so twice the bytes written
    rc, r4, w4 = chunk_bytes(lib, WIDEN)
    assert rc == 0 and r4 > 0 and w4 == 2 * r4


def test_chunk_bytes_rejects_unknown_mode(lib):
    assert chunk_bytes(lib, 4)[0] == 1
    assert chunk_bytes(lib, -1)[0] == 1


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


@pytest.mark.parametrize("mode, sched, wgs, src, dst, nchunks, sink", [
    (READ, SWEEP, 512, FAKE, FAKE, 0, FAKE),          # no chunks
    (READ, SWEEP, 512, FAKE, FAKE, -5, FAKE),
    (READ, SWEEP, 0, FAKE, FAKE, 10, FAKE),           # no workgroups for a sweep
    (COPY, RANGE, -1, FAKE, FAKE, 10, FAKE),
    (READ, SWEEP, 512, None, FAKE, 10, FAKE),         # a read mix without a source
    (WRITE, SWEEP, 512, FAKE, None, 10, FAKE),        # a write mix without a destination
    (WIDEN, ONESHOT, 0, FAKE, None, 10, FAKE),
    (COPY, SWEEP, 512, FAKE, FAKE, 10, None),         # no sink
    (7, SWEEP, 512, FAKE, FAKE, 10, FAKE),            # unknown mode
])
def test_stream_rejects_bad_arguments(lib, mode, sched, wgs, src, dst, nchunks, sink):
    assert lib.lap_stream(mode, sched, wgs, 0, 0, src, dst, nchunks, sink, None) == 1
