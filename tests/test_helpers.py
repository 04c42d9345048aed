"""The test helpers' parallel input draws (CPU): chunks drawn on a thread
pool equal the same chunks drawn one after another, in order."""

import numpy as np

import workloads
from helpers import drawn_chunks


def test_drawn_chunks_match_serial_draws():
    w = workloads.Workload(31, "adhoc", "chunk", 2, 3, 32, 1000, 11, "bf16",
                           outlier_frac=0.05, outlier_scale=8.0)
    serial = [workloads.chunk_qkv(w, n) for n in range(w.chunks)]
    for ahead in (1, 3, 8, 50):
        seen = []
        for n, got in drawn_chunks(lambda c: workloads.chunk_qkv(w, c), range(w.chunks),
                                   ahead=ahead):
            seen.append(n)
            for a, b in zip(got, serial[n]):
                assert np.array_equal(a, b)
        assert seen == list(range(w.chunks))


def test_drawn_chunks_order_and_subsets():
    order = [5, 0, 3, 3, 9]
    got = [(n, x) for n, x in drawn_chunks(lambda c: c * c, order, ahead=2)]
    assert got == [(n, n * n) for n in order]
    assert list(drawn_chunks(lambda c: c, [])) == []
