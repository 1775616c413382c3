"""Pins of the oracle's packed-weight index map: a bijection on the canonical bytes,
round trip bit-exact (the model card's pack/unpack pair is bit-exact), zero padding."""

import numpy as np
import pytest

from oracle import repack as P


@pytest.mark.parametrize("N,K", [(32, 64), (128, 256), (40, 96), (1, 16), (65, 208)])
def test_round_trip_and_bijection(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = rng.integers(0, 127, size=(K // 16, N), dtype=np.uint8)
    packed = P.repack(qw, ws)
    assert packed.size == P.packed_bytes(N, K)
    q2, w2 = P.unpack(packed, N, K)
    assert np.array_equal(q2, qw) and np.array_equal(w2, ws)
    # the array form and the element-by-element form state the same map
    assert np.array_equal(P.repack_loops(qw, ws), packed)
    q3, w3 = P.unpack_loops(packed, N, K)
    assert np.array_equal(q3, qw) and np.array_equal(w3, ws)
    # every canonical byte appears exactly once, padding is zero
    pad = packed.size - qw.size - ws.size
    assert np.array_equal(np.sort(packed), np.sort(np.concatenate([qw.ravel(), ws.ravel(), np.zeros(pad, np.uint8)])))


def test_fragment_order_of_one_chunk():
    N, K = 64, 128
    qw = np.arange(N * K // 2, dtype=np.int64).reshape(N, K // 2).astype(np.uint8)
    ws = np.arange(K // 16 * N).reshape(K // 16, N).astype(np.uint8)
    packed = P.repack(qw, ws)
    NP, KP = 2, 2
    # chunk (p=1, q=1), dword for h=1, c=3, t=2 -> channel 35, k = 64 + 32 + 8 = 104
    base = 1024 * (1 * NP + 1)
    d = (1 * 32 + 3) * 4 + 2
    assert list(packed[base + 4 * d: base + 4 * d + 4]) == list(qw[35, 52:56])
    sbase = 1024 * NP * KP + 128 * (1 * NP + 1)
    assert packed[sbase + 3 * 4 + 2] == ws[6, 35]
    assert P.packed_bytes(10240, 3840) == 10240 * 3840 // 2 + 10240 * 3840 // 16
