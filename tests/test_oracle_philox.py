"""Pins of the oracle's Philox4x32-10 and the uniforms drawn from it."""
import os

import numpy as np

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        vals = [int(t, 16) for t in line.split()]
        rows.append((vals[0:4], vals[4:6], vals[6:10]))
    return rows


def test_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, want in rows:
        got = philox.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
        assert [int(x) for x in got] == want


def test_vectorised_matches_single():
    ctr = np.array([[b, j, 1, 7] for b in range(5) for j in range(9)], dtype=np.uint64)
    many = philox.philox4x32_10(ctr, (123, 456))
    for i in range(len(ctr)):
        one = philox.philox4x32_10(ctr[i:i + 1], (123, 456))[0]
        assert np.array_equal(one, many[i])


def test_accept_uniforms_range_and_fp32_exact():
    u = philox.accept_uniforms(seed=99, b=3, n=4096, step=11)
    assert np.all(u > 0) and np.all(u <= 1)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)


def test_uniformity_chi2():
    u = np.concatenate([philox.accept_uniforms(seed=5, b=b, n=4096, step=0) for b in range(16)])
    counts, _ = np.histogram(u, bins=64, range=(0, 1))
    exp = len(u) / 64
    chi2 = float(np.sum((counts - exp) ** 2 / exp))
    # 63 degrees of freedom: the 0.999 quantile is about 103
    assert chi2 < 103, chi2


def test_race_clocks_are_exponential():
    E = philox.race_clocks(seed=17, b=2, ids=np.arange(200000), purpose=philox.PURPOSE_SAMPLE, step=3)
    assert np.all(E > 0)
    assert abs(E.mean() - 1.0) < 0.01
    assert abs(np.mean(E > 1.0) - np.exp(-1.0)) < 0.005
    for w in range(4):   # each of the four words of a block on its own
        Ew = E[w::4]
        assert abs(Ew.mean() - 1.0) < 0.02 and abs(np.mean(Ew > 1.0) - np.exp(-1.0)) < 0.01


def test_stream_words_read_blocks_in_order():
    """Id v reads word v mod 4 of the block at counter (b, v div 4, purpose, step)."""
    ids = np.arange(12)
    got = philox.stream_words(5, 7, ids, philox.PURPOSE_SAMPLE, 9)
    ctr = np.array([[7, i, philox.PURPOSE_SAMPLE, 9] for i in range(3)], dtype=np.uint64)
    blocks = philox.philox4x32_10(ctr, philox.key_from_seed(5))
    assert np.array_equal(got, blocks.reshape(-1))
    # word 0 of each block is the same word the accept uniforms take
    assert np.array_equal(got[::4], philox.words(5, 7, np.arange(3), philox.PURPOSE_SAMPLE, 9))


def test_purposes_and_steps_are_distinct_streams():
    a = philox.words(1, 0, np.arange(64), philox.PURPOSE_ACCEPT, 0)
    b = philox.words(1, 0, np.arange(64), philox.PURPOSE_SAMPLE, 0)
    c = philox.words(1, 0, np.arange(64), philox.PURPOSE_ACCEPT, 1)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
