"""The device's Philox4x32-10 words against the host oracle's, written separately
from the published definition (Salmon et al., SC'11): word 0 of counters (the accept
uniforms) and the output stream words (the race clocks), over a million counters,
several keys, streams, purposes and steps, and start indices that are not a multiple
of four."""
import numpy as np
import pytest
import torch

from oracle import philox

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mod():
    import draft_block_verification_row_amd as m
    m.lib()
    return m


CASES = [
    # (seed, b, purpose, step, idx0, n)
    (0, 0, philox.PURPOSE_ACCEPT, 0, 0, 1 << 20),
    (64, 63, philox.PURPOSE_ACCEPT, 12345, 7, 4096),
    (0xFFFFFFFFFFFFFFFF, 4095, philox.PURPOSE_SAMPLE, 0xFFFFFFFF, 129280 - 5, 4096),
    (2 ** 40 + 3, 17, philox.walk_purpose(4), 9, 3, 1 << 18),
]


@pytest.mark.parametrize("seed,b,purpose,step,idx0,n", CASES)
def test_counter_words(mod, seed, b, purpose, step, idx0, n):
    got = mod.random_words(seed, b, purpose, step, idx0, n, kind=0).cpu().numpy().view(np.uint32)
    ref = philox.words(seed, b, idx0 + np.arange(n, dtype=np.int64), purpose, step).astype(np.uint32)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed,b,purpose,step,idx0,n", CASES)
def test_stream_words(mod, seed, b, purpose, step, idx0, n):
    got = mod.random_words(seed, b, purpose, step, idx0, n, kind=1).cpu().numpy().view(np.uint32)
    ref = philox.stream_words(seed, b, idx0 + np.arange(n, dtype=np.int64), purpose, step).astype(np.uint32)
    assert np.array_equal(got, ref)
