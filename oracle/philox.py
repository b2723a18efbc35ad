"""Philox4x32-10, written from its published definition, and the uniforms drawn from it.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Philox4x32-R is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11).  One round maps a
counter (c0, c1, c2, c3) under a key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with 32x32->64-bit products, M0 = 0xD2511F53, M1 = 0xCD9E8D57.  Ten rounds are
applied; the key is advanced by the Weyl constants (0x9E3779B9, 0xBB67AE85)
before every round but the first.

The verify pages say nothing about the random source (they use uniforms u_i in
the block test and a seeded sampler).  The reading used here: every random
number of one verify call is a pure function of (seed, stream, index, purpose,
step), so calls are replayable and independent of how streams are sharded.

    key     = (seed & 0xffffffff, seed >> 32)
    counter = (b, idx, purpose, step & 0xffffffff), output word 0 is used

purposes: ACCEPT (idx = draft slot j) gives the uniform of the accept tests;
SAMPLE gives the exponential clocks of the verifiers' sampler and 16 + j those
of slot j of the drafter's walk; DRAFT is reserved for drafting harnesses.

The sampler needs one clock per vocabulary id.  Those are read off the
generator's output stream for (b, purpose, step): counter (b, i, purpose, step)
yields the 128-bit block of words 4i .. 4i+3, so id v takes word v mod 4 of the
block at i = v div 4 (the four output words of one counter, in order).
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_SAMPLE = 3
WALK_PURPOSE_BASE = 16


def walk_purpose(j: int) -> int:
    """Purpose word of the clocks of slot j of the drafter's walk (apart from the verifiers')."""
    return WALK_PURPOSE_BASE + int(j)

_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32_10(counters, key) -> np.ndarray:
    """Apply Philox4x32-10 to an (N, 4) array of uint32 counters under key (k0, k1).

    Returns an (N, 4) uint32 array.  Arithmetic is done in uint64 so the 64-bit
    products are exact.
    """
    ctr = np.asarray(counters, dtype=np.uint64).reshape(-1, 4)
    c0, c1, c2, c3 = (ctr[:, i].copy() for i in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = np.uint64(M0) * c0
        p1 = np.uint64(M1) * c2
        c0, c1, c2, c3 = ((p1 >> _S32) ^ c1 ^ k0, p1 & _MASK,
                          (p0 >> _S32) ^ c3 ^ k1, p0 & _MASK)
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def key_from_seed(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & 0xFFFFFFFF, seed >> 32)


def words(seed: int, b, idx, purpose: int, step: int) -> np.ndarray:
    """Output word 0 for counters (b, idx, purpose, step); b and idx broadcast."""
    b = np.asarray(b, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    b, idx = np.broadcast_arrays(b, idx)
    n = b.size
    ctr = np.empty((n, 4), dtype=np.uint64)
    ctr[:, 0] = b.reshape(-1).astype(np.uint64)
    ctr[:, 1] = idx.reshape(-1).astype(np.uint64)
    ctr[:, 2] = np.uint64(purpose)
    ctr[:, 3] = np.uint64(int(step) & 0xFFFFFFFF)
    return philox4x32_10(ctr, key_from_seed(seed))[:, 0].reshape(b.shape)


def accept_uniforms(seed: int, b: int, n: int, step: int) -> np.ndarray:
    """u_{b,j} = ((x >> 8) + 1) * 2^-24 in (0, 1], j = 0..n-1 (exact in fp32 and fp64)."""
    x = words(seed, b, np.arange(n), PURPOSE_ACCEPT, step).astype(np.float64)
    return (np.floor(x / 256.0) + 1.0) * 2.0 ** -24


def stream_words(seed: int, b: int, ids, purpose: int, step: int) -> np.ndarray:
    """Word v of the output stream of (b, purpose, step) for every id v: word (v mod 4) of
    the block at counter (b, v div 4, purpose, step)."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    n = ids.size
    ctr = np.empty((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.uint64(int(b) & 0xFFFFFFFF)
    ctr[:, 1] = (ids // 4).astype(np.uint64)
    ctr[:, 2] = np.uint64(purpose)
    ctr[:, 3] = np.uint64(int(step) & 0xFFFFFFFF)
    blocks = philox4x32_10(ctr, key_from_seed(seed))
    return blocks[np.arange(n), ids % 4]


def race_clocks(seed: int, b: int, ids, purpose: int, step: int) -> np.ndarray:
    """Exponential clocks E_v = -ln(U_v), U_v = ((x_v >> 8) + 1/2) * 2^-24 in (0, 1) (fp64),
    x_v = word v of the stream of (b, purpose, step)."""
    x = stream_words(seed, b, ids, purpose, step).astype(np.float64)
    U = (np.floor(x / 256.0) + 0.5) * 2.0 ** -24
    return -np.log(U)
