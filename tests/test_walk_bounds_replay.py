"""Host replay of the index formulas of the drafter walk's kernels.

Every global address that the resident walk (one launch for all slots) and the two
launches per slot form is recomputed here, on the CPU, from the kernels' own index
expressions, for every thread of every workgroup and every slot, and checked
against the size of the buffer it falls in: the caller's tensors at their
documented shapes and the workspace regions at the sizes the library lays out.
Besides the edge shapes (one id, fewer ids than a vector, odd vocabularies, more
streams than groups, two blocks of streams, 32 slots, every Markov rank), the
cases include the shape on which the resident walk first ran with the workspace's
clock region left unset: some workgroups draw nothing there (17 groups, 6
streams), so the drawing workgroups' clocks go through that region.
"""
from __future__ import annotations

import numpy as np
import pytest

K_GROUP, K_WAVE_COLS, K_THREADS, K_CHUNK, K_WAVES = 256, 64, 256, 16, 4
K_WALK_ROWS, K_WALK_CHUNKS = 64, 4
K_SYNC_STRIDE, K_GO_COPIES, K_GO_STRIDE = 16, 16, 32
K_WALK_SUBS = 16
K_GRID_COUNT_LINES = 2 * (K_WALK_SUBS + 1)
K_GO_BASE = K_SYNC_STRIDE * (1 + K_GRID_COUNT_LINES)
K_SYNC_INTS = K_GO_BASE + K_GO_COPIES * K_GO_STRIDE
K_WALK_CLOCK_BYTES = 64 * 256 * 2
TID = np.arange(K_THREADS)


class Mem:
    """Buffers by name with their sizes in elements; accesses are index arrays."""

    def __init__(self, sizes):
        self.sizes = dict(sizes)
        self.count = 0

    def at(self, name, idx, n=1, mask=None):
        idx = np.asarray(idx, dtype=np.int64).ravel()
        if mask is not None:
            idx = idx[np.asarray(mask).ravel()]
        if idx.size == 0:
            return
        size = self.sizes[name]
        assert size is not None, f"{name} is absent but was accessed"
        lo, hi = int(idx.min()), int(idx.max()) + n
        assert lo >= 0 and hi <= size, f"{name}[{lo}:{hi}] outside [0, {size})"
        self.count += idx.size


class Walk:
    def __init__(self, B, k, V, R=0, bf16=True, counts=None, temps=True, anchors=True, seed=0):
        rng = np.random.default_rng(seed)
        self.B, self.k, self.V, self.R = B, k, V, R
        self.esz = 2 if bf16 else 4
        self.NG = (V + K_GROUP - 1) // K_GROUP
        self.vec = (V * self.esz) % 16 == 0 and V >= 16
        self.ks = R // 32
        self.counts = counts
        gam = np.full(B, k) if counts is None else np.clip(np.asarray(counts), 0, k)
        # drawn tokens: ids below gamma_b, -1 past it
        self.drawn = np.where(np.arange(k)[None, :] < gam[:, None], rng.integers(0, V, size=(B, k)), -1)
        self.anchor = rng.integers(-1, V, size=B) if anchors else None
        NG, ND, NT = self.NG, B * k, B * (k + 1)
        # race: the walk's 32-byte candidate records in a region laid out for the
        # verifiers' 16-byte ones or these, whichever is larger
        clk_bytes = max(B * NG * K_GROUP * 2, 2 * min(B, NG) * K_WALK_CLOCK_BYTES)
        self.mem = Mem(dict(
            draft=ND * V, tokens=ND, logq=ND,
            num_drafts=None if counts is None else B, temperature=B if temps else None,
            anchor=B if anchors else None, W1=V * R if R else None, W2t=V * R if R else None,
            tpart=NG * NT, race=max(ND * NG * 16, B * NG * 32) // 32, clk=clk_bytes // 8, sync=K_SYNC_INTS))

    # window of each thread in group g
    def lane(self, g):
        w, q = TID >> 6, (TID & 63) >> 4
        cb = g * K_GROUP + w * K_WAVE_COLS
        cw = cb + 16 * q
        c0 = np.minimum(cw, self.V - 16) if self.vec else cw
        return c0

    def row_load(self, row, c0):
        """raw_load of 16 ids from column c0 of draft rows `row` (arrays over threads)."""
        if self.vec:
            self.mem.at("draft", row * self.V + c0, 16)
        else:
            for e in range(16):
                self.mem.at("draft", row * self.V + c0 + e, mask=(c0 + e) < self.V)

    def load_rows(self, j, r0, c0):
        n = TID & 15
        for cc in range(K_WALK_CHUNKS):
            row = np.minimum(r0 + cc * K_CHUNK + n, self.B - 1) * self.k + j
            self.row_load(row, c0)

    def slab(self, g):
        if not self.R:
            return
        n, q = TID & 15, (TID & 63) >> 4
        cb = g * K_GROUP + (TID >> 6) * K_WAVE_COLS
        for s in range(4):
            if self.vec:
                vr = np.minimum(cb + 16 * (n >> 2), self.V - 16) + 4 * s + (n & 3)
            else:
                vr = cb + 16 * (n >> 2) + 4 * s + (n & 3)
                vr = np.where(vr < self.V, vr, self.V - 1)
            for kk in range(self.ks):
                self.mem.at("W2t", vr * self.R + kk * 32 + 8 * q, 8)

    def prev_raw(self, b, j):
        """The previous-token word a thread reads for stream b at slot j (stand-ins included)."""
        if j > 0:
            self.mem.at("tokens", b * self.k + j - 1)
            return self.drawn[b, j - 1]
        if self.anchor is not None:
            self.mem.at("anchor", b)
            return self.anchor[b]
        self.mem.at("tokens", b * self.k)   # stand-in word, replaced
        return np.full(np.shape(b), -1)

    def block(self, g, j, r0):
        """walk_block: per-stream inputs, W1 staging, partial and candidate stores."""
        t = TID[TID < K_WALK_ROWS]
        b = np.minimum(r0 + t, self.B - 1)
        if self.mem.sizes["temperature"] is not None:
            self.mem.at("temperature", b)
        else:
            self.mem.at("tokens", b * self.k)
        pv = self.prev_raw(b, j)
        has = j > 0 or self.anchor is not None
        prev = np.where(has & (pv >= 0) & (pv < self.V), pv, -1)
        if self.R:
            for u in range(0, K_WALK_ROWS * 4 * self.ks, K_THREADS):
                uu = u + TID
                ok = uu < K_WALK_ROWS * 4 * self.ks
                row, piece = uu[ok] // (4 * self.ks), uu[ok] % (4 * self.ks)
                p = prev[row]
                self.mem.at("W1", np.where(p >= 0, p, 0) * self.R + 8 * piece, 8)
        live = r0 + t < self.B
        self.mem.at("tpart", g * self.B + r0 + t, mask=live)
        self.mem.at("race", g * self.B + r0 + t, mask=live)

    def pick(self, b, j, NG, greedy):
        """walk_pick_body for stream b at slot j (one workgroup)."""
        k, B = self.k, self.B
        if self.counts is not None:
            self.mem.at("num_drafts", b)
            gamma = int(np.clip(self.counts[b], 0, k))
        else:
            self.mem.at("tokens", b * k)
            gamma = k
        if self.mem.sizes["temperature"] is not None:
            self.mem.at("temperature", b)
        else:
            self.mem.at("tokens", b * k)
        pr = int(self.prev_raw(np.array([b]), j)[0])
        g0, g1 = np.minimum(TID, NG - 1), np.minimum(TID + K_THREADS, NG - 1)
        for gg in (g0, g1):
            self.mem.at("tpart", gg * B + b)
            self.mem.at("race", gg * B + b)
        self.mem.at("sync", 1)
        if j >= gamma:
            self.mem.at("tokens", b * k + j)
            self.mem.at("logq", b * k + j)
            return
        for gi0 in range(2 * K_THREADS, NG, K_THREADS):
            gi = gi0 + TID
            self.mem.at("tpart", gi * B + b, mask=gi < NG)
            self.mem.at("race", gi * B + b, mask=gi < NG)
        prev = pr if (self.R and 0 <= pr < self.V and (j > 0 or self.anchor is not None)) else -1
        drow = (b * k + j) * self.V
        if greedy:
            gsel = NG - 1   # any group: the addresses are clamped the same way for each
            v = gsel * K_GROUP + TID
            if prev >= 0:
                SL = 4 * self.ks
                RPI = 64 // SL
                NI = K_GROUP // K_WAVES // RPI
                w, l = TID >> 6, TID & 63
                sl, ri = l % SL, l // SL
                self.mem.at("W1", prev * self.R + 8 * sl, 8)
                for n in range(NI):
                    vv = np.minimum(gsel * K_GROUP + w * 64 + n * RPI + ri, self.V - 1)
                    self.mem.at("W2t", vv * self.R + 8 * sl, 8)
            self.mem.at("draft", drow + v, mask=v < self.V)
        else:
            l = TID & 63
            for cand in (0, self.V - 1, self.V // 2):   # candidates are ids in [0, V)
                if prev >= 0:
                    for i in range(4):
                        r = l + 64 * i
                        self.mem.at("W1", prev * self.R + r, mask=r < self.R)
                        self.mem.at("W2t", cand * self.R + r, mask=r < self.R)
                self.mem.at("draft", drow + cand)
        self.mem.at("tokens", b * k + j)
        self.mem.at("logq", b * k + j)


def replay_resident(p: Walk, greedy=False):
    NG, B, k = p.NG, p.B, p.k
    G = NG
    NP, NO = min(B, G), G - min(B, G)
    slot_words = K_WALK_CHUNKS * 4 * K_THREADS
    # the wait words cleared before the launch
    p.mem.at("sync", np.arange(4))
    p.mem.at("sync", K_GO_BASE + K_GO_STRIDE * np.arange(K_GO_COPIES))
    p.mem.at("sync", K_SYNC_STRIDE * np.arange(K_GRID_COUNT_LINES + 1))

    def arrive(phase):   # a sub-counter, the parity's top counter, then every go copy
        base = K_SYNC_STRIDE * (1 + (phase & 1) * (K_WALK_SUBS + 1))
        p.mem.at("sync", base + K_SYNC_STRIDE * np.arange(K_WALK_SUBS + 1))
        p.mem.at("sync", K_GO_BASE + K_GO_STRIDE * np.arange(K_GO_COPIES))

    def wait(g):
        p.mem.at("sync", K_GO_BASE + K_GO_STRIDE * (g % K_GO_COPIES))
        p.mem.at("sync", 1)

    for g in range(G):
        c0 = p.lane(g)
        picker = g < NP
        p.load_rows(0, 0, c0)
        p.slab(g)
        for j in range(k):
            if picker and j > 0 and NO > 0:
                p.mem.at("clk", ((j & 1) * NP + g) * slot_words + TID[None, :] + K_THREADS * np.arange(16)[:, None])
            for r0 in range(0, B, K_WALK_ROWS):
                if r0 > 0:
                    p.load_rows(j, r0, c0)
                p.block(g, j, r0)
            last = j + 1 == k
            arrive(2 * j + 1)
            if picker:
                wait(g)
                for b in range(g, B, G):
                    p.pick(b, j, NG, greedy)
                if not last:
                    arrive(2 * j + 2)
                    p.load_rows(j + 1, 0, c0)
                    wait(g)
            elif not last:
                for t in range(g - NP, NP * K_WALK_CHUNKS, NO):
                    pg, cc = divmod(t, K_WALK_CHUNKS)
                    base = ((j + 1) & 1) * NP + pg
                    p.mem.at("clk", base * slot_words + cc * 4 * K_THREADS + TID[None, :]
                             + K_THREADS * np.arange(4)[:, None])
                arrive(2 * j + 2)
                p.load_rows(j + 1, 0, c0)
                wait(g)


def replay_separate(p: Walk, greedy=False):
    for j in range(p.k):
        for g in range(p.NG):
            c0 = p.lane(g)
            p.load_rows(j, 0, c0)
            p.slab(g)
            for r0 in range(0, p.B, K_WALK_ROWS):
                if r0 > 0:
                    p.load_rows(j, r0, c0)
                p.block(g, j, r0)
        for b in range(p.B):
            p.pick(b, j, p.NG, greedy)


CASES = [
    # (B, k, V, R, bf16, counts, temps, anchors)
    (6, 5, 4099, 128, False, None, True, True),             # some workgroups draw nothing
    (64, 5, 129280, 256, True, None, True, True),           # the headline walk
    (100, 4, 50000, 128, True, "ragged", True, False),      # two blocks of streams
    (600, 2, 1000, 256, True, None, False, True),           # more streams than groups
    (1, 1, 1, 32, False, None, True, True),                 # one id
    (3, 32, 7, 64, False, "ragged", True, True),            # fewer ids than a window, 32 slots
    (9, 3, 131072, 32, True, None, True, True),             # 512 groups
    (5, 5, 257, 0, True, None, False, False),               # no Markov head, one id past a group
    (70, 3, 16, 256, True, "ragged", True, True),           # one window per row
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}-k{c[1]}-V{c[2]}-R{c[3]}" for c in CASES])
@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
def test_every_walk_access_in_bounds(case, greedy):
    B, k, V, R, bf16, counts, temps, anchors = case
    rng = np.random.default_rng(B + V)
    cnt = None if counts is None else rng.integers(-1, k + 2, size=B)
    for replay in (replay_resident, replay_separate):
        p = Walk(B, k, V, R, bf16, cnt, temps, anchors, seed=V)
        replay(p, greedy)
        assert p.mem.count > 0


def test_offloaded_clocks_fit_their_region():
    """The drawing workgroups' clocks (two slot parities) fit the clock region whenever
    some workgroups draw nothing, at every batch and vocabulary size."""
    for B in (1, 2, 6, 63, 64, 65, 200):
        for V in (16, 255, 256, 4099, 16384, 50000, 131072):
            NG = (V + K_GROUP - 1) // K_GROUP
            NP = min(B, NG)
            region = max(B * NG * K_GROUP * 2, 2 * min(B, NG) * K_WALK_CLOCK_BYTES)
            assert 2 * NP * K_WALK_CHUNKS * 4 * K_THREADS * 8 <= region
