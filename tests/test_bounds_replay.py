"""Host replay of the device index formulas of the verify kernels.

Every address that the pack, scan, pass-2 and finalize phases form is recomputed
here, on the CPU, from the same index expressions the kernels use, for every thread
of every workgroup, and checked against the size of the buffer it falls in (the
caller's tensors at their documented shapes, the workspace regions at the sizes the
library lays out).  The configurations are the edge cases: absent per-stream
counts, temperatures and anchors; streams with no drafts; the largest block
(k = 32); vocabularies smaller than one group, not a multiple of the vector width,
or of 16 ids; every Markov rank; and item lists at their fullest.

The last test replays the prologue of a scan variant that was tried and withdrawn
after the device reported an illegal address: it read gamma_b from a stand-in
address when the counts are absent and used that raw word to place its token
gathers.  At the shapes of the test that faulted it reaches far past the logits.
"""
from __future__ import annotations


import numpy as np
import pytest

K_GROUP, K_WAVE_COLS, K_WAVES, K_THREADS, K_CHUNK, K_MAX_K = 256, 64, 4, 256, 16, 32
K_SCAN_ROWS, K_SCAN_GROUPS, K_LOADS = 6, 256, 8
K_STAGE_ITER = K_SCAN_ROWS * K_SCAN_GROUPS // K_THREADS
K_QUEUES, K_QUEUE_STRIDE = 8, 32
K_SYNC_STRIDE, K_GRID_SUBS, K_GO_COPIES, K_GO_STRIDE = 16, 16, 16, 32
K_GRID_COUNT_LINES = 2 * (K_GRID_SUBS + 1)
K_GO_BASE = K_SYNC_STRIDE * (1 + K_GRID_COUNT_LINES)
K_SYNC_INTS = K_GO_BASE + K_GO_COPIES * K_GO_STRIDE


class Mem:
    """Buffers by name with their sizes in elements; every access is checked."""

    def __init__(self, sizes):
        self.sizes = dict(sizes)
        self.hi = {n: -1 for n in sizes}
        self.count = 0

    def at(self, name, idx, n=1):
        """An access of n consecutive elements starting at idx."""
        size = self.sizes[name]
        assert size is not None, f"{name} is absent but was read"
        assert 0 <= idx and idx + n <= size, f"{name}[{idx}:{idx + n}] outside [0, {size})"
        self.hi[name] = max(self.hi[name], idx + n - 1)
        self.count += 1


class Problem:
    def __init__(self, B, k, V, R=0, bf16=True, counts=None, temps=None, anchors=None, tokens=None, seed=0):
        rng = np.random.default_rng(seed)
        self.B, self.k, self.V, self.R = B, k, V, R
        self.esz = 2 if bf16 else 4
        self.NG = (V + K_GROUP - 1) // K_GROUP
        self.NT, self.ND = B * (k + 1), B * k
        self.vec = (V * self.esz) % 16 == 0 and V >= 16
        self.tokens = rng.integers(0, V, size=(B, k)) if tokens is None else np.asarray(tokens)
        self.counts = None if counts is None else np.asarray(counts)
        self.temps = None if temps is None else np.asarray(temps, dtype=np.float32)
        self.anchors = None if anchors is None else np.asarray(anchors)
        self.ks = R // 32
        tiles = (self.ND + K_CHUNK - 1) // K_CHUNK
        self.mem = Mem(dict(
            target=self.NT * V, draft=self.ND * V, tokens=B * k,
            num_drafts=None if counts is None else B, temperature=None if temps is None else B,
            anchor=None if anchors is None else B,
            W1=V * R if R else None, W2t=V * R if R else None,
            tpart=self.NG * self.NT, dpart=self.NG * self.ND, wgrp=self.NG * self.ND,
            tm=self.NT, tl2s=self.NT, dm=self.ND, dl2s=self.ND, logP=self.NT, lpx=self.ND, lqx=self.ND,
            info=4 * B, info2=4 * B, rowmask=B, items=self.ND, nitems=K_QUEUE_STRIDE * (1 + K_QUEUES),
            btile=tiles * 8 * 64, race=self.NG * self.ND, sync=K_SYNC_INTS, clk=B * self.NG * 64,
            accepted_len=B, out_tokens=self.NT, diag=self.NT * 5))

    # the device's per-stream readers ---------------------------------------------
    def gamma(self, b):
        if self.counts is None:
            return self.k
        self.mem.at("num_drafts", b)
        g = int(self.counts[b])
        return 0 if g < 0 else min(g, self.k)

    def temp(self, b):
        if self.temps is None:
            return 1.0
        self.mem.at("temperature", b)
        return float(self.temps[b])

    def draft_prev(self, b, j):
        if j == 0:
            if self.anchors is None:
                return -1
            self.mem.at("anchor", b)
            prev = int(self.anchors[b])
        else:
            self.mem.at("tokens", b * self.k + j - 1)
            prev = int(self.tokens[b, j - 1])
        return prev if 0 <= prev < self.V else -1

    def clamp_tok(self, x):
        return 0 if x < 0 else (self.V - 1 if x >= self.V else x)

    def row_load(self, name, row, c0, n=16, vec=None):
        """raw_load / load1 of n ids from column c0 of a logits row."""
        vec = self.vec if vec is None else vec
        if vec:
            self.mem.at(name, row * self.V + c0, n)
        else:
            for i in range(n):
                if c0 + i < self.V:
                    self.mem.at(name, row * self.V + c0 + i)


# ---------------------------------------------------------------------------
# pack: one 64-lane workgroup per 16 draft rows
# ---------------------------------------------------------------------------
def replay_pack(p: Problem, fused_grid: int):
    nchd = (p.ND + K_CHUNK - 1) // K_CHUNK
    for c in range(nchd):
        for l in range(64):
            n, q = l & 15, l >> 4
            if c == 0 and l < 2:
                p.mem.at("nitems", l)
            if c == 0 and l < K_QUEUES:
                p.mem.at("nitems", K_QUEUE_STRIDE * (1 + l))
            if fused_grid > 0 and c == 0:   # error word, counters, go copies
                if l < 4:
                    p.mem.at("sync", l)
                if l < K_GO_COPIES:
                    p.mem.at("sync", K_GO_BASE + K_GO_STRIDE * l)
                for i in range(l, K_GRID_COUNT_LINES + 1, 64):
                    p.mem.at("sync", K_SYNC_STRIDE * i)
            if p.R == 0:
                continue
            drc = min(c * K_CHUNK + n, p.ND - 1)
            b, j = divmod(drc, p.k)
            pv = p.draft_prev(b, j)
            for kk in range(8):
                kc = kk if kk < p.ks else 0
                p.mem.at("W1", max(pv, 0) * p.R + kc * 32 + 8 * q, 8)
            for kk in range(p.ks):
                p.mem.at("btile", (c * p.ks * 64 + l + kk * 64) * 1)


# ---------------------------------------------------------------------------
# scan: one workgroup per stream
# ---------------------------------------------------------------------------
def stage_load(p, b, r0, nt, nd, g0, ng, tid):
    k1 = p.k + 1
    for i in range(K_STAGE_ITER):
        e = tid + K_THREADS * i
        gl, r = min(e // K_SCAN_ROWS, ng - 1), e % K_SCAN_ROWS
        gg = g0 + gl
        p.mem.at("tpart", gg * p.NT + b * k1 + r0 + (r if r < nt else 0))
        p.mem.at("dpart", gg * p.ND + b * p.k + min(r0 + (r if r < nd else 0), p.k - 1))


def replay_greedy_scan(p, b, gamma):
    k1 = p.k + 1
    for tid in range(K_THREADS):
        w, l = tid >> 6, tid & 63
        for r in range(w, gamma + 1, K_WAVES):
            row = b * k1 + r
            for g0 in range(0, p.NG, 64 * K_LOADS):
                for u in range(K_LOADS):
                    p.mem.at("tpart", min(g0 + l + 64 * u, p.NG - 1) * p.NT + row)
            for gs in range(p.NG):   # the group found by the search: any of them
                for i in range(K_GROUP // 64):
                    v = gs * K_GROUP + (K_GROUP // 64) * l + i
                    if v < p.V:
                        p.mem.at("target", row * p.V + v)
    for j in range(gamma):
        p.mem.at("tokens", b * p.k + j)
    p.mem.at("info", 4 * b, 4)
    p.mem.at("rowmask", b)
    for tid in range(gamma + 1):
        p.mem.at("logP", b * k1 + tid)
    for tid in range(gamma):
        p.mem.at("lpx", b * p.k + tid)
        p.mem.at("lqx", b * p.k + tid)


def scan_masks(p, b, gamma, method, rng):
    """The (stop, mask) pairs the scan can reach for this stream: the extremes and a draw."""
    out = []
    if method == 0:
        for t in sorted({0, gamma, int(rng.integers(0, gamma + 1))}):
            t = min(t, gamma)
            out.append((t, (1 << t) if t < gamma else 0))
    else:
        out.append((gamma, 0))   # top test passed: the bonus row
        if gamma > 0:
            for f in sorted({0, gamma - 1, int(rng.integers(0, gamma))}):
                full = 0
                for i in range(f, gamma):
                    full |= 1 << i
                out.append((-1, full))   # every row above f may pass
                out.append((-1, 1 << f))
    return out


def replay_scan(p: Problem, b, method, stop_mask, s_base, bonus_slot):
    """One stream's scan; stop_mask the decision taken; s_base its first list slot,
    bonus_slot the slot of its bonus item (or None)."""
    k1 = p.k + 1
    gamma = p.gamma(b)
    T = p.temp(b)
    if T == 0.0:
        replay_greedy_scan(p, b, gamma)
        return
    ngp = min(p.NG, K_SCAN_GROUPS)
    for tid in range(K_THREADS):
        stage_load(p, b, 0, min(K_SCAN_ROWS, gamma), min(K_SCAN_ROWS, gamma), 0, ngp, tid)
    for tid in range(K_THREADS):
        w, l = tid >> 6, tid & 63
        for j0 in range(w, gamma, 2 * K_WAVES):
            for u in range(2):
                j = min(j0 + K_WAVES * u, gamma - 1)
                p.mem.at("tokens", b * p.k + j)
                x = p.clamp_tok(int(p.tokens[b, j]))
                pv = p.draft_prev(b, j) if p.R else -1
                p.row_load("target", b * k1 + j, x, 1, vec=False)
                p.row_load("draft", b * p.k + j, x, 1, vec=False)
                if p.R:
                    r = min(4 * l, max(p.R - 4, 0))
                    p.mem.at("W1", max(pv, 0) * p.R + r, 4)
                    p.mem.at("W2t", x * p.R + r, 4)
    for r0 in range(0, gamma, K_SCAN_ROWS):
        nt = min(K_SCAN_ROWS, gamma - r0)
        for g0 in range(0, p.NG, K_SCAN_GROUPS):
            ng = min(K_SCAN_GROUPS, p.NG - g0)
            if r0 > 0 or g0 > 0:
                for tid in range(K_THREADS):
                    stage_load(p, b, r0, nt, nt, g0, ng, tid)
        for slot in range(2 * K_SCAN_ROWS):
            is_t = slot < K_SCAN_ROWS
            j = r0 + (slot if is_t else slot - K_SCAN_ROWS)
            if j < gamma:
                if is_t:
                    p.mem.at("tm", b * k1 + j); p.mem.at("tl2s", b * k1 + j)
                else:
                    p.mem.at("dm", b * p.k + j); p.mem.at("dl2s", b * p.k + j)
    for j in range(gamma):
        p.mem.at("lpx", b * p.k + j); p.mem.at("lqx", b * p.k + j)
    stop, mask = stop_mask
    p.mem.at("info", 4 * b, 4)
    p.mem.at("rowmask", b)
    if mask:
        p.mem.at("nitems", 0)
    if stop == gamma:
        p.mem.at("nitems", 1)
        assert bonus_slot is not None
        p.mem.at("items", bonus_slot)
    p.mem.at("info2", 4 * b, 2)
    for tid in range(gamma + 1):
        p.mem.at("logP", b * k1 + tid)
    for i in range(gamma):
        if (mask >> i) & 1:
            if p.R:
                p.draft_prev(b, i)
            p.mem.at("items", s_base + bin(mask & ((1 << i) - 1)).count("1"))
    if p.R and mask:
        it = s_base
        for i in range(gamma):
            if not (mask >> i) & 1:
                continue
            for tid in range(4 * p.ks):
                kk, q = tid >> 2, tid & 3
                prev = p.draft_prev(b, i)
                p.mem.at("btile", ((it >> 4) * p.ks + kk) * 64 + (it & 15) + 16 * q)
                if prev >= 0:
                    p.mem.at("W1", prev * p.R + kk * 32 + 8 * q, 8)
            it += 1


# ---------------------------------------------------------------------------
# pass 2: one workgroup per 256-id group; NI listed rows, NB bonus rows
# ---------------------------------------------------------------------------
def w2_slab(p, cb, n, q):
    for s in range(4):
        if p.vec:
            vr = min(cb + 16 * (n >> 2), p.V - 16) + 4 * s + (n & 3)
        else:
            vr = cb + 16 * (n >> 2) + 4 * s + (n & 3)
            vr = vr if vr < p.V else p.V - 1
        for kk in range(p.ks):
            p.mem.at("W2t", vr * p.R + kk * 32 + 8 * q, 8)


def replay_pass2(p: Problem, NI, NB, item_rows):
    """item_rows: (dr, tr) stored at each item slot (stale slots hold anything)."""
    for g in range(p.NG):
        for tid in range(K_THREADS):
            w, l = tid >> 6, tid & 63
            n, q = l & 15, l >> 4
            cb = (g * K_WAVES + w) * K_WAVE_COLS
            cw = cb + 16 * q
            c0 = min(cw, p.V - 16) if p.vec else cw
            if p.R:
                w2_slab(p, cb, n, q)

            def rows_of(c):
                it = min(c * K_CHUNK + n, p.ND - 1)
                p.mem.at("items", it)
                dr, tr = item_rows[it]
                return min(max(dr, 0), p.ND - 1), min(max(tr, 0), p.NT - 1)

            def fetch(h):
                p.row_load("target", h[1], c0)
                p.row_load("draft", h[0], c0)

            fetch(rows_of(0))
            rows_of(1)
            p.mem.at("nitems", 0); p.mem.at("nitems", 1)
            nch = (NI + K_CHUNK - 1) // K_CHUNK
            if p.R and NI > 0:
                for kk in range(p.ks):
                    p.mem.at("btile", l + kk * 64)
            for c in range(nch):
                rows_of(c + 2)
                p.mem.at("items", min(c * K_CHUNK + n, p.ND - 1))
                if p.R:
                    cc = min(c + 1, nch - 1)
                    for kk in range(p.ks):
                        p.mem.at("btile", cc * p.ks * 64 + l + kk * 64)
                fetch(rows_of(c + 1))
                if c % 16 == 15 or c == nch - 1:
                    it = (c - c % 16) * K_CHUNK + tid
                    if tid < (c % 16 + 1) * K_CHUNK and it < NI:
                        p.mem.at("items", it)
                        dr = min(max(item_rows[it][0], 0), p.ND - 1)
                        p.mem.at("wgrp", g * p.ND + dr)
                        p.mem.at("race", g * p.ND + it)
            for c in range((NB + K_CHUNK - 1) // K_CHUNK):
                ib = p.ND - 1 - min(c * K_CHUNK + n, NB - 1)
                p.mem.at("items", ib)
                tr = min(max(item_rows[ib][1], 0), p.NT - 1)
                p.row_load("target", tr, c0)
                if tid < K_CHUNK and c * K_CHUNK + tid < NB:
                    p.mem.at("race", g * p.ND + (p.ND - 1 - (c * K_CHUNK + tid)))


# ---------------------------------------------------------------------------
# finalize: one workgroup per stream
# ---------------------------------------------------------------------------
def replay_finalize(p: Problem, b, method, stop_mask, s_base, bonus_slot, diag=True):
    k1 = p.k + 1
    p.mem.at("info", 4 * b, 4)
    gamma = p.gamma(b)
    stop, mask = stop_mask
    f = 0
    if stop == -1:
        f = (mask & -mask).bit_length() - 1
    p.mem.at("rowmask", b)
    T = p.temp(b)
    if T == 0.0:
        s = gamma   # the scan's stop lies in [0, gamma]; the largest reads the most tokens
        for tid in range(p.k + 1):
            p.mem.at("out_tokens", b * k1 + tid)
            if tid < s:
                p.mem.at("tokens", b * p.k + tid)
            if diag:
                p.mem.at("diag", (b * k1 + tid) * 5, 5)
        p.mem.at("accepted_len", b)
        return
    p.mem.at("info2", 4 * b, 2)
    if method == 1 and stop < 0:
        for i in range(f + 1, gamma):
            if (mask >> i) & 1:
                dr = b * p.k + i
                for g0 in range(0, p.NG, 64 * K_LOADS):
                    for l in range(64):
                        for u in range(K_LOADS):
                            p.mem.at("wgrp", min(g0 + l + 64 * u, p.NG - 1) * p.ND + dr)
                p.mem.at("logP", b * k1 + i)
    # the stop slot: the decided one, or (block) f or any listed row above it
    stops = [stop] if stop >= 0 else [f] + [i for i in range(f + 1, gamma) if (mask >> i) & 1]
    for s in stops:
        tr = b * k1 + s
        dr = b * p.k + (s if s < gamma else 0)
        resid = s < gamma
        it = min(max(s_base + bin(mask & ((1 << s) - 1)).count("1") if resid else bonus_slot, 0), p.ND - 1)
        for tid in range(K_THREADS):
            p.mem.at("race", min(tid, p.NG - 1) * p.ND + it)
            p.mem.at("race", min(tid + K_THREADS, p.NG - 1) * p.ND + it)
            for gi in range(tid + 2 * K_THREADS, p.NG, K_THREADS):
                p.mem.at("race", gi * p.ND + it)
        for v in {0, p.V - 1, p.V // 2}:   # a candidate id is checked 0 <= v < V before use
            p.row_load("target", tr, v, 1, vec=False)
            if resid:
                p.row_load("draft", dr, v, 1, vec=False)
                if p.R:
                    prev = p.draft_prev(b, s)
                    if prev >= 0:
                        p.mem.at("W1", prev * p.R, p.R)
                    p.mem.at("W2t", v * p.R, p.R)
        if resid:
            p.mem.at("tm", tr); p.mem.at("tl2s", tr); p.mem.at("dm", dr); p.mem.at("dl2s", dr)
            if method == 1:
                p.mem.at("logP", tr)
        for v0 in range(0, p.V, 4):   # the full-row fallback
            for i in range(4):
                if v0 + i < p.V:
                    p.mem.at("target", tr * p.V + v0 + i)
        for tid in range(p.k + 1):
            p.mem.at("out_tokens", b * k1 + tid)
            if tid < s:
                p.mem.at("tokens", b * p.k + tid)
            if diag:
                p.mem.at("diag", (b * k1 + tid) * 5, 5)
                if tid <= gamma:
                    p.mem.at("logP", b * k1 + tid)
                if tid < gamma:
                    p.mem.at("lpx", b * p.k + tid); p.mem.at("lqx", b * p.k + tid)
        p.mem.at("accepted_len", b)


# ---------------------------------------------------------------------------
# race clocks: written by the workgroups with no stream to scan, read by pass 2
# ---------------------------------------------------------------------------
def replay_clock_rows(p: Problem, nslots):
    """clock_rows of every slot: an equal share of the B NG rows, 4 rows per wave per turn."""
    rows = p.B * p.NG
    per = (rows + nslots - 1) // nslots
    for slot in range(nslots):
        r0, r1 = slot * per, min(slot * per + per, rows)
        for w in range(K_WAVES):
            for rb in range(r0 + 4 * w, r1, 4 * K_WAVES):
                b, grp = divmod(rb, p.NG)
                for u in range(4):
                    if u > 0:
                        grp += 1
                        while grp >= p.NG:
                            grp -= p.NG
                            b += 1
                    if rb + u < r1:
                        for l in range(64):
                            p.mem.at("clk", min(b, p.B - 1) * p.NG * 64 + grp * 64 + l)


def replay_pass2_clocks(p: Problem, streams):
    """load_clocks of every lane of every group, for the streams pass 2 races."""
    for b in streams:
        sb = min(max(b, 0), p.B - 1)
        for g in range(p.NG):
            for w in range(K_WAVES):
                for q in range(4):
                    cw = (g * K_WAVES + w) * K_WAVE_COLS + 16 * q
                    c0 = min(cw, p.V - 16) if p.vec else cw
                    for i in range(4):
                        p.mem.at("clk", sb * p.NG * 64 + (c0 >> 2) + i)


# ---------------------------------------------------------------------------
# a whole call: list slots assigned as the scan's atomics would, worst cases first
# ---------------------------------------------------------------------------
def replay_call(p: Problem, method, rng, fused_grid=0):
    replay_pack(p, fused_grid)
    choices = []
    for b in range(p.B):
        gamma = p.gamma(b)
        opts = scan_masks(p, b, gamma, method, rng)
        # the fullest list first (largest mask), then a random reachable one
        opts.sort(key=lambda sm: (-bin(sm[1]).count("1"), sm[0] != gamma))
        choices.append(opts[0] if b % 2 == 0 else opts[int(rng.integers(0, len(opts)))])
    NI = sum(bin(m).count("1") for _, m in choices)
    NB = sum(1 for b, (s, m) in enumerate(choices) if s == p.gamma(b))
    assert NI + NB <= p.ND, "listed rows and bonus rows overlap in the item list"
    item_rows = [(int(x), int(y)) for x, y in rng.integers(-5, 10 ** 6, size=(p.ND, 2))]   # stale slots
    base, nb = 0, 0
    slots = []
    for b, (s, m) in enumerate(choices):
        bonus = None
        if s == p.gamma(b):
            bonus = p.ND - 1 - nb
            item_rows[bonus] = (-1, b * (p.k + 1) + s)
            nb += 1
        for i in range(p.k):
            if (m >> i) & 1:
                item_rows[base + bin(m & ((1 << i) - 1)).count("1")] = (b * p.k + i, b * (p.k + 1) + i)
        slots.append((base, bonus))
        replay_scan(p, b, method, (s, m), base, bonus)
        base += bin(m).count("1")
    replay_pass2(p, NI, NB, item_rows)
    replay_clock_rows(p, p.NG)   # the separate scan launch: NG workgroups past the B scanning ones
    if fused_grid > 0:           # the fused launch: the workgroups with no stream, else all of them
        replay_clock_rows(p, fused_grid - p.B if fused_grid > p.B else fused_grid)
    replay_pass2_clocks(p, [-1, 0, p.B - 1, p.B + 3])   # the record's stream is clamped
    for b, (s, m) in enumerate(choices):
        replay_finalize(p, b, method, (s, m), slots[b][0], slots[b][1])
    return p.mem


EDGE = [
    # B, k, V, R, bf16, counts, temps, anchors
    (3, 5, 1000, 256, True, None, None, None),                 # every optional input absent
    (4, 3, 16, 32, False, [0, 3, 1, 0], [1.0, 0.0, 0.7, 0.0], [2, -1, 15, 99]),
    (2, 32, 300, 64, True, [32, 0], [1.0, 0.5], [0, 299]),     # the largest block
    (5, 4, 7, 0, False, [4, 0, 9, -3, 2], None, None),        # V < 16, no Markov, counts out of range
    (3, 6, 333, 128, True, [6, 6, 0], [0.9, 1.0, 1.0], None),  # odd V: bf16 rows not 16-byte multiples
    (2, 5, 513, 32, False, None, [0.0, 1.0], [1, 2]),          # one id past two groups, fp32
    (1, 1, 1, 0, True, None, None, None),                      # one id
    (17, 2, 256, 64, True, [2] * 17, None, None),              # B*k = 34: list spans three chunks
]


@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("method", [0, 1])
def test_every_access_in_bounds(case, method):
    B, k, V, R, bf16, counts, temps, anchors = EDGE[case]
    rng = np.random.default_rng(100 + case)
    toks = rng.integers(-3, V + 3, size=(B, k))   # ids out of range are clamped by the kernels
    p = Problem(B, k, V, R, bf16, counts, temps, anchors, toks, seed=case)
    mem = replay_call(p, method, rng, fused_grid=max(p.NG, B))
    assert mem.count > 0
    # the replay reached the ends of the regions it is meant to cover
    assert mem.hi["target"] >= 0 and mem.hi["draft"] >= 0


# ---------------------------------------------------------------------------
# the withdrawn scan variant
# ---------------------------------------------------------------------------
def variant_gather_rows(p: Problem, b, gamma_used):
    """Token gathers as that variant placed them: waves 0 and 1 gather slots
    16 w + (l & 15) for lanes whose slot is below gamma, clamped to gamma - 1."""
    rows = []
    for tid in range(K_THREADS):
        w, l = tid >> 6, tid & 63
        if not (w < 2 and 16 * w < gamma_used):
            continue
        jg = min(16 * w + (l & 15), max(gamma_used - 1, 0))
        rows.append((b * (p.k + 1) + jg, b * p.k + jg, b * p.k + jg))
    return rows


def test_withdrawn_variant_reads_past_the_logits_when_counts_are_absent():
    """B = 8, k = 5, V = 1000, bf16, counts absent.  With gamma_b = k (the clamped
    value) every gather is in bounds; with the raw word read from the stand-in address
    (the stream's first draft token, an id up to 999) the gathers address target rows
    up to 73 of 48 and draft rows up to 66 of 40, 50 KB past the end of a 96 KB tensor."""
    B, k, V = 8, 5, 1000
    rng = np.random.default_rng(7)
    toks = rng.integers(40, V, size=(B, k))
    p = Problem(B, k, V, 256, True, None, [1.0, 0.0] * 4, list(range(B)), toks)
    for b in range(B):
        for tr, dr, ti in variant_gather_rows(p, b, p.gamma(b)):
            assert tr < p.NT and dr < p.ND and ti < p.B * p.k
    b = B - 1
    raw = int(toks[0, 0])    # the stand-in address is the tokens tensor's first word
    rows = variant_gather_rows(p, b, raw)
    max_tr = max(r[0] for r in rows)
    max_dr = max(r[1] for r in rows)
    assert (max_tr, max_dr) == (b * (k + 1) + 31, b * k + 31) == (73, 66)
    assert max_tr >= p.NT and max_dr >= p.ND
    past = (max_tr + 1) * V * 2 - p.NT * V * 2
    assert past == 52000 and p.NT * V * 2 == 96000
    with pytest.raises(AssertionError):
        for tr, dr, _ in rows:
            p.row_load("target", tr, 0, 1, vec=False)
