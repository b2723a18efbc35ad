"""Seeded synthetic workloads for the verify sampler.

This module only *makes inputs*: logits, draft tokens, Markov factors,
temperatures, confidence-head inputs and the verify-cost table.  It holds none
of the verification arithmetic (no softmax normaliser, no acceptance test, no
residual, no sampler) and both the HIP path's tests and the CPU oracle read the
same arrays from it.

Recipes (every array comes from numpy PCG64 with the listed seed):

* ``c1``  B=4, k=3, V=16, fp32.  target ~ N(0, 2^2); draft = 0.8*target + 0.6*N(0, 2^2);
  no Markov bias; T = 1.
* ``c2``  B=1, k=5, V=129280, fp32.  target = N(0, 3^2) - 1.1*ln(rank) with a
  seeded per-stream rank permutation (a Zipf(s=1.1) rank bias); draft =
  rho*target + sqrt(1-rho^2)*N(0, 3^2) with rho = 0.7; W1, W2 bf16 ~ N(0, 0.02^2);
  anchor ~ U[0, V); T = 1.
* ``c3``  B=16, k=5, V=129280, bf16, the c2 recipe with rho_b ~ U[0.3, 0.95] and
  T_b ~ U[0.6, 1.0] per stream.
* ``h``   B=64, k=5, V=129280, bf16, the c3 recipe (the headline shape).
* ``c4``  B=64, k=9, V=129280, bf16, rho_j = 0.9*0.85^j for slot j, T = 1.
* ``c5``  B=256, k=5, V=129280, bf16, the c3 recipe plus a confidence head:
  hidden [B, k, 4096] bf16 ~ N(0, 1), w [4096] bf16 ~ N(0, 1/4096), bias +1.0,
  verify_ms[t] = 10 + 2.4 t for t = 0..63.

Draft tokens are drawn slot by slot with the Gumbel-max trick on the *stored*
draft logits divided by T (x_j = argmax_v d_j(v)/T + G_v, G Gumbel noise from
PCG64).  Where the Markov bias is on, the draw ignores it: the bias has a
standard deviation of about 0.006 nats against logits of scale 3, so the draws
stay close to the drafter's distribution.  The verifier's outputs are a
deterministic function of the tokens it is handed, so parity does not depend on
this choice; where exact draft statistics matter (``c1``, no Markov bias) the
draw is exactly from the drafter's distribution.

Storage: bf16 tensors are returned as ``uint16`` arrays holding the bf16 bit
patterns (round to nearest even from float32), fp32 tensors as ``float32``.
``W2t`` is the [V, R] row-major storage of the math factor W2 [R, V]
(``W2t[v, r] = W2[r, v]``), the layout a linear layer keeps its weight in.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

V_FULL = 129280
RANK = 256
HIDDEN = 4096


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even) and return the 16-bit patterns."""
    import torch  # CPU conversion only: torch rounds float32 -> bfloat16 to nearest even
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    B: int
    k: int
    V: int
    dtype: str                      # "f32" or "bf16": storage of both logit tensors
    target: np.ndarray              # [B, k+1, V]
    draft: np.ndarray               # [B, k, V]
    draft_tokens: np.ndarray        # [B, k] int32
    temperature: np.ndarray         # [B] float32
    anchor: np.ndarray              # [B] int32, -1 = slot 0 unbiased
    W1: Optional[np.ndarray] = None   # [V, R] uint16 (bf16)
    W2t: Optional[np.ndarray] = None  # [V, R] uint16 (bf16), W2t[v, r] = W2[r, v]
    num_drafts: Optional[np.ndarray] = None  # [B] int32 or None (= k)
    seed: int = 0
    step: int = 0
    hidden: Optional[np.ndarray] = None      # [B, k, H] uint16 (bf16)
    conf_w: Optional[np.ndarray] = None      # [H] uint16 (bf16)
    conf_b: float = 0.0
    verify_ms: Optional[np.ndarray] = None   # [n_ms] float32
    meta: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return 0 if self.W1 is None else int(self.W1.shape[1])

    def logits_f32(self, which: str) -> np.ndarray:
        arr = self.target if which == "target" else self.draft
        return bf16_bits_to_f32(arr) if self.dtype == "bf16" else arr

    def with_step(self, step: int) -> "Workload":
        return replace(self, step=int(step))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _gumbel_drafts(rng: np.random.Generator, draft_f32: np.ndarray, temperature: np.ndarray) -> np.ndarray:
    """x_j = argmax_v(d_j(v)/T + Gumbel), one slot at a time, from PCG64 noise."""
    B, k, V = draft_f32.shape
    toks = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        for j in range(k):
            u = rng.random(V)
            u = np.clip(u, 1e-300, 1.0 - 1e-16)
            g = -np.log(-np.log(u))
            toks[b, j] = int(np.argmax(draft_f32[b, j].astype(np.float64) / float(temperature[b]) + g))
    return toks


def _zipf_target(rng: np.random.Generator, rows: int, V: int, sigma: float, zipf_s: float) -> np.ndarray:
    rank = rng.permutation(V).astype(np.float64) + 1.0
    base = rng.standard_normal((rows, V), dtype=np.float32) * np.float32(sigma)
    return base - np.float32(zipf_s) * np.log(rank).astype(np.float32)[None, :]


def make_tiny(seed: int = 1, B: int = 4, k: int = 3, V: int = 16, rho: float = 0.8,
              sigma: float = 2.0) -> Workload:
    """The exhaustive-check shape: fp32 logits, no Markov bias, T = 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    target = (rng.standard_normal((B, k + 1, V)) * sigma).astype(np.float32)
    noise = (rng.standard_normal((B, k, V)) * sigma).astype(np.float32)
    draft = (rho * target[:, :k].astype(np.float64) + np.sqrt(1 - rho * rho) * noise).astype(np.float32)
    temperature = np.ones(B, dtype=np.float32)
    toks = _gumbel_drafts(rng, draft, temperature)
    return Workload(name="c1", B=B, k=k, V=V, dtype="f32", target=target, draft=draft,
                    draft_tokens=toks, temperature=temperature,
                    anchor=np.full(B, -1, dtype=np.int32), seed=seed, step=0)


def make_zipf(name: str, seed: int, B: int, k: int, V: int = V_FULL, dtype: str = "bf16",
              rho=(0.3, 0.95), temp=(0.6, 1.0), markov: bool = True, R: int = RANK,
              sigma: float = 3.0, zipf_s: float = 1.1, rho_per_slot=None,
              confidence: bool = False, H: int = HIDDEN, greedy_every: int = 0,
              draft_vocab: int = 0) -> Workload:
    """Zipf-biased Gaussian target logits with a correlated draft (c2..c5 recipes).

    ``rho`` / ``temp`` are a fixed value or a (lo, hi) range drawn per stream;
    ``rho_per_slot`` (length k) overrides rho slot by slot.  ``greedy_every`` = m > 0
    sets T = 0 on every m-th stream (mixed batches); such a stream's drafts copy the
    position of the target row's largest logit with probability 3/4 and of the draft
    row's otherwise, so that greedy blocks are partly kept.  ``draft_vocab`` = K > 0
    gives the drafter a reduced vocabulary: a seeded set of K ids keeps its draft
    logits and every other id gets -inf (the drafter's logits scattered into the
    target's columns); ``meta["draft_vocab"]`` holds the sorted ids.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    target = np.empty((B, k + 1, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    draft = np.empty((B, k, V), dtype=target.dtype)
    rhos = np.empty((B, k), dtype=np.float64)
    temperature = np.empty(B, dtype=np.float32)
    for b in range(B):
        if rho_per_slot is not None:
            rhos[b] = np.asarray(rho_per_slot, dtype=np.float64)
        elif isinstance(rho, tuple):
            rhos[b] = rng.uniform(rho[0], rho[1])
        else:
            rhos[b] = float(rho)
        temperature[b] = np.float32(rng.uniform(temp[0], temp[1]) if isinstance(temp, tuple) else temp)
        t = _zipf_target(rng, k + 1, V, sigma, zipf_s)
        noise = rng.standard_normal((k, V), dtype=np.float32) * np.float32(sigma)
        r = rhos[b][:, None].astype(np.float32)
        d = r * t[:k] + np.sqrt(1.0 - r * r) * noise
        if draft_vocab > 0:
            if b == 0:
                keep = np.zeros(V, dtype=bool)
                keep[rng.choice(V, size=draft_vocab, replace=False)] = True
            d = np.where(keep[None, :], d, np.float32(-np.inf)).astype(np.float32)
        target[b] = _store(t, dtype)
        draft[b] = _store(d, dtype)
    stored_draft = bf16_bits_to_f32(draft) if dtype == "bf16" else draft
    greedy = np.zeros(B, dtype=bool)
    if greedy_every > 0:
        greedy[::greedy_every] = True
        temperature[greedy] = 0.0
    toks = _gumbel_drafts(rng, stored_draft, np.where(greedy, 1.0, temperature).astype(np.float32))
    if greedy.any():
        stored_target = bf16_bits_to_f32(target) if dtype == "bf16" else target
        for b in np.nonzero(greedy)[0]:
            for j in range(k):
                src = stored_target[b, j] if rng.random() < 0.75 else stored_draft[b, j]
                toks[b, j] = int(np.argmax(src))
    anchor = rng.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    W1 = W2t = None
    if markov:
        W1 = f32_to_bf16_bits(rng.standard_normal((V, R), dtype=np.float32) * np.float32(0.02))
        W2t = f32_to_bf16_bits(rng.standard_normal((V, R), dtype=np.float32) * np.float32(0.02))
    wl = Workload(name=name, B=B, k=k, V=V, dtype=dtype, target=target, draft=draft,
                  draft_tokens=toks, temperature=temperature, anchor=anchor, W1=W1, W2t=W2t,
                  seed=seed, step=0, meta={"rho": rhos})
    if draft_vocab > 0:
        wl.meta["draft_vocab"] = np.nonzero(keep)[0].astype(np.int32)
    if confidence:
        wl.hidden = f32_to_bf16_bits(rng.standard_normal((B, k, H), dtype=np.float32))
        wl.conf_w = f32_to_bf16_bits(rng.standard_normal(H, dtype=np.float32) / np.float32(np.sqrt(H)))
        wl.conf_b = 1.0
        wl.verify_ms = (10.0 + 2.4 * np.arange(64)).astype(np.float32)
    return wl


def make(name: str, V: Optional[int] = None, B: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    """Named configurations; ``V``/``B``/``seed`` shrink or reseed a recipe for small tests."""
    name = name.lower()
    if name == "c1":
        return make_tiny(seed=1 if seed is None else seed)
    if name == "c2":
        return make_zipf("c2", 2 if seed is None else seed, B or 1, 5, V or V_FULL, "f32", rho=0.7, temp=1.0)
    if name == "c3":
        return make_zipf("c3", 3 if seed is None else seed, B or 16, 5, V or V_FULL, "bf16")
    if name == "h":
        return make_zipf("h", 64 if seed is None else seed, B or 64, 5, V or V_FULL, "bf16")
    if name == "h_nomarkov":
        return make_zipf("h_nomarkov", 64 if seed is None else seed, B or 64, 5, V or V_FULL, "bf16",
                         markov=False)
    if name == "c4":
        return make_zipf("c4", 4 if seed is None else seed, B or 64, 9, V or V_FULL, "bf16", temp=1.0,
                         rho_per_slot=[0.9 * 0.85 ** j for j in range(9)])
    if name == "c5":
        return make_zipf("c5", 5 if seed is None else seed, B or 256, 5, V or V_FULL, "bf16",
                         confidence=True)
    raise KeyError(name)


def full_input_bytes(wl: Workload) -> int:
    """Bytes of every input tensor one verify call may read (logits, W2, gathered W1 rows)."""
    e = 2 if wl.dtype == "bf16" else 4
    n = e * wl.V * wl.B * (2 * wl.k + 1)
    if wl.W1 is not None:
        n += 2 * wl.V * wl.R + 2 * wl.R * wl.B * wl.k
    return n
