"""Python binding of libdspark_verify.so (gfx950 DSpark verify sampler).

Argument marshalling only: every step of the verify path runs in the HIP
kernels behind the C ABI of ``include/dspark_verify.h``.  PyTorch supplies
device memory and the current stream.  There is no fallback: if the built
library is missing, importing a function raises.

bf16 tensors may be passed as ``torch.bfloat16`` or as 16-bit integer tensors
holding the bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdspark_verify.so")

DSPARK_F32 = 0
DSPARK_BF16 = 1
MAX_K = 32
STAGES = 5   # launches per verify call


class VerifyProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("target_logits", ctypes.c_void_p), ("draft_logits", ctypes.c_void_p),
        ("draft_tokens", ctypes.c_void_p), ("num_drafts", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("W2t", ctypes.c_void_p),
        ("anchor_tokens", ctypes.c_void_p), ("R", ctypes.c_int32), ("step", ctypes.c_uint32),
        ("seed", ctypes.c_uint64),
    ]


class VerifyOutputs(ctypes.Structure):
    _fields_ = [("accepted_len", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p), ("diag", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (built by ``python -m draft_block_verification_row_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m draft_block_verification_row_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_uint32
        L.dspark_workspace_bytes.argtypes = [ctypes.POINTER(VerifyProblem)]
        L.dspark_workspace_bytes.restype = sz
        for name in ("dspark_verify_tokenwise", "dspark_verify_block"):
            f = getattr(L, name)
            f.argtypes = [ctypes.POINTER(VerifyProblem), ctypes.POINTER(VerifyOutputs), vp, sz, vp]
            f.restype = i32
        L.dspark_verify_noalloc.argtypes = [ctypes.POINTER(VerifyProblem), ctypes.POINTER(VerifyOutputs), i32, vp]
        L.dspark_verify_noalloc.restype = i32
        L.dspark_draft_sample.argtypes = [ctypes.POINTER(VerifyProblem), vp, vp, vp, sz, vp]
        L.dspark_draft_sample.restype = i32
        L.dspark_draft_launches.argtypes = [ctypes.POINTER(VerifyProblem), ctypes.POINTER(i32)]
        L.dspark_draft_launches.restype = i32
        L.dspark_draft_scatter.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
        L.dspark_draft_scatter.restype = i32
        L.dspark_k_for_batch.argtypes = [vp, i32, i32, i32]
        L.dspark_k_for_batch.restype = i32
        L.dspark_markov_bias.argtypes = [vp, vp, i32, i32, vp, i32, vp, i32, vp, vp]
        L.dspark_markov_bias.restype = i32
        L.dspark_adaptive_k.argtypes = [vp, vp, ctypes.c_float, i32, i32, i32, vp, i32, vp, vp, vp, vp]
        L.dspark_adaptive_k.restype = i32
        L.dspark_schedule_batch.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp, vp]
        L.dspark_schedule_batch.restype = i32
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.dspark_cost_table_create.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(vp)]
        L.dspark_cost_table_create.restype = i32
        L.dspark_cost_table_destroy.argtypes = [vp]
        L.dspark_cost_table_destroy.restype = None
        L.dspark_cost_table_begin.argtypes = [vp, i32, vp]
        L.dspark_cost_table_begin.restype = i32
        L.dspark_cost_table_end.argtypes = [vp, vp]
        L.dspark_cost_table_end.restype = i32
        L.dspark_cost_table_poll.argtypes = [vp, ctypes.POINTER(i32)]
        L.dspark_cost_table_poll.restype = i32
        L.dspark_cost_table_observe.argtypes = [vp, i32, ctypes.c_float]
        L.dspark_cost_table_observe.restype = i32
        L.dspark_cost_table_read.argtypes = [vp, vp, i32]
        L.dspark_cost_table_read.restype = i32
        L.dspark_cost_table_stats.argtypes = [vp, i64p, i64p, ctypes.POINTER(i32)]
        L.dspark_cost_table_stats.restype = i32
        L.dspark_cost_table_log.argtypes = [vp, vp, vp, i32]
        L.dspark_cost_table_log.restype = i32
        L.dspark_random_words.argtypes = [ctypes.c_uint64, u32, u32, u32, u32, i32, i32, vp, vp]
        L.dspark_random_words.restype = i32
        L.dspark_w2_transpose.argtypes = [vp, i32, i32, vp, vp]
        L.dspark_w2_transpose.restype = i32
        L.dspark_verify_launches.argtypes = [vp, vp]
        L.dspark_verify_launches.restype = i32
        L.dspark_status_string.argtypes = [i32]
        L.dspark_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


class DsparkError(RuntimeError):
    pass


def _check(status: int) -> None:
    if status != 0:
        raise DsparkError(f"dspark status {status}: {lib().dspark_status_string(status).decode()}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape, dtypes, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _problem(target, draft, draft_tokens, num_drafts, temperature, W1, W2t, anchor, seed, step):
    if target.dim() != 3:
        raise ValueError("target_logits must be [B, k+1, V]")
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    if target.dtype == torch.float32:
        dt, dts = DSPARK_F32, (torch.float32,)
    elif target.dtype in _BF16:
        dt, dts = DSPARK_BF16, _BF16
    else:
        raise ValueError("logits must be float32 or bf16")
    _need(target, "target_logits", (B, k + 1, V), dts, dev)
    _need(draft, "draft_logits", (B, k, V), dts, dev)
    _need(draft_tokens, "draft_tokens", (B, k), (torch.int32,), dev)
    if num_drafts is not None:
        _need(num_drafts, "num_drafts", (B,), (torch.int32,), dev)
    if temperature is not None:
        _need(temperature, "temperature", (B,), (torch.float32,), dev)
    R = 0
    if W1 is not None:
        if W2t is None:
            raise ValueError("W2t is required with W1")
        R = int(W1.shape[1])
        _need(W1, "W1", (V, R), _BF16, dev)
        _need(W2t, "W2t", (V, R), _BF16, dev)
    if anchor is not None:
        _need(anchor, "anchor_tokens", (B,), (torch.int32,), dev)
    p = VerifyProblem(B=B, k=k, V=V, dtype=dt, target_logits=_ptr(target), draft_logits=_ptr(draft),
                      draft_tokens=_ptr(draft_tokens), num_drafts=_ptr(num_drafts),
                      temperature=_ptr(temperature), W1=_ptr(W1), W2t=_ptr(W2t) if W1 is not None else None,
                      anchor_tokens=_ptr(anchor), R=R, step=int(step) & 0xFFFFFFFF,
                      seed=int(seed) & 0xFFFFFFFFFFFFFFFF)
    return p, (B, k, V)


def workspace_bytes(B: int, k: int, V: int, dtype: int = DSPARK_BF16) -> int:
    p = VerifyProblem(B=B, k=k, V=V, dtype=dtype)
    n = lib().dspark_workspace_bytes(ctypes.byref(p))
    if n == 0:
        raise ValueError("invalid problem sizes")
    return int(n)


def _verify(fname, target, draft, draft_tokens, num_drafts=None, temperature=None, W1=None, W2t=None,
            anchor=None, seed=0, step=0, diag=False, workspace=None, out=None, stage_events=None):
    p, (B, k, V) = _problem(target, draft, draft_tokens, num_drafts, temperature, W1, W2t, anchor, seed, step)
    dev = target.device
    need = lib().dspark_workspace_bytes(ctypes.byref(p))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, k + 1, dtype=torch.int32, device=dev)
        dg = torch.empty(B, k + 1, 5, dtype=torch.float64, device=dev) if diag else None
    else:
        acc, toks, dg = out
    ev = None
    if stage_events is not None:   # DSPARK_STAGES + 1 raw hipEvent_t handles
        ev = (ctypes.c_void_p * len(stage_events))(*stage_events)
    o = VerifyOutputs(accepted_len=_ptr(acc), out_tokens=_ptr(toks), diag=_ptr(dg),
                      stage_events=ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None)
    _check(getattr(lib(), fname)(ctypes.byref(p), ctypes.byref(o), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev)))
    return acc, toks, dg


def verify_launches(target, draft, draft_tokens, num_drafts=None, temperature=None, W1=None, W2t=None,
                    anchor=None) -> int:
    """Launches a verify call of this problem makes on the current device (2 or 5)."""
    p, _ = _problem(target, draft, draft_tokens, num_drafts, temperature, W1, W2t, anchor, 0, 0)
    n = ctypes.c_int32(0)
    _check(lib().dspark_verify_launches(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def verify_tokenwise(target, draft, draft_tokens, **kw):
    """Token-by-token verification; returns (accepted_len [B], out_tokens [B, k+1], diag or None)."""
    return _verify("dspark_verify_tokenwise", target, draft, draft_tokens, **kw)


def verify_block(target, draft, draft_tokens, **kw):
    """Block verification; returns (accepted_len [B], out_tokens [B, k+1], diag or None)."""
    return _verify("dspark_verify_block", target, draft, draft_tokens, **kw)


def random_words(seed: int, b: int, purpose: int, step: int, idx0: int, n: int, kind: int, device="cuda:0"):
    """The generator words a call draws (kind 0: word 0 of counter (b, idx0 + i, purpose,
    step); kind 1: word idx0 + i of the stream of (b, purpose, step)); uint32 as int32 [n]."""
    dev = torch.device(device)
    out = torch.empty(n, dtype=torch.int32, device=dev)
    _check(lib().dspark_random_words(int(seed) & 0xFFFFFFFFFFFFFFFF, int(b) & 0xFFFFFFFF, int(purpose) & 0xFFFFFFFF,
                                     int(step) & 0xFFFFFFFF, int(idx0) & 0xFFFFFFFF, int(n), int(kind), _ptr(out),
                                     _stream(dev)))
    return out


def w2_transpose(W2, out=None):
    """W2 [R, V] bf16 -> W2t [V, R] bf16 (the layout the verify problem takes), one launch."""
    if W2.dim() != 2:
        raise ValueError("W2 must be [R, V]")
    R, V = W2.shape
    dev = W2.device
    _need(W2, "W2", (R, V), _BF16, dev)
    out = torch.empty(V, R, dtype=W2.dtype, device=dev) if out is None else out
    _need(out, "out", (V, R), _BF16, dev)
    _check(lib().dspark_w2_transpose(_ptr(W2), R, V, _ptr(out), _stream(dev)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20
_METHODS = {"tokenwise": 0, "block": 1}


def verify_noalloc(method, target, draft, draft_tokens, num_drafts=None, temperature=None, W1=None, W2t=None,
                   anchor=None, seed=0, step=0, diag=False, out=None):
    """Either verifier on the library's static per-device scratch (no workspace, no
    allocation inside the call).  ``method`` is "tokenwise" or "block".  Output
    tensors are allocated here unless ``out`` = (accepted_len, out_tokens, diag or
    None) is given.  Calls that overlap on one device race on the shared scratch."""
    if method not in _METHODS:
        raise ValueError(f"method must be one of {sorted(_METHODS)}")
    p, (B, k, V) = _problem(target, draft, draft_tokens, num_drafts, temperature, W1, W2t, anchor, seed, step)
    dev = target.device
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, k + 1, dtype=torch.int32, device=dev)
        dg = torch.empty(B, k + 1, 5, dtype=torch.float64, device=dev) if diag else None
    else:
        acc, toks, dg = out
    o = VerifyOutputs(accepted_len=_ptr(acc), out_tokens=_ptr(toks), diag=_ptr(dg), stage_events=None)
    _check(lib().dspark_verify_noalloc(ctypes.byref(p), ctypes.byref(o), _METHODS[method], _stream(dev)))
    return acc, toks, dg


def _walk_problem(draft, num_drafts, temperature, W1, W2t, anchor, seed, step):
    if draft.dim() != 3:
        raise ValueError("draft_logits must be [B, k, V]")
    B, k, V = draft.shape
    dev = draft.device
    if draft.dtype == torch.float32:
        dt, dts = DSPARK_F32, (torch.float32,)
    elif draft.dtype in _BF16:
        dt, dts = DSPARK_BF16, _BF16
    else:
        raise ValueError("logits must be float32 or bf16")
    _need(draft, "draft_logits", (B, k, V), dts, dev)
    if num_drafts is not None:
        _need(num_drafts, "num_drafts", (B,), (torch.int32,), dev)
    if temperature is not None:
        _need(temperature, "temperature", (B,), (torch.float32,), dev)
    R = 0
    if W1 is not None:
        if W2t is None:
            raise ValueError("W2t is required with W1")
        R = int(W1.shape[1])
        _need(W1, "W1", (V, R), _BF16, dev)
        _need(W2t, "W2t", (V, R), _BF16, dev)
    if anchor is not None:
        _need(anchor, "anchor_tokens", (B,), (torch.int32,), dev)
    return VerifyProblem(B=B, k=k, V=V, dtype=dt, target_logits=None, draft_logits=_ptr(draft), draft_tokens=None,
                         num_drafts=_ptr(num_drafts), temperature=_ptr(temperature), W1=_ptr(W1),
                         W2t=_ptr(W2t) if W1 is not None else None, anchor_tokens=_ptr(anchor), R=R,
                         step=int(step) & 0xFFFFFFFF, seed=int(seed) & 0xFFFFFFFFFFFFFFFF)


def draft_sample(draft, num_drafts=None, temperature=None, W1=None, W2t=None, anchor=None, seed=0, step=0,
                 logq=False, workspace=None, out=None):
    """The drafter's Markov walk: x_j ~ softmax((d_j + W1[x_{j-1}] W2)/T) slot by slot.

    draft [B, k, V]; returns (tokens [B, k] int32 with -1 past gamma_b, log q_j(x_j) [B, k] fp64 or None).
    """
    p = _walk_problem(draft, num_drafts, temperature, W1, W2t, anchor, seed, step)
    B, k, _ = draft.shape
    dev = draft.device
    need = lib().dspark_workspace_bytes(ctypes.byref(p))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    toks = torch.empty(B, k, dtype=torch.int32, device=dev) if out is None else out
    _need(toks, "tokens_out", (B, k), (torch.int32,), dev)
    lq = torch.empty(B, k, dtype=torch.float64, device=dev) if logq else None
    _check(lib().dspark_draft_sample(ctypes.byref(p), _ptr(toks), _ptr(lq), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(dev)))
    return toks, lq


def draft_launches(draft, num_drafts=None, temperature=None, W1=None, W2t=None, anchor=None) -> int:
    """Launches a walk of this problem makes on the current device (2, or 2 k)."""
    p = _walk_problem(draft, num_drafts, temperature, W1, W2t, anchor, 0, 0)
    n = ctypes.c_int32(0)
    _check(lib().dspark_draft_launches(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def draft_scatter(reduced, vocab_ids, V: int, out=None):
    """Scatter reduced-vocabulary draft logits [..., K] into [..., V] columns, -inf elsewhere."""
    dev = reduced.device
    K = int(reduced.shape[-1])
    rows = int(reduced.numel() // K) if K else 0
    if reduced.dtype == torch.float32:
        dt, dts = DSPARK_F32, (torch.float32,)
    elif reduced.dtype in _BF16:
        dt, dts = DSPARK_BF16, _BF16
    else:
        raise ValueError("logits must be float32 or bf16")
    _need(reduced, "reduced", tuple(reduced.shape), dts, dev)
    _need(vocab_ids, "vocab_ids", (K,), (torch.int32,), dev)
    if out is None:
        out = torch.empty(*reduced.shape[:-1], V, dtype=reduced.dtype, device=dev)
    _need(out, "out", tuple(reduced.shape[:-1]) + (V,), dts, dev)
    _check(lib().dspark_draft_scatter(_ptr(reduced), _ptr(vocab_ids), rows, K, V, dt, _ptr(out), _stream(dev)))
    return out


def k_for_batch(schedule, batch: int, k_default: int) -> int:
    """Draft count for a batch size from (lo, hi, k) triples, e.g. [[1, 4, 5], [5, 8, 3], [9, 32, 3]]."""
    flat = [int(x) for t in schedule for x in t]
    arr = (ctypes.c_int32 * len(flat))(*flat)
    return int(lib().dspark_k_for_batch(ctypes.cast(arr, ctypes.c_void_p), len(schedule), int(batch), int(k_default)))


def markov_bias(W1, W2t, prev_tokens, logits_in=None, out=None):
    """out[i] = logits_in[i] + W1[prev_tokens[i]] . W2 (fp32 [rows, V])."""
    dev = W1.device
    V, R = W1.shape
    rows = int(prev_tokens.shape[0])
    _need(W1, "W1", (V, R), _BF16, dev)
    _need(W2t, "W2t", (V, R), _BF16, dev)
    _need(prev_tokens, "prev_tokens", (rows,), (torch.int32,), dev)
    dt = DSPARK_F32
    if logits_in is not None:
        dt = DSPARK_F32 if logits_in.dtype == torch.float32 else DSPARK_BF16
        _need(logits_in, "logits_in", (rows, V), (torch.float32,) + _BF16, dev)
    if out is None:
        out = torch.empty(rows, V, dtype=torch.float32, device=dev)
    _need(out, "out", (rows, V), (torch.float32,), dev)
    _check(lib().dspark_markov_bias(_ptr(W1), _ptr(W2t), V, R, _ptr(prev_tokens), rows, _ptr(logits_in), dt,
                                    _ptr(out), _stream(dev)))
    return out


def adaptive_k(hidden, w, bias: float, verify_ms, want_c: bool = True):
    """Confidence head + adaptive count; returns (n [B] int32, c [B, k], a [B, k])."""
    dev = hidden.device
    B, k, H = hidden.shape
    _need(hidden, "hidden", (B, k, H), _BF16, dev)
    _need(w, "w", (H,), _BF16, dev)
    ms = (ctypes.c_float * len(verify_ms))(*[float(x) for x in verify_ms])
    n = torch.empty(B, dtype=torch.int32, device=dev)
    c = torch.empty(B, k, dtype=torch.float32, device=dev) if want_c else None
    a = torch.empty(B, k, dtype=torch.float32, device=dev) if want_c else None
    _check(lib().dspark_adaptive_k(_ptr(hidden), _ptr(w), float(bias), B, k, H, ctypes.cast(ms, ctypes.c_void_p),
                                   len(verify_ms), _ptr(n), _ptr(c), _ptr(a), _stream(dev)))
    return n, c, a


MAX_SCHEDULE = 4096


def schedule_batch(c, verify_ms, n_out=None, total_out=None, expected_out=None):
    """Batch-level scheduler: per-stream draft counts for one verify batch.

    c: [B, k] fp32 confidences on the GPU; verify_ms: fp32 cost table on the same
    device indexed by the batch's token count (at least B (k + 1) + 1 entries).
    Returns (n [B] int32, total tokens [1] int32, expected accepted tokens [1]
    fp64), all device tensors; no host synchronisation.
    """
    dev = c.device
    B, k = c.shape
    _need(c, "c", (B, k), (torch.float32,), dev)
    _need(verify_ms, "verify_ms", None, (torch.float32,), dev)
    if verify_ms.dim() != 1:
        raise ValueError("verify_ms must be 1-D")
    n = torch.empty(B, dtype=torch.int32, device=dev) if n_out is None else n_out
    _need(n, "n_out", (B,), (torch.int32,), dev)
    total = torch.empty(1, dtype=torch.int32, device=dev) if total_out is None else total_out
    expected = torch.empty(1, dtype=torch.float64, device=dev) if expected_out is None else expected_out
    _need(total, "total_out", (1,), (torch.int32,), dev)
    _need(expected, "expected_out", (1,), (torch.float64,), dev)
    _check(lib().dspark_schedule_batch(_ptr(c), B, k, _ptr(verify_ms), verify_ms.numel(), _ptr(n), _ptr(total),
                                       _ptr(expected), _stream(dev)))
    return n, total, expected


class CostTable:
    """Online verify-cost table: boot curve + live medians of timed verify steps.

    Bracket each pure verify step with ``begin(num_tokens)`` / ``end()`` on the
    stream it runs on; completed timings are read back by ``poll()`` (or the next
    ``begin``) without waiting on the GPU.
    """

    def __init__(self, boot_ms, window: int = 32, min_samples: int = 3, rebuild_every: int = 32):
        boot = [float(x) for x in boot_ms]
        arr = (ctypes.c_float * len(boot))(*boot)
        h = ctypes.c_void_p()
        self._h = None
        _check(lib().dspark_cost_table_create(ctypes.cast(arr, ctypes.c_void_p), len(boot), window, min_samples,
                                              rebuild_every, ctypes.byref(h)))
        self._h = h
        self.n = len(boot)

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.dspark_cost_table_destroy(self._h)
            self._h = None

    def begin(self, num_tokens: int, stream=None) -> None:
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
        _check(lib().dspark_cost_table_begin(self._h, int(num_tokens), st))

    def end(self, stream=None) -> None:
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
        _check(lib().dspark_cost_table_end(self._h, st))

    def poll(self) -> int:
        n = ctypes.c_int32(0)
        _check(lib().dspark_cost_table_poll(self._h, ctypes.byref(n)))
        return n.value

    def observe(self, num_tokens: int, ms: float) -> None:
        _check(lib().dspark_cost_table_observe(self._h, int(num_tokens), float(ms)))

    def table(self):
        import numpy as np
        out = np.empty(self.n, dtype=np.float32)
        _check(lib().dspark_cost_table_read(self._h, out.ctypes.data, self.n))
        return out

    def stats(self):
        f, d, q = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
        _check(lib().dspark_cost_table_stats(self._h, ctypes.byref(f), ctypes.byref(d), ctypes.byref(q)))
        return dict(filed=f.value, dropped=d.value, in_flight=q.value)

    def log(self):
        import numpy as np
        cap = 65536
        t = np.empty(cap, dtype=np.int32)
        m = np.empty(cap, dtype=np.float32)
        n = lib().dspark_cost_table_log(self._h, t.ctypes.data, m.ctypes.data, cap)
        return t[:n].copy(), m[:n].copy()
