"""The C ABI: the library loads, exports every function the header declares, and the
binding's struct layouts match the header's (checked with the host C compiler).
No compute call is made (no GPU needed)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark_verify.h")


def _built_lib():
    import draft_block_verification_row_amd as m
    if not os.path.exists(m.LIB_PATH):
        from draft_block_verification_row_amd import build
        build.build()
    return m


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("dspark_verify_tokenwise", "dspark_verify_block", "dspark_markov_bias", "dspark_adaptive_k",
              "dspark_draft_sample", "dspark_draft_scatter", "dspark_k_for_batch", "dspark_workspace_bytes",
              "dspark_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    m = _built_lib()
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    L = m.lib()
    for n in _declared_functions():
        assert hasattr(L, n)


def test_struct_layout_matches_header():
    m = _built_lib()
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "dspark_verify.h"
#define P(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("problem %zu\n", sizeof(dspark_verify_problem));
  printf("outputs %zu\n", sizeof(dspark_verify_outputs));
  P(dspark_verify_problem, B) P(dspark_verify_problem, k) P(dspark_verify_problem, V)
  P(dspark_verify_problem, dtype) P(dspark_verify_problem, target_logits) P(dspark_verify_problem, draft_logits)
  P(dspark_verify_problem, draft_tokens) P(dspark_verify_problem, num_drafts) P(dspark_verify_problem, temperature)
  P(dspark_verify_problem, W1) P(dspark_verify_problem, W2t) P(dspark_verify_problem, anchor_tokens)
  P(dspark_verify_problem, R) P(dspark_verify_problem, step) P(dspark_verify_problem, seed)
  P(dspark_verify_outputs, accepted_len) P(dspark_verify_outputs, out_tokens) P(dspark_verify_outputs, diag)
  P(dspark_verify_outputs, stage_events)
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.rsplit(" ", 1) for l in lines if l.strip())
    assert int(got["problem"]) == ctypes.sizeof(m.VerifyProblem)
    assert int(got["outputs"]) == ctypes.sizeof(m.VerifyOutputs)
    for name, _ in m.VerifyProblem._fields_:
        assert int(got[f"dspark_verify_problem.{name}"]) == getattr(m.VerifyProblem, name).offset, name
    for name, _ in m.VerifyOutputs._fields_:
        assert int(got[f"dspark_verify_outputs.{name}"]) == getattr(m.VerifyOutputs, name).offset, name


def test_host_side_errors_without_gpu():
    """Host-checkable preconditions return a status before anything is enqueued."""
    m = _built_lib()
    L = m.lib()
    p = m.VerifyProblem(B=0, k=5, V=100, dtype=1)
    assert L.dspark_workspace_bytes(ctypes.byref(p)) == 0
    p = m.VerifyProblem(B=2, k=33, V=100, dtype=1)
    assert L.dspark_workspace_bytes(ctypes.byref(p)) == 0
    p = m.VerifyProblem(B=2, k=5, V=100, dtype=1)
    assert L.dspark_workspace_bytes(ctypes.byref(p)) > 0
    o = m.VerifyOutputs()
    # NULL logits -> invalid argument (1)
    assert L.dspark_verify_block(ctypes.byref(p), ctypes.byref(o), None, 0, None) == 1
    # workspace missing -> workspace error (3)
    p.target_logits = p.draft_logits = p.draft_tokens = 256
    o.accepted_len = o.out_tokens = 256
    assert L.dspark_verify_tokenwise(ctypes.byref(p), ctypes.byref(o), None, 0, None) == 3
    # unsupported rank (2)
    p.W1 = p.W2t = 256
    p.R = 48
    assert L.dspark_verify_block(ctypes.byref(p), ctypes.byref(o), 256, 1 << 30, None) == 2
    assert L.dspark_status_string(4) == b"HIP launch failed"
    # adaptive: verify_ms too short (needs k + 2 entries)
    ms = (ctypes.c_float * 3)(1.0, 2.0, 3.0)
    assert L.dspark_adaptive_k(256, 256, 0.0, 4, 5, 16, ctypes.cast(ms, ctypes.c_void_p), 3, 256, None, None,
                               None) == 1
    # draft walk: no output buffer (1), no workspace (3), unsupported rank (2)
    q = m.VerifyProblem(B=2, k=5, V=100, dtype=1, draft_logits=256)
    assert L.dspark_draft_sample(ctypes.byref(q), None, None, 256, 1 << 30, None) == 1
    assert L.dspark_draft_sample(ctypes.byref(q), 256, None, None, 0, None) == 3
    q.W1 = q.W2t = 256
    q.R = 48
    assert L.dspark_draft_sample(ctypes.byref(q), 256, None, 256, 1 << 30, None) == 2


def test_k_for_batch_schedule():
    """The pages' production schedule [[1, 4, 5], [5, 8, 3], [9, 32, 3]] (host only)."""
    m = _built_lib()
    sched = [[1, 4, 5], [5, 8, 3], [9, 32, 3]]
    assert [m.k_for_batch(sched, b, 2) for b in (1, 4, 5, 8, 9, 32, 33)] == [5, 5, 3, 3, 3, 3, 2]
    assert m.k_for_batch([], 7, 4) == 4


def test_draft_scatter_host_errors():
    m = _built_lib()
    L = m.lib()
    assert L.dspark_draft_scatter(None, 256, 2, 4, 10, 1, 256, None) == 1
    assert L.dspark_draft_scatter(256, 256, 2, 11, 10, 1, 256, None) == 1   # K > V
    assert L.dspark_draft_scatter(256, 256, 0, 4, 10, 1, 256, None) == 0    # nothing to do


def test_stream_read_library_loads():
    """The measured-read-ceiling library beside the sampler builds, loads and exports
    its one function; argument checks run on the host (no launch)."""
    m = _built_lib()
    path = os.path.join(os.path.dirname(m.LIB_PATH), "libdspark_stream_read.so")
    if not os.path.exists(path):
        from draft_block_verification_row_amd import build
        build.build()
    L = ctypes.CDLL(path)
    f = L.dspark_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(None, 16, 1, 16, None) == 1            # null source
    assert f(16, 24, 1, 16, None) == 1              # size not a multiple of 16
    assert f(16, 16, 0, 16, None) == 1              # empty grid
    assert f(16, 0, 1, 16, None) == 0               # nothing to read: no launch
