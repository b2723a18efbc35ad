"""The launch plan a verify call reports, and the two plans' agreement: a call whose
stages run as phases of one resident launch returns exactly what the same call returns
with one launch per stage."""
import os

import numpy as np
import pytest

import workloads
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mod():
    import draft_block_verification_row_amd as m
    m.lib()
    return m


def _plan(mod, dev):
    return mod.verify_launches(dev["target"], dev["draft"], dev["draft_tokens"], num_drafts=dev["num_drafts"],
                               temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"], anchor=dev["anchor"])


def test_reported_plans(mod):
    h = H.to_dev(workloads.make("h", B=4))
    assert _plan(mod, h) == 2
    odd = H.to_dev(workloads.make("h", V=333, B=4))   # bf16 rows of 666 bytes: no 16-byte vectors
    assert _plan(mod, odd) == 5
    os.environ["DSPARK_VERIFY_LAUNCH"] = "separate"
    try:
        assert _plan(mod, h) == 5
    finally:
        del os.environ["DSPARK_VERIFY_LAUNCH"]


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_fused_and_separate_launches_agree(mod, method):
    wl = workloads.make_zipf("plan", seed=9, B=24, k=5, V=12000, dtype="bf16", greedy_every=5)
    wl.num_drafts = np.array([5, 0, 3] * 8, dtype=np.int32)
    dev = H.to_dev(wl)
    assert _plan(mod, dev) == 2
    for step in range(3):
        a = H.run_gpu(mod, dev, method, wl.seed, step)
        os.environ["DSPARK_VERIFY_LAUNCH"] = "separate"
        try:
            b = H.run_gpu(mod, dev, method, wl.seed, step)
        finally:
            del os.environ["DSPARK_VERIFY_LAUNCH"]
        assert np.array_equal(a["accepted_len"], b["accepted_len"])
        assert np.array_equal(a["out_tokens"], b["out_tokens"])
        assert np.array_equal(a["diag"], b["diag"], equal_nan=True)
