"""Host logic of the online cost table and the scheduler's argument checks (no GPU).

The cost table's filing, windows, medians and rebuild cadence run on the host;
``observe`` files a time without any HIP call, so the library's table can be
compared with the oracle's bit for bit here.
"""
import ctypes
import os

import numpy as np
import pytest

from oracle import schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _m():
    import draft_block_verification_row_amd as m
    if not os.path.exists(m.LIB_PATH):
        from draft_block_verification_row_amd import build
        build.build()
    return m


@pytest.mark.parametrize("window,min_samples,rebuild_every,seed", [
    (32, 3, 32, 0), (32, 3, 32, 1), (5, 2, 7, 2), (1, 1, 1, 3), (8, 8, 3, 4)])
def test_observed_table_matches_oracle(window, min_samples, rebuild_every, seed):
    m = _m()
    g = np.random.default_rng(seed)
    n = 40
    boot = (10.0 + 2.4 * np.arange(n)).astype(np.float32)
    t = m.CostTable(boot, window=window, min_samples=min_samples, rebuild_every=rebuild_every)
    obs = []
    for i in range(700):
        tok = int(g.choice([3, 4, 5, 9, 17, 39, 40, -2])) if i % 5 else int(g.integers(0, n))
        ms = float(np.float32(g.uniform(0.5, 30.0)))
        obs.append((tok, ms))
        t.observe(tok, ms)
        if i % 37 == 0:
            _, hist = schedule.online_table(boot, obs, window, min_samples, rebuild_every)
            assert np.array_equal(t.table(), hist[-1]), i
    table, _ = schedule.online_table(boot, obs, window, min_samples, rebuild_every)
    assert np.array_equal(t.table(), table)
    filed = [(a, b) for (a, b) in obs if 0 <= a < n]
    st = t.stats()
    assert st["filed"] == len(filed) and st["dropped"] == len(obs) - len(filed) and st["in_flight"] == 0
    lt, lm = t.log()
    assert lt.tolist() == [a for a, _ in filed]
    assert np.array_equal(lm, np.array([b for _, b in filed], dtype=np.float32))
    assert t.poll() == 0          # no event pair was ever begun: nothing to read, no HIP call


def test_cost_table_argument_checks():
    m = _m()
    L = m.lib()
    boot = (ctypes.c_float * 4)(1.0, 2.0, 3.0, 4.0)
    bad = (ctypes.c_float * 4)(1.0, 0.0, 3.0, 4.0)
    h = ctypes.c_void_p()
    vp = ctypes.cast(boot, ctypes.c_void_p)
    assert L.dspark_cost_table_create(vp, 4, 32, 3, 32, None) == 1
    assert L.dspark_cost_table_create(None, 4, 32, 3, 32, ctypes.byref(h)) == 1
    assert L.dspark_cost_table_create(ctypes.cast(bad, ctypes.c_void_p), 4, 32, 3, 32, ctypes.byref(h)) == 1
    assert L.dspark_cost_table_create(vp, 4, 2, 3, 32, ctypes.byref(h)) == 1      # min_samples > window
    assert L.dspark_cost_table_create(vp, 4, 32, 3, 0, ctypes.byref(h)) == 1
    assert L.dspark_cost_table_create(vp, 4, 32, 3, 32, ctypes.byref(h)) == 0
    out = (ctypes.c_float * 4)()
    assert L.dspark_cost_table_read(h, ctypes.cast(out, ctypes.c_void_p), 5) == 1
    assert L.dspark_cost_table_read(h, ctypes.cast(out, ctypes.c_void_p), 4) == 0
    assert list(out) == [1.0, 2.0, 3.0, 4.0]
    assert L.dspark_cost_table_observe(h, 1, ctypes.c_float(-1.0)) == 1
    assert L.dspark_cost_table_end(h, None) == 1                                  # end without begin
    L.dspark_cost_table_destroy(h)
    assert L.dspark_status_string(5) == b"host allocation failed"


def test_schedule_batch_host_errors():
    m = _m()
    L = m.lib()
    assert L.dspark_schedule_batch(None, 4, 3, 256, 100, 256, None, None, None) == 1
    assert L.dspark_schedule_batch(256, 4, 0, 256, 100, 256, None, None, None) == 1
    assert L.dspark_schedule_batch(256, 4, 3, 256, 16, 256, None, None, None) == 1      # needs B(k+1)+1 = 17
    assert L.dspark_schedule_batch(256, 4097, 1, 256, 9000, 256, None, None, None) == 2  # B k > 4096
