"""HIP path vs the fp64 oracle, through the C ABI, on seeded workloads.

Sizes span several 256-id groups with ragged tails, every logit dtype, Markov
ranks, ragged draft counts, and the full 129280-id vocabulary at the shapes the
benchmark times.  Probabilities within tolerance; accepted lengths and tokens
bit-exact except where the oracle's decision margin is below 1e-6.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dspark as odsp
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mod():
    import draft_block_verification_row_amd as m
    m.lib()
    return m


def _run(mod, wl, method, steps, label):
    dev = H.to_dev(wl)
    t = H.Tally()
    for step in steps:
        g = H.run_gpu(mod, dev, method, wl.seed, step)
        o = H.run_oracle(wl, method, step)
        H.compare(g, o, wl, method, t, label=f"{label}/step{step}")
    print(f"[{label} {method}] {t.summary()}", flush=True)
    H.assert_clean(t)
    return t


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_tiny_exhaustive_shape(mod, method):
    wl = workloads.make("c1")
    _run(mod, wl, method, range(200), "c1")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_tiny_ragged(mod, method):
    wl = workloads.make("c1")
    wl.num_drafts = np.array([0, 1, 2, 3], dtype=np.int32)
    _run(mod, wl, method, range(50), "c1-ragged")


SMALL = [
    # (V, dtype, R, B, k, markov)
    (1000, "bf16", 256, 3, 4, True),
    (333, "bf16", 64, 3, 4, True),
    (4099, "f32", 128, 2, 5, True),
    (2048, "bf16", 32, 5, 3, True),
    (777, "f32", 256, 2, 6, False),
]


@pytest.mark.parametrize("V,dtype,R,B,k,markov", SMALL)
@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_small_shapes(mod, method, V, dtype, R, B, k, markov):
    wl = workloads.make_zipf(f"small{V}", seed=V + R, B=B, k=k, V=V, dtype=dtype, R=R, markov=markov,
                             sigma=1.5, rho=(0.6, 0.99))
    _run(mod, wl, method, range(20), f"V{V}-{dtype}-R{R}")


LARGE_V = [
    # (V, dtype, R, B, k): more than 512 groups (V > 131072), one pass of the scan per
    # 512 groups; k > 5 also splits the rows into passes of 6; odd V takes the
    # unaligned (non-vector) loads.  Small ranks keep the fp64 oracle fast.
    (140001, "bf16", 32, 2, 7),
    (200000, "bf16", 64, 3, 5),
    (150000, "f32", 32, 2, 3),
]


@pytest.mark.parametrize("V,dtype,R,B,k", LARGE_V)
@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_vocab_past_512_groups(mod, method, V, dtype, R, B, k):
    wl = workloads.make_zipf(f"largeV{V}", seed=V % 1000 + k, B=B, k=k, V=V, dtype=dtype, R=R, sigma=1.5,
                             rho=(0.6, 0.99), greedy_every=3 if B > 2 else 0)
    _run(mod, wl, method, range(3), f"V{V}-{dtype}-k{k}")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_single_stream_fp32_full_vocab(mod, method):
    wl = workloads.make("c2")
    _run(mod, wl, method, range(3), "c2")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_small_batch_bf16(mod, method):
    wl = workloads.make("c3")
    _run(mod, wl, method, range(2), "c3")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_headline_shape(mod, method):
    """B=64, k=5, V=129280 bf16 with the Markov bias: the shape the benchmark times."""
    wl = workloads.make("h")
    _run(mod, wl, method, [0], "h")


def test_overlong_drafts_block(mod):
    wl = workloads.make("c4")
    _run(mod, wl, "block", [0], "c4")


def test_adaptive_then_ragged_block(mod):
    wl = workloads.make("c5", B=64)
    dev = H.to_dev(wl)
    hid = torch.from_numpy(wl.hidden.view(np.int16)).cuda()
    w = torch.from_numpy(wl.conf_w.view(np.int16)).cuda()
    n, c, a = mod.adaptive_k(hid, w, wl.conf_b, wl.verify_ms)
    torch.cuda.synchronize()
    ref = odsp.adaptive_k(wl.hidden, wl.conf_w, wl.conf_b, wl.verify_ms)
    assert np.allclose(c.cpu().numpy(), ref["c"], rtol=1e-5, atol=0)
    assert np.allclose(a.cpu().numpy(), ref["a"], rtol=1e-5, atol=0)
    n_g = n.cpu().numpy()
    near = ref["margin"] < H.NEAR
    assert np.array_equal(n_g[~near], ref["n"][~near])
    # ragged block verification over the chosen counts, without a host round trip
    dev["num_drafts"] = n
    g = H.run_gpu(mod, dev, "block", wl.seed, 0)
    wl.num_drafts = n_g
    o = H.run_oracle(wl, "block", 0)
    t = H.Tally()
    H.compare(g, o, wl, "block", t, label="c5-ragged")
    print(f"[c5 adaptive] n histogram {np.bincount(n_g, minlength=6).tolist()} {t.summary()}", flush=True)
    H.assert_clean(t)


@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (333, "bf16"), (129280, "bf16")])
def test_markov_bias_standalone(mod, V, dtype):
    wl = workloads.make_zipf("mb", seed=11, B=3, k=3, V=V, dtype=dtype, sigma=3.0)
    prev = np.array([5, -1, V - 1, 17, 0, V + 5, 3], dtype=np.int32)
    rows = len(prev)
    rng = np.random.Generator(np.random.PCG64(3))
    logits = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    if dtype == "bf16":
        logits_dev = torch.from_numpy(workloads.f32_to_bf16_bits(logits).view(np.int16)).cuda()
        logits_f = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(logits)).astype(np.float64)
    else:
        logits_dev = torch.from_numpy(logits).cuda()
        logits_f = logits.astype(np.float64)
    W1 = torch.from_numpy(wl.W1.view(np.int16)).cuda()
    W2t = torch.from_numpy(wl.W2t.view(np.int16)).cuda()
    pv = torch.from_numpy(prev).cuda()
    out = mod.markov_bias(W1, W2t, pv, logits_dev)
    bias_only = mod.markov_bias(W1, W2t, pv)
    torch.cuda.synchronize()
    ref = odsp.markov_bias(wl.W1, wl.W2t, np.where((prev >= 0) & (prev < V), prev, -1))
    assert np.max(np.abs(bias_only.cpu().numpy() - ref)) < 1e-6
    assert np.max(np.abs(out.cpu().numpy() - (ref + logits_f))) < 1e-6


def test_run_to_run_bit_identical(mod):
    wl = workloads.make("c3")
    dev = H.to_dev(wl)
    for method in ("tokenwise", "block"):
        a = H.run_gpu(mod, dev, method, 5, 9)
        b = H.run_gpu(mod, dev, method, 5, 9)
        assert np.array_equal(a["accepted_len"], b["accepted_len"])
        assert np.array_equal(a["out_tokens"], b["out_tokens"])
        assert np.array_equal(np.nan_to_num(a["diag"], nan=7.0), np.nan_to_num(b["diag"], nan=7.0))


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_maximum_draft_count(mod, method):
    """k = 32 (the largest block the library takes): six passes of row statistics in
    the scan, a 32-bit candidate mask; ragged counts from 0 to 32 and a greedy stream."""
    wl = workloads.make_zipf("maxk", seed=32, B=4, k=32, V=700, dtype="bf16", R=64, sigma=1.5,
                             rho=(0.8, 0.995), greedy_every=4)
    wl.num_drafts = np.array([32, 0, 17, 31], dtype=np.int32)
    _run(mod, wl, method, range(4), "k32")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_batch_wider_than_a_workgroup(mod, method):
    """B = 600 streams (more than the 256 threads that fill the per-workgroup stream
    table in one step), mixed greedy and sampled, ragged counts."""
    wl = workloads.make_zipf("wideB", seed=600, B=600, k=2, V=300, dtype="bf16", R=32, sigma=1.5,
                             rho=(0.6, 0.99), greedy_every=5)
    wl.num_drafts = (np.arange(600) % 3).astype(np.int32)
    _run(mod, wl, method, range(2), "B600")
