#!/usr/bin/env python3
"""Throughput of the DSpark verify sampler on one MI355X.

Workload: B=64 streams, k=5 drafts, V=129280, bf16 logits, Markov bias rank 256
(the headline shape).  One step verifies the batch the way a serving step
would use this library: the confidence head + adaptive count over the batch's
hidden states, then token-wise verification and block verification of the same
draft blocks (so a step verifies 2*B blocks).  Inputs are resident in HBM before
the timed region; several copies of the whole input set rotate so that no call
finds its inputs in the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` = verified draft blocks per second.
``roofline`` is for the dominant launch (row statistics, pass 1), timed with
HIP events recorded around it by the library's stage hook on the same stream,
and compared both with the published HBM peak and with a plain streaming read
measured on the same device (the package's stream-read kernel).
``cpu_baseline`` is the fp64 oracle on the host, on the same batch.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

METRIC = "verified draft blocks/s (B x k x V) and achieved HBM GB/s at B=64,k=5,V=129280"
HBM_PEAK_GBS = 8000.0
STAGE_NAMES = ["pack W1 tiles", "pass1 row statistics", "scan", "pass2 residual masses", "finalize/sampler"]

# HBM traffic of one pass-1 launch at this workload, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE; profiles/pass1_headline_b64_k5_v129280_hbm_bytes.md):
# FETCH_SIZE scaled by 2.0 (a 256 MiB device copy reads as 128 MiB), WRITE_SIZE by 1.0.
# Valid only for the kernel sources it was measured on (hash below); otherwise null.
PASS1_TRAFFIC = {"src_sha256_16": "4932efc03d18dfe3", "fetch_bytes": 114280.4 * 1024 * 2.0,
                 "write_bytes": 2937.1 * 1024 * 1.0}


def kernel_src_hash() -> str:
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in ("kernels.hip", "common.hpp"):
        with open(os.path.join(here, "draft_block_verification_row_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the call's stream)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.h.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def ms(self, a, b) -> float:
        if self.h.hipEventSynchronize(b) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        f = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(f.value)

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


def read_ceiling(torch, dev, nbytes=1 << 30, nbuf=3, reps=12):
    """Measured streaming-read rate of the device: the package's plain read kernel over
    nbuf rotating buffers of nbytes (together well beyond the Infinity Cache), at a few
    grid sizes; returns the best (GB/s, grid)."""
    here = os.path.dirname(os.path.abspath(__file__))
    L = ctypes.CDLL(os.path.join(here, "draft_block_verification_row_amd", "libdspark_stream_read.so"))
    L.dspark_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.dspark_stream_read.restype = ctypes.c_int
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    bufs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=gen) for _ in range(nbuf)]
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def launch(i, grid):
        if L.dspark_stream_read(bufs[i % nbuf].data_ptr(), nbytes, grid, sink.data_ptr(), stream) != 0:
            raise RuntimeError("dspark_stream_read failed")

    best = (0.0, 0)
    for grid in (2048, 4096, 8192, 16384):
        for i in range(nbuf):
            launch(i, grid)
        torch.cuda.synchronize()
        t0.record()
        for i in range(reps):
            launch(i, grid)
        t1.record()
        torch.cuda.synchronize()
        gbps = reps * nbytes / (t0.elapsed_time(t1) * 1e-3) / 1e9
        best = max(best, (gbps, grid))
    del bufs
    return best


def alg_bytes(B, k, V, R, e, s, gamma) -> float:
    """Algorithmic bytes of one verify call: every draft-slot row pair once, the bonus row
    only where it is sampled, W2 once and the gathered W1 rows, plus the small I/O."""
    rows = float(np.sum(2 * gamma + (s == gamma)))
    return e * V * rows + 2.0 * R * V + 2.0 * R * float(np.sum(gamma)) + 16.0 * B * k


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=3, help="rotating copies of the input set")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the verify path has no multi-GPU launcher (streams shard "
              "across GPUs with no collective). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import workloads
    import draft_block_verification_row_amd as dv

    dv.lib()  # fails loudly without the built HIP library
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating the headline workload (B=64, k=5, V=129280, bf16, Markov rank 256)")
    wl = workloads.make_zipf("h", 64, 64, 5, confidence=True)
    B, k, V, R = wl.B, wl.k, wl.V, wl.R

    def up(x):
        a = np.ascontiguousarray(x)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    base = dict(target=up(wl.target), draft=up(wl.draft), tokens=up(wl.draft_tokens.astype(np.int32)),
                temp=up(wl.temperature), anchor=up(wl.anchor.astype(np.int32)), W1=up(wl.W1), W2t=up(wl.W2t),
                hidden=up(wl.hidden), w=up(wl.conf_w))
    sets = [base] + [{kk: v.clone() for kk, v in base.items()} for _ in range(args.sets - 1)]
    ws_bytes = dv.workspace_bytes(B, k, V, dv.DSPARK_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = {m: (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, k + 1, dtype=torch.int32, device=dev),
                None) for m in ("tokenwise", "block")}
    verify = {"tokenwise": dv.verify_tokenwise, "block": dv.verify_block}
    ms_table = wl.verify_ms

    def call(method, s, step, ev=None):
        return verify[method](s["target"], s["draft"], s["tokens"], temperature=s["temp"], W1=s["W1"],
                              W2t=s["W2t"], anchor=s["anchor"], seed=wl.seed, step=step, workspace=ws,
                              out=outs[method], stage_events=ev)

    def one_step(i, evs=None):
        # consecutive verify calls never share an input set, so neither finds the
        # other's logits in the Infinity Cache
        s0, s1 = sets[(2 * i) % len(sets)], sets[(2 * i + 1) % len(sets)]
        dv.adaptive_k(s0["hidden"], s0["w"], wl.conf_b, ms_table, want_c=False)
        call("tokenwise", s0, i, None if evs is None else evs[0])
        call("block", s1, i, None if evs is None else evs[1])

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        one_step(args.warmup + i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # per-launch times: a separate pass with the library's stage events
    hip = HipEvents()
    nprof = min(args.steps, 50)
    stage_ms = {m: np.zeros(dv.STAGES) for m in ("tokenwise", "block")}
    realized = {}
    all_ev = []
    for i in range(nprof):
        evs = (hip.create(dv.STAGES + 1), hip.create(dv.STAGES + 1))
        all_ev.append(evs)
        one_step(i, evs)
    torch.cuda.synchronize()
    for evs in all_ev:
        for m, e in zip(("tokenwise", "block"), evs):
            stage_ms[m] += np.array([hip.ms(e[j], e[j + 1]) for j in range(dv.STAGES)])
        hip.destroy(evs[0] + evs[1])
    for m in stage_ms:
        stage_ms[m] /= nprof
    for m in ("tokenwise", "block"):
        call(m, sets[0], 0)
        torch.cuda.synchronize()
        realized[m] = outs[m][0].cpu().numpy()

    gamma = np.full(B, k)
    e = 2
    bytes_call = {m: alg_bytes(B, k, V, R, e, realized[m], gamma) for m in realized}
    # pass 1 reads target and draft rows 0..gamma-1 of every stream, W2 and the gathered
    # W1 rows: all of it algorithmic (a sampled bonus row is read by pass 2, only where
    # the verifier stops there)
    full_pass1 = e * V * float(np.sum(2 * gamma)) + 2.0 * R * V + 2.0 * R * float(np.sum(gamma))
    P1 = STAGE_NAMES.index("pass1 row statistics")
    t_pass1 = 0.5 * (stage_ms["tokenwise"][P1] + stage_ms["block"][P1])
    alg_pass1 = full_pass1
    achieved = alg_pass1 / (t_pass1 * 1e-3) / 1e9
    blocks_per_s = 2 * B / (ms_step * 1e-3)
    step_bytes = bytes_call["tokenwise"] + bytes_call["block"] + 2.0 * B * k * 4096
    result = {
        "metric": METRIC,
        "value": round(blocks_per_s, 1),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "headline: B=64 k=5 V=129280, bf16 logits (Zipf-biased Gaussian target, correlated "
                        "draft), Markov bias rank 256, T_b in [0.6, 1.0], seed 64",
            "step": "confidence head + adaptive n, token-wise verify, block verify (2*B blocks per step)",
            "B": B, "k": k, "V": V, "R": R, "input_sets_rotated": args.sets,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (round(PASS1_TRAFFIC["fetch_bytes"] + PASS1_TRAFFIC["write_bytes"])
                        if kernel_src_hash() == PASS1_TRAFFIC["src_sha256_16"] else None),
            "kernel": "pass1_kernel (row statistics + fused Markov MFMA)",
            "kernel_ms": round(t_pass1, 5),
            "alg_bytes_per_launch": int(alg_pass1),
            "bytes_read_by_design_per_launch": int(full_pass1),
            "frac_on_bytes_read": round(full_pass1 / (t_pass1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "stage_ms": {m: [round(x, 5) for x in stage_ms[m]] for m in stage_ms},
        "stages": STAGE_NAMES,
        "blocks_per_s_by_verifier": {m: round(B / (float(np.sum(stage_ms[m])) * 1e-3), 1) for m in stage_ms},
        "logits_per_s": round(2 * B * k * V / (ms_step * 1e-3), 1),
        "step_alg_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "accepted_mean": {m: round(float(np.mean(realized[m])), 4) for m in realized},
    }

    # the measured read ceiling of this device, beside the published peak
    log("timing a plain streaming read (3 x 1 GiB buffers)")
    ceil_gbps, ceil_grid = read_ceiling(torch, dev)
    result["roofline"]["measured_read_GBps"] = round(ceil_gbps, 1)
    result["roofline"]["frac_of_measured_read"] = round(achieved / ceil_gbps, 4)
    result["stream_read_ceiling"] = {
        "GBps": round(ceil_gbps, 1), "grid": ceil_grid, "bytes_per_launch": 1 << 30, "buffers": 3,
        "kernel": "dspark_stream_read: grid-stride 16-B loads, 256-thread groups, random bytes",
    }

    # the drafter's Markov walk at the same shape (the step before verification)
    log("timing the drafter walk (B=64, k=5 slots)")
    wtoks = torch.empty(B, k, dtype=torch.int32, device=dev)
    for i in range(5):
        s = sets[i % len(sets)]
        dv.draft_sample(s["draft"], temperature=s["temp"], W1=s["W1"], W2t=s["W2t"], anchor=s["anchor"],
                        seed=wl.seed, step=i, workspace=ws, out=wtoks)
    nwalk = 30
    torch.cuda.synchronize()
    t0.record()
    for i in range(nwalk):
        s = sets[i % len(sets)]
        dv.draft_sample(s["draft"], temperature=s["temp"], W1=s["W1"], W2t=s["W2t"], anchor=s["anchor"],
                        seed=wl.seed, step=1000 + i, workspace=ws, out=wtoks)
    t1.record()
    torch.cuda.synchronize()
    walk_ms = t0.elapsed_time(t1) / nwalk
    walk_alg = 2.0 * V * B * k + 2.0 * R * V + 2.0 * R * B * k   # draft rows once, W2 once, W1 rows
    walk_read = 2.0 * V * B * k + k * 2.0 * R * V + 2.0 * R * B * k   # W2 is read again for every slot
    result["draft_walk"] = {
        "ms_per_call": round(walk_ms, 5),
        "drafts_per_s": round(B * k / (walk_ms * 1e-3), 1),
        "alg_GBps": round(walk_alg / (walk_ms * 1e-3) / 1e9, 1),
        "bytes_read_by_design_GBps": round(walk_read / (walk_ms * 1e-3) / 1e9, 1),
        "launches": 2 * k,
    }

    # batch-level scheduler at the adaptive ragged shape (B=256 streams, k=5), and the
    # host cost of the online cost table's event pairs around each call
    log("timing the batch scheduler (B=256, k=5) and the online cost table")
    Bs, ks = 256, 5
    gsch = np.random.Generator(np.random.PCG64(5))
    c_s = torch.from_numpy(gsch.uniform(0.5, 0.95, size=(Bs, ks)).astype(np.float32)).to(dev)
    ms_s = torch.from_numpy((10.0 + 0.05 * np.arange(Bs * (ks + 1) + 1)).astype(np.float32)).to(dev)
    n_s = torch.empty(Bs, dtype=torch.int32, device=dev)
    for _ in range(10):
        dv.schedule_batch(c_s, ms_s, n_out=n_s)
    nsch = 200
    tot_s = torch.empty(1, dtype=torch.int32, device=dev)
    exp_s = torch.empty(1, dtype=torch.float64, device=dev)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(nsch):
        dv.schedule_batch(c_s, ms_s, n_out=n_s, total_out=tot_s, expected_out=exp_s)
    t1.record()
    torch.cuda.synchronize()
    sched_ms = t0.elapsed_time(t1) / nsch   # bounded by the Python call, not the kernel
    n_eager = n_s.clone()
    # the kernel alone: 20 launches captured in a HIP graph, replayed 10 times, every
    # replay's counts checked against the eager ones
    sched_graph_ms = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(20):
                    dv.schedule_batch(c_s, ms_s, n_out=n_s, total_out=tot_s, expected_out=exp_s)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        total_ms = 0.0
        for _ in range(10):
            n_s.fill_(-1)
            t0.record()
            graph.replay()
            t1.record()
            torch.cuda.synchronize()
            total_ms += t0.elapsed_time(t1)
            if not torch.equal(n_s, n_eager):
                raise RuntimeError("graph replay of the scheduler disagrees with the eager call")
        sched_graph_ms = total_ms / 200
        del graph
    except RuntimeError as e:
        log(f"scheduler graph timing skipped: {e}")
    table = dv.CostTable((10.0 + 0.05 * np.arange(Bs * (ks + 1) + 1)).astype(np.float32))
    host_s = 0.0
    for _ in range(nsch):
        h0 = time.perf_counter()
        table.begin(Bs + ks)
        host_s += time.perf_counter() - h0
        dv.schedule_batch(c_s, ms_s, n_out=n_s, total_out=tot_s, expected_out=exp_s)
        h0 = time.perf_counter()
        table.end()
        table.poll()
        host_s += time.perf_counter() - h0
    torch.cuda.synchronize()
    table.poll()
    result["batch_schedule"] = {
        "B": Bs, "k": ks,
        "us_per_call_python": round(sched_ms * 1e3, 2),
        "us_per_launch_graph": None if sched_graph_ms is None else round(sched_graph_ms * 1e3, 2),
        "drafts_chosen": int(n_s.sum().item()),
        "cost_table_host_us_per_step": round(host_s / nsch * 1e6, 2),
        "cost_table_filed": table.stats()["filed"],
    }
    del table

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_reference_bytes"] = 2 * (args.copy_mib << 20)
        del src, dst

    if not args.no_cpu_baseline:
        from oracle import dspark as odsp   # cpu_baseline leg only
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            blas_threads = 1
        log("timing the fp64 oracle on the host (the same batch, both verifiers + adaptive head; ~10 s)")
        # whole steps (successive Philox steps) until about 10 s of host work, at most 20
        c0 = time.perf_counter()
        nsteps = 0
        while nsteps < 20 and (nsteps == 0 or time.perf_counter() - c0 < 10.0):
            odsp.adaptive_k(wl.hidden, wl.conf_w, wl.conf_b, wl.verify_ms)
            for m in ("tokenwise", "block"):
                odsp.verify(wl.target, wl.draft, wl.dtype, wl.draft_tokens, wl.temperature, wl.anchor, wl.W1,
                            wl.W2t, seed=wl.seed, step=nsteps, method=m)
            nsteps += 1
        cpu_s = time.perf_counter() - c0
        result["cpu_baseline"] = {
            "value": round(2 * B * nsteps / cpu_s, 3),
            "unit": "blocks/s",
            "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{nsteps} full steps of the same batch (adaptive head + token-wise + block verify of {B} "
                      f"streams, steps 0..{nsteps - 1}) in fp64 numpy, {cpu_s:.1f} s; elementwise work "
                      f"single-threaded, BLAS products on {blas_threads} threads",
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
