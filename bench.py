"""Benchmark of the batched lossless token verification hot path on one MI355X.

A step is one pass of the whole path over one batch of the hierarchical
workload (B=256 sequences, k=8 drafted tokens, V=128256, bf16 logits of the
three exits L_d, L_i, L_f, windows of N_i=4): spec_verify_hier_rollback (row
statistics of every logit row, both verification stages, correction draws,
and the rollback of the batch's paged-KV block tables).  Inputs are synthetic
(seeded, see workloads/) and resident in HBM before the timed region.

Prints one JSON line: verified draft tokens/s (B*k per step), whole-step and
row-statistics-kernel HBM bandwidth against the 8 TB/s peak, and the CPU oracle
timed on a bounded sample of the same workload on this host's cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""

import argparse
import ctypes
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft tokens/s + achieved HBM GB/s (% peak), B=256 k=8 V=128256 bf16"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "rowstats_hier_B256_k8_V128256_bf16_traffic.json")
ROWSTATS_SRC = os.path.join(ROOT, "lossless_token_verification_amd", "csrc", "rowstats.hip")

# --- CPU baseline (the oracle, on a bounded sample of the same workload) ----

_CPU = {}


def _cpu_worker(seqs):
    from oracle import verify
    w = _CPU
    verify.spec_verify_hier(w["ld"], w["li"], w["lf"], w["tok"], w["temp"], 0, 0, 4,
                            sequences=seqs)
    return len(seqs)


def cpu_baseline(sample_seqs, procs):
    """Oracle wall time on ``sample_seqs`` sequences shaped like the workload,
    over ``procs`` forked worker processes (started before any GPU use)."""
    import numpy as np
    import workloads
    w = workloads.make_hier(sample_seqs, 8, 128256, seed=(3, 1000), ctx=(512, 4096))
    _CPU.update(ld=workloads.to_numpy_raw(w["ld_logits"]), li=workloads.to_numpy_raw(w["li_logits"]),
                lf=workloads.to_numpy_raw(w["lf_logits"]), tok=w["draft_tokens"].numpy(),
                temp=w["temperature"].numpy())
    del w
    chunks = [list(c) for c in np.array_split(np.arange(sample_seqs), procs * 2) if len(c)]
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        pool.map(_cpu_worker, [[0]] * procs)          # warm the workers
        t0 = time.perf_counter()
        done = sum(pool.map(_cpu_worker, chunks))
        dt = time.perf_counter() - t0
    _CPU.clear()
    return dict(value=done * 8 / dt, unit="verified draft tokens/s", cores=procs, kind="oracle",
                sample=f"{done} sequences of the B=256 k=8 V=128256 bf16 hierarchical workload "
                       f"(L_d, L_i, L_f logits, window 4), NumPy float64 oracle over {procs} "
                       f"processes, {dt:.2f} s wall",
                seconds=dt)


# --- GPU --------------------------------------------------------------------

class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b]) == 0
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def _traffic(launch_bytes):
    """HBM traffic per row-statistics launch from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(ROWSTATS_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if t.get("rowstats_source_sha256") != sha:
            return None
        return int(t["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--cpu-sample", type=int, default=256, help="sequences in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification path shards by sequence with no "
              "exchange, so a multi-GPU figure is N independent copies of this one; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        procs = max(1, min(16, os.cpu_count() or 1))
        cpu = cpu_baseline(args.cpu_sample, procs)
        print(f"[bench] cpu baseline: {cpu['value']:.1f} tokens/s on {procs} processes",
              file=sys.stderr, flush=True)

    import torch
    import lossless_token_verification_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make("hier", 0, device=dev)
    B, k, V = w["B"], w["k"], w["V"]
    table0, lens0 = w["block_table"].clone(), w["seq_lens"].clone()
    ws = sv.alloc_workspace(sv.workspace_bytes(B, k, V, torch.bfloat16, 3), dev)
    rows = B * (k + 2 * (k + 1))
    launch_bytes = rows * V * 2          # every logit row of L_d, L_i, L_f read once
    print(f"[bench] workload ready: {rows} rows, {launch_bytes} B per step", file=sys.stderr,
          flush=True)

    ev = HipEvents(2 * args.steps + 2)

    bufs = {}

    def step(i, events=None):
        # verification of both stages and the paged-KV rollback, one call
        return sv.spec_verify_hier_rollback(w["ld_logits"], w["li_logits"], w["lf_logits"],
                                            w["draft_tokens"], w["temperature"], table, lens,
                                            block_size=w["block_size"], max_freed=1,
                                            window=w["window"], seed=0, offset=i,
                                            workspace=ws, events=events,
                                            out=bufs.get("out"))

    table, lens = table0.clone(), lens0.clone()
    bufs["out"] = step(999999)
    for i in range(args.warmup):
        step(1000000 + i)
    torch.cuda.synchronize()
    table.copy_(table0)
    lens.copy_(lens0)
    torch.cuda.synchronize()
    hip = ev.hip
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    hip.hipEventRecord(ev.ev[-2], stream)
    t_host = time.perf_counter()
    for i in range(args.steps):
        step(i, events=(ev.ev[2 * i].value, ev.ev[2 * i + 1].value))
    t_host = time.perf_counter() - t_host
    hip.hipEventRecord(ev.ev[-1], stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(2 * args.steps, 2 * args.steps + 1)
    k1_ms = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)]
    ev.close()

    ms_step = total_ms / args.steps
    k1_avg = sum(k1_ms) / len(k1_ms)
    value = B * k / (ms_step / 1e3)
    step_gbps = launch_bytes / (ms_step / 1e3) / 1e9
    k1_gbps = launch_bytes / (k1_avg / 1e3) / 1e9
    traffic = _traffic(launch_bytes)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "hierarchical verify + KV rollback, B=256 k=8 V=128256 bf16 "
                               "logits of L_d/L_i/L_f, window N_i=4, 16-slot KV blocks",
                   "B": B, "k": k, "V": V, "logits": "bf16", "window": w["window"],
                   "block_size": w["block_size"]},
        "host_enqueue_us_per_step": round(t_host / args.steps * 1e6, 1),
        "hbm_gbps_step": round(step_gbps, 1),
        "hbm_frac_of_peak_step": round(step_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "rowstats_kernel<bf16>",
                     "achieved": round(k1_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k1_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": launch_bytes, "avg_launch_us": round(k1_avg * 1e3, 2)},
        "cpu_baseline": ({kk: v for kk, v in cpu.items() if kk != "seconds"} if cpu else None),
    }
    if cpu:
        line["cpu_baseline"]["value"] = round(cpu["value"], 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
