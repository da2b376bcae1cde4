"""Benchmark of the batched lossless token verification hot path on one MI355X.

A step is one pass of the whole path over one batch of the hierarchical
workload (B=256 sequences, k=8 drafted tokens, V=128256, bf16 logits of the
three exits L_d, L_i, L_f, windows of N_i=4): spec_verify_hier_rollback (row
statistics of every logit row, both verification stages, correction draws,
and the rollback of the batch's paged-KV block tables).  Inputs are synthetic
(seeded, see workloads/), drawn on the host and resident in HBM before the
timed region.

Before the counted warm-up steps the step runs back to back for --settle-ms
(400 ms by default): in the first tens of milliseconds of sustained load the
chip's power management holds the shader clock at 1.2-1.9 GHz before it
settles at 2.2-2.3 GHz, and a serving loop that verifies continuously runs in
the settled state.  The timed steps are full steps; the line reports each
step's time distribution beside the total.

Prints one JSON line: verified draft tokens/s (B*k per step), whole-step and
row-statistics-kernel HBM bandwidth against the 8 TB/s peak, the oracle timed
on the first timed step's inputs on this host's cores, and the parity of that
step's outputs with the oracle's.  After the timed steps, the other workloads
(the single-stage ones, call by call with their parity, and the fused LM-head
verify) are measured into the line's "other_workloads" (--no-other-workloads
skips them).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--settle-ms 400]
"""

import argparse
import csv
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
ROWSTATS_SRC = [os.path.join(ROOT, "lossless_token_verification_amd", "csrc", f)
                for f in ("rowstats.hip", "sv_stats.h", "sv_common.h")]


def _rowstats_sha():
    """Digest of the sources the row-statistics kernel is compiled from."""
    h = hashlib.sha256()
    for fn in ROWSTATS_SRC:
        with open(fn, "rb") as f:
            h.update(f.read())
    return h.hexdigest()

# --- the oracle leg: CPU baseline and parity of the timed outputs -----------
#
# The headline inputs are drawn on the host; worker processes are forked from
# that state before any GPU call, so that they read the very logits, drafts and
# temperatures the GPU consumes.  After the timed steps the oracle verifies the
# first timed step's inputs (Philox offset 0): its wall time is the CPU
# baseline, its outputs the reference the GPU's outputs are compared with.

_CPU = {}
HOST_SHARE = 16   # host CPU cores per GPU on the measured machine (the pool's size)


def _cpu_worker(job):
    """Oracle of the hierarchical verify on a list of sequences; returns the
    per-sequence outputs and infos (near-tie events need them)."""
    from oracle import verify
    seqs, offset, flips = job
    w = _CPU
    r = verify.spec_verify_hier(w["ld"], w["li"], w["lf"], w["tok"], w["temp"], 0, offset, 4,
                                sequences=seqs, flips=flips)
    keys = ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop")
    return {b: ({k: r[k][b] for k in keys}, r["infos"][b]) for b in seqs}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_pool(host, procs):
    """Fork ``procs`` oracle workers over the host inputs (before any GPU use)."""
    _CPU.update(ld=workloads_raw(host["ld_logits"]), li=workloads_raw(host["li_logits"]),
                lf=workloads_raw(host["lf_logits"]), tok=host["draft_tokens"].numpy(),
                temp=host["temperature"].numpy())
    return mp.get_context("fork").Pool(procs)


def workloads_raw(t):
    import workloads
    return workloads.to_numpy_raw(t)


def oracle_leg(pool, procs, B, k, offset, p1_seqs):
    """The oracle on the first timed step's inputs: every sequence over the
    pool (one untimed pass whose outputs are kept, then two timed passes), and
    the first ``p1_seqs`` sequences in this process alone (P = 1).  Returns
    (results {b: (outputs, info)}, cpu_baseline dict)."""
    import numpy as np
    chunks = [c.tolist() for c in np.array_split(np.arange(B), procs * 4) if len(c)]
    res = {}
    for part in pool.map(_cpu_worker, [(c, offset, None) for c in chunks]):
        res.update(part)
    times = []
    for _ in range(2):
        t0 = time.perf_counter()
        pool.map(_cpu_worker, [(c, offset, None) for c in chunks])
        times.append(time.perf_counter() - t0)
    t_pool = min(times)
    t0 = time.perf_counter()
    _cpu_worker((list(range(p1_seqs)), offset, None))
    t_one = time.perf_counter() - t0
    base = dict(value=round(B * k / t_pool, 2), unit="verified draft tokens/s", cores=procs,
                kind="oracle",
                sample=f"the first timed step's inputs (B={B} k={k} V=128256 bf16 L_d/L_i/L_f, "
                       f"window 4, Philox offset {offset}): all {B} sequences over {procs} "
                       f"forked processes, best of 2 passes ({t_pool:.2f} s); one process "
                       f"over the first {p1_seqs} sequences ({t_one:.2f} s); NumPy float64",
                p1_value=round(p1_seqs * k / t_one, 2), p1_sequences=p1_seqs,
                cpu_model=_cpu_model(), os_cpu_count=os.cpu_count())
    return res, base


def parity_of_step(pool, res, gpu, offset, kv):
    """Compares one step's GPU outputs with the oracle's: bit for bit where the
    outcome is unique; at a near tie the GPU must give the oracle's outcome or
    the one with that decision flipped (re-run by the oracle).  The rolled-back
    block tables and lengths are compared with the oracle's rollback of the
    GPU's own num_drop (bit for bit, every sequence)."""
    import numpy as np
    from oracle import blocktable, verify
    keys = ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop")
    g = {k: gpu[k].cpu().numpy() for k in keys}
    exact = as_oracle = as_flip = unresolved = 0
    mismatched = []
    flips = {}
    for b, (ref, info) in sorted(res.items()):
        same = all(np.array_equal(g[k][b], ref[k]) for k in keys)
        ev = verify.near_tie_event(info, 1e-5, 1e-6)
        if ev is None:
            exact += 1
            if not same:
                mismatched.append(b)
        elif same:
            as_oracle += 1
        elif ev["flip"] is None:
            unresolved += 1
        else:
            flips[b] = ev
    if flips:
        alt = {}
        for part in pool.map(_cpu_worker, [([b], offset, {b: e}) for b, e in flips.items()]):
            alt.update(part)
        for b in flips:
            if all(np.array_equal(g[k][b], alt[b][0][k]) for k in keys):
                as_flip += 1
            else:
                mismatched.append(b)
    table0, lens0, table, lens, freed, nfreed = kv
    t2, l2, f2, n2 = blocktable.kv_blocktable_truncate(table0, lens0, g["num_drop"], 16, 1)
    kv_ok = bool(np.array_equal(table, t2) and np.array_equal(lens, l2) and
                 np.array_equal(freed, f2) and np.array_equal(nfreed, n2))
    return dict(step=0, sequences=len(res), exact=exact, near_tie_as_oracle=as_oracle,
                near_tie_as_flipped=as_flip, near_tie_unresolved=unresolved,
                mismatched=sorted(mismatched)[:16], n_mismatched=len(mismatched),
                kv_state_equal=kv_ok)


# --- HBM traffic from rocprofv3 counters -------------------------------------

COPY_ELEMS = 1 << 28            # fp32 elements of the calibration copy (1 GiB each way)


def calibration_copy(dev):
    """A plain copy of known size (reads and writes COPY_ELEMS * 4 bytes),
    launched next to the profiled steps so that FETCH_SIZE / WRITE_SIZE can
    be converted into bytes."""
    import torch
    x = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        torch.mul(x, 2.0, out=y)
    torch.cuda.synchronize()
    del x, y


def _counter_rows(d):
    """(dispatch id, kernel name, counter name, value) of every dispatch in the
    counter_collection.csv files under directory ``d``."""
    out = []
    for root, _, files in os.walk(d):
        for fn in files:
            if not fn.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(root, fn), newline="") as f:
                for r in csv.DictReader(f):
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                                float(r["Counter_Value"])))
    return out


def _per_dispatch(rows, counter, ids):
    vals = [v for i, _, c, v in rows if c == counter and i in ids]
    if not vals:
        raise SystemExit(f"no {counter} samples for the requested kernel")
    return sum(vals) / len(vals), len(vals)


def _ids(rows):
    """Dispatch ids of the row-statistics kernel, and of the calibration copy
    (the last three kernel dispatches of the process; the runtime's own
    buffer-copy kernels that read results back to the host come after it)."""
    names = {i: n for i, n, _, _ in rows}
    stats = {i for i, n in names.items() if "rowstats_kernel<1, false>" in n}
    last = sorted(i for i, n in names.items() if not n.startswith("__amd_rocclr_"))[-3:]
    if len({names[i] for i in last}) != 1 or any(i in stats for i in last):
        raise SystemExit("the last three dispatches are not the calibration copy")
    return stats, set(last)


def traffic_from(fetch_dir, write_dir):
    """Write the traffic summary of the row-statistics kernel from two
    counter runs (FETCH_SIZE, then WRITE_SIZE), each scaled by the reading of
    the same counter for the calibration copy."""
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    (fs, fc), (ws, wc) = _ids(fr), _ids(wr)
    f_k, nf = _per_dispatch(fr, "FETCH_SIZE", fs)
    w_k, nw = _per_dispatch(wr, "WRITE_SIZE", ws)
    f_c, _ = _per_dispatch(fr, "FETCH_SIZE", fc)
    w_c, _ = _per_dispatch(wr, "WRITE_SIZE", wc)
    copy_bytes = COPY_ELEMS * 4
    kf, kw = copy_bytes / (f_c * 1024.0), copy_bytes / (w_c * 1024.0)
    fetch_b, write_b = f_k * 1024.0 * kf, w_k * 1024.0 * kw
    sha = _rowstats_sha()
    out = {
        "kernel": "rowstats_kernel<bf16>",
        "workload": "hierarchical verify, B=256 k=8 V=128256 bf16",
        "fetch_kib_per_dispatch": round(f_k, 1), "write_kib_per_dispatch": round(w_k, 1),
        "dispatches": [nf, nw],
        "copy_fetch_kib": round(f_c, 1), "copy_write_kib": round(w_c, 1),
        "copy_bytes_each_way": copy_bytes,
        "fetch_scale": round(kf, 5), "write_scale": round(kw, 5),
        "hbm_fetch_bytes_per_launch": int(fetch_b), "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
        "rowstats_source_sha256": sha,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


# --- GPU --------------------------------------------------------------------

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


class HipEvents:
    """Raw hipEvent_t handles for timing only (the library has them take its
    kernels' start and end times).  They carry no system-scope fence: nothing
    waits on them for data."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(
                ctypes.byref(e), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) == 0
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
        if t.get("rowstats_source_sha256") != _rowstats_sha():
            return None
        return int(t["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _dist_us(ms):
    """Distribution of per-step times (ms in, us out): the first and last five
    steps in order, then median, p10 and p90 over all steps."""
    us = [round(x * 1e3, 1) for x in ms]
    srt = sorted(us)
    n = len(srt)
    return dict(first5=us[:5], last5=us[-5:], median=srt[n // 2], p10=srt[n // 10],
                p90=srt[min(n - 1, (9 * n) // 10)])


def _draw_and_sequential_bytes(out, w, B, k, V):
    """Bytes beside the headline, from one step's outputs (bf16 rows of V):
    the rows the draws re-read after the stream -- L_i, L_d (none for the
    bonus) and L_f at a1 when stage 2 reaches y, L_f and L_i at a2 when it
    rejects a draft before a1, none for a greedy sequence -- and the rows a
    sequential verification would have to read: L_d and L_i up to a1, L_f up
    to stage 2's stop."""
    import numpy as np
    a1 = out["accept_len_inter"].cpu().numpy().astype(np.int64)
    a2 = out["accept_len_final"].cpu().numpy().astype(np.int64)
    t = w["temperature"]
    sampled = (t.cpu().numpy() > 0) if t is not None else np.ones(B, dtype=bool)
    early = a2 < a1
    draw_rows = np.where(early, 2, np.where(a1 < k, 3, 2)) * sampled
    seq_rows = np.minimum(a1 + 1, k) + (a1 + 1) + (np.minimum(a1, a2) + 1)
    row_bytes = V * 2
    return int(draw_rows.sum()) * row_bytes, int(seq_rows.sum()) * row_bytes


MFMA_BF16_PEAK_TFLOPS = 2500.0


def measure_lmhead(steps, warmup, dev, settle_ms=0.0):
    """The fused LM-head verify (B=128, k=4, d=4096, V=128256, bf16 hidden
    states and head): ``steps`` spec_verify_lmhead_single calls back to back,
    each with the statistics GEMM bracketed by its own HIP events.  Returns
    the per-call time and the statistics GEMM's rate against the bf16 dense
    MFMA peak (2 * rows * V * d flops per launch, rows = B * (2k + 1))."""
    import torch
    import lossless_token_verification_amd as sv
    import workloads

    w = workloads.make("lmhead", 0, device=dev)
    B, k, V, d = w["B"], w["k"], w["V"], w["d"]
    ws = sv.alloc_workspace(sv.lmhead_workspace_bytes(B, k, V, d), dev)
    rows = B * (2 * k + 1)
    flops = 2.0 * rows * V * d
    print(f"[bench] LM-head workload ready: {rows} rows, {flops / 1e12:.3f} TFLOP per GEMM",
          file=sys.stderr, flush=True)
    ev = HipEvents(2 * steps + 2)
    bufs = {}

    def step(i, events=None):
        return sv.spec_verify_lmhead_single(w["h_draft"], w["h_target"], w["w_vocab"],
                                            w["draft_tokens"], w["temperature"], seed=0,
                                            offset=i, workspace=ws, events=events,
                                            out=bufs.get("out"))

    bufs["out"] = step(999999)
    settle_steps = _settle(step, settle_ms, torch.cuda.synchronize) if settle_ms > 0 else 0
    for i in range(warmup):
        step(1000000 + i)
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev.hip.hipEventRecord(ev.ev[-2], stream)
    for i in range(steps):
        step(i, events=(ev.ev[2 * i].value, ev.ev[2 * i + 1].value))
    ev.hip.hipEventRecord(ev.ev[-1], stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(2 * steps, 2 * steps + 1)
    g_ms = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)]
    ev.close()
    g_avg = sum(g_ms) / len(g_ms)
    tflops = flops / (g_avg / 1e3) / 1e12
    return dict(B=B, k=k, V=V, d=d, ms_per_call=round(total_ms / steps, 5),
                settle_ms=settle_ms, settle_steps=settle_steps,
                roofline={"bound": "mfma", "kernel": "lmhead_gemm<stats>",
                          "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                          "traffic": None, "flops_per_launch": flops,
                          "avg_launch_us": round(g_avg * 1e3, 2)})


def bench_lmhead(args):
    """The fused LM-head verify as the step (see measure_lmhead)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = measure_lmhead(args.steps, args.warmup, dev, args.settle_ms)
    B, k, V, d, ms_step = m["B"], m["k"], m["V"], m["d"], m["ms_per_call"]
    line = {
        "metric": "verified draft tokens/s, fused LM-head verify B=128 k=4 d=4096 V=128256 bf16",
        "value": round(B * k / (ms_step / 1e3), 1),
        "unit": "verified draft tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "fused LM-head single-stage verify, B=128 k=4 d=4096 "
                               "V=128256, bf16 hidden states and head", "B": B, "k": k,
                   "d": d, "V": V},
        "roofline": m["roofline"],
        "cpu_baseline": None,
        "settle_ms": m["settle_ms"], "settle_steps": m["settle_steps"],
    }
    print(json.dumps(line), flush=True)


SINGLE_KEYS = ("accept_len", "out_tokens", "num_emitted", "num_drop")


def _single_parity(w, gpu, offset):
    """One single-stage call's GPU outputs against the oracle's on the same
    inputs, as parity_of_step does for the headline: bit for bit where the
    outcome is unique, the oracle's outcome or the one with that near-tie
    decision flipped otherwise."""
    import numpy as np
    import workloads
    from oracle import verify
    d = workloads.to_numpy_raw(w["draft_logits"])
    t = workloads.to_numpy_raw(w["target_logits"])
    tok = w["draft_tokens"].cpu().numpy()
    temp = w["temperature"].cpu().numpy() if w.get("temperature") is not None else None
    ref = verify.spec_verify_single(d, t, tok, temp, 0, offset)
    g = {k: gpu[k].cpu().numpy() for k in SINGLE_KEYS}
    exact = as_oracle = as_flip = unresolved = 0
    mismatched = []
    for b in range(w["B"]):
        same = all(np.array_equal(g[k][b], ref[k][b]) for k in SINGLE_KEYS)
        ev = verify.near_tie_event(ref["infos"][b], 1e-5, 1e-6)
        if ev is None:
            exact += 1
            if not same:
                mismatched.append(b)
        elif same:
            as_oracle += 1
        elif ev["flip"] is None:
            unresolved += 1
        else:
            alt = verify.spec_verify_single(d, t, tok, temp, 0, offset, sequences=[b],
                                            flips={b: ev})
            if all(np.array_equal(g[k][b], alt[k][b]) for k in SINGLE_KEYS):
                as_flip += 1
            else:
                mismatched.append(b)
    return dict(sequences=w["B"], exact=exact, near_tie_as_oracle=as_oracle,
                near_tie_as_flipped=as_flip, near_tie_unresolved=unresolved,
                mismatched=mismatched[:16], n_mismatched=len(mismatched))


def measure_single(name, steps, warmup, dev, parity=False):
    """The single-stage verify on one of the single-stage workloads.  Each call
    is bracketed by its own HIP events; between calls a 1 GiB buffer is
    written (outside the events), so that the logits are not served from the
    256 MB memory-side cache ("cold"); a second pass without it gives the
    warm figure.  Algorithmic bytes: every draft and target row read once.
    With ``parity`` the first timed call's outputs are compared with the
    oracle's."""
    import torch
    import lossless_token_verification_amd as sv
    import workloads

    w = workloads.make(name, 0, device=dev)
    B, k, V = w["B"], w["k"], w["V"]
    es = 2 if w["dtype"] == "bf16" else 4
    algo = B * (2 * k + 1) * V * es
    ws = sv.alloc_workspace(sv.workspace_bytes(B, k, V, w["draft_logits"].dtype, 2), dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev = HipEvents(2 * steps)
    first = {}

    def call(i):
        return sv.spec_verify_single(w["draft_logits"], w["target_logits"], w["draft_tokens"],
                                     w.get("temperature"), seed=0, offset=i, workspace=ws)

    for i in range(warmup):
        call(1000000 + i)
    torch.cuda.synchronize()
    res = {}
    for mode in ("cold", "warm"):
        for i in range(steps):
            if mode == "cold":
                flush.fill_(float(i))
            ev.hip.hipEventRecord(ev.ev[2 * i], stream)
            out = call(i)
            ev.hip.hipEventRecord(ev.ev[2 * i + 1], stream)
            if mode == "cold" and i == 0:
                first = out
        torch.cuda.synchronize()
        ts = sorted(ev.elapsed_ms(2 * i, 2 * i + 1) * 1e3 for i in range(steps))
        res[mode] = dict(median_us=round(ts[len(ts) // 2], 2), p10_us=round(ts[len(ts) // 10], 2),
                         p90_us=round(ts[(9 * len(ts)) // 10], 2))
    ev.close()
    del flush
    us = res["cold"]["median_us"]
    gbps = algo / (us * 1e-6) / 1e9
    m = dict(workload=name, B=B, k=k, V=V, logits=w["dtype"],
             value=round(B * k / (us * 1e-6), 1), unit="verified draft tokens/s",
             per_call=res,
             roofline_call={"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                            "bytes_per_call": algo,
                            "t_roof_us": round(algo / (HBM_PEAK_GBPS * 1e9) * 1e6, 2)})
    if parity:
        m["parity"] = _single_parity(w, first, 0)
    return m


def bench_single(args):
    """The single-stage verify on --workload as the step (see measure_single)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = measure_single(args.workload, args.steps, args.warmup, dev)
    us = m["per_call"]["cold"]["median_us"]
    line = {
        "metric": f"verified draft tokens/s, single-stage verify, {args.workload} workload",
        "value": m["value"], "unit": "verified draft tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "B": m["B"], "k": m["k"], "V": m["V"],
                   "logits": m["logits"]},
        "per_call": m["per_call"],
        "roofline_call": m["roofline_call"],
    }
    print(json.dumps(line), flush=True)


def other_workloads(dev, parity):
    """The workloads beside the headline, measured after its timed steps (not
    part of the step): the three single-stage workloads (20 cold and 20 warm
    calls each; with ``parity``, part of the oracle leg, the first cold call's
    outputs compared with the oracle) and the fused LM-head verify (10
    calls after 200 ms of back-to-back calls: the oracle leg leaves the GPU
    idle long enough for its clocks to drop)."""
    res = {}
    for name in ("tiny", "batched", "mixed_temp"):
        print(f"[bench] other workload: {name}", file=sys.stderr, flush=True)
        res[name] = measure_single(name, 20, 5, dev, parity=parity)
    print("[bench] other workload: lmhead", file=sys.stderr, flush=True)
    res["lmhead"] = measure_lmhead(10, 3, dev, settle_ms=200.0)
    return res


def bench_tentative(args):
    """The hierarchy across calls on the hierarchical workload: per step one
    intermediate round (stage 1 on L_d, L_i; the output and its L_i rows
    appended to the pending state) and one flush of every sequence's pending
    tokens against the final exit (min_pending 1), i.e. the one-call
    hierarchy split at the call boundary."""
    import torch
    import lossless_token_verification_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make("hier", 0, device=dev)
    B, k, V = w["B"], w["k"], w["V"]
    cap = k + 1
    lf = torch.zeros((B, cap + 1, V), dtype=torch.bfloat16, device=dev)
    lf[:, :k + 1] = w["lf_logits"]
    # fresh logits every step, as in the headline bench (see --rotate)
    copies = [(w["ld_logits"], w["li_logits"], lf)]
    for _ in range(max(1, args.rotate) - 1):
        copies.append(tuple(t.clone() for t in copies[0]))
    pend = sv.make_pending(B, cap, V, torch.bfloat16, dev)
    ws = sv.alloc_workspace(sv.tentative_workspace_bytes(B, k, V, torch.bfloat16, cap), dev)
    print("[bench] tentative workload ready", file=sys.stderr, flush=True)

    def step(i):
        ld, li, lf_i = copies[i % len(copies)]
        sv.spec_verify_tentative_round(ld, li, w["draft_tokens"],
                                       w["temperature"], pend, seed=0, offset=2 * i,
                                       workspace=ws)
        return sv.spec_verify_tentative_flush(lf_i, w["temperature"], pend, min_pending=1,
                                              seed=0, offset=2 * i, workspace=ws)

    settle_steps = _settle(step, args.settle_ms, torch.cuda.synchronize) if args.settle_ms > 0 else 0
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = HipEvents(2)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev.hip.hipEventRecord(ev.ev[0], stream)
    for i in range(args.steps):
        out = step(1000 + i)
    ev.hip.hipEventRecord(ev.ev[1], stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / args.steps
    ev.close()
    n = out["num_emitted"].cpu()
    rows_read = B * k + B * (k + 1) + 2 * int(n.clamp(min=1).sum())
    line = {
        "metric": "verified draft tokens/s, hierarchy across calls (round + flush), "
                  "B=256 k=8 V=128256 bf16",
        "value": round(B * k / (ms / 1e3), 1), "unit": "verified draft tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "hierarchical workload; one intermediate round, then a flush "
                               "of the pending tokens against the final exit",
                   "B": B, "k": k, "V": V, "capacity": cap, "input_copies": len(copies)},
        "approx_rows_read_per_step": rows_read,
        "settle_ms": args.settle_ms, "settle_steps": settle_steps,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-p1-seqs", type=int, default=64,
                    help="sequences the one-process oracle timing covers")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (CPU baseline and parity of the timed outputs)")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="hier, lmhead and tentative paths: run the step back to back this "
                         "long before the counted warm-up steps, so that the timed steps see "
                         "the clocks of sustained load (0: none)")
    ap.add_argument("--rotate", type=int, default=4,
                    help="hier and tentative paths: copies of the logits the steps cycle through (1: every "
                         "step reads the same buffers, whose re-read rows the next step can "
                         "find in the memory-side cache)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a copy of known size (for counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 counter runs into the traffic file and exit")
    ap.add_argument("--path", choices=("hier", "hier_lazy", "lmhead", "tentative", "single"),
                    default="hier",
                    help="hier: the hierarchical verify + rollback step (default); hier_lazy: "
                         "the same step reading only the L_f rows stage 2 can reach; lmhead: "
                         "the fused LM-head verify; tentative: the hierarchy across calls, "
                         "one intermediate round then a flush of the pending tokens; single: "
                         "the single-stage verify on --workload")
    ap.add_argument("--workload", choices=("tiny", "batched", "mixed_temp"), default="batched",
                    help="single path only: the single-stage workload")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="headline only: skip the single-stage and LM-head workloads measured "
                         "after the timed steps")
    ap.add_argument("--byproducts", choices=("none", "entropy", "outcome", "all"), default="none",
                    help="hier path only: also compute the row entropies, the outcome export "
                         "(acceptance mass and the 8 largest residual tokens per position), "
                         "or both, in every step")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification path shards by sequence with no "
              "exchange, so a multi-GPU figure is N independent copies of this one; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.path == "lmhead":
        bench_lmhead(args)
        return
    if args.path == "tentative":
        bench_tentative(args)
        return
    if args.path == "single":
        bench_single(args)
        return

    bench_hier(args)


def _settle(step, ms, sync):
    """Runs ``step`` back to back for ``ms`` of wall time (then synchronises):
    the chip's power management needs tens of milliseconds of sustained load
    before its clocks settle; a serving loop that verifies continuously runs
    in that settled state.  Returns the number of steps run."""
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step(2000000 + n)
            n += 1
        sync()
    return n


def bench_hier(args):
    """The headline: spec_verify_hier_rollback on the hierarchical workload
    (or its lazy / by-product variants)."""
    lazy = args.path == "hier_lazy"
    byp = args.byproducts != "none"
    if lazy and byp:
        raise SystemExit("by-products need every row streamed: use --path hier")
    headline = not lazy and not byp
    import torch
    import workloads

    # inputs: drawn on the host for the headline (the oracle leg reads the same
    # arrays in forked workers), on the device for the other modes
    pool, procs = None, 0
    if headline:
        host = workloads.make("hier", 0, device="cpu")
        if not args.no_cpu_baseline:
            procs = max(1, min(HOST_SHARE, os.cpu_count() or 1))
            pool = oracle_pool(host, procs)
        print("[bench] host inputs ready", file=sys.stderr, flush=True)

    import lossless_token_verification_amd as sv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if headline:
        w = {kk: (v.to(dev) if torch.is_tensor(v) else v) for kk, v in host.items()}
    else:
        w = workloads.make("hier", 0, device=dev)
    B, k, V = w["B"], w["k"], w["V"]
    table0, lens0 = w["block_table"].clone(), w["seq_lens"].clone()
    ws = sv.alloc_workspace(sv.workspace_bytes(B, k, V, torch.bfloat16, 3), dev)
    rows = B * (k + 2 * (k + 1))
    launch_bytes = rows * V * 2          # every logit row of L_d, L_i, L_f read once
    print(f"[bench] workload ready: {rows} rows, {launch_bytes} B per step", file=sys.stderr,
          flush=True)

    call = sv.spec_verify_hier_rollback_lazy if lazy else sv.spec_verify_hier_rollback
    extra = dict(entropy=args.byproducts in ("entropy", "all"),
                 outcome=args.byproducts in ("outcome", "all"))
    extra["top_m"] = 8 if extra["outcome"] else 0

    # The steps cycle through `rotate` copies of the logits, as a serving loop
    # verifies fresh logits every step: a step never finds the rows an earlier
    # step read (the draws re-read up to 197 MB) in the 256 MB memory-side cache.
    copies = [(w["ld_logits"], w["li_logits"], w["lf_logits"])]
    for _ in range(max(1, args.rotate) - 1):
        copies.append(tuple(t.clone() for t in copies[0]))
    # each timed step has its own outputs and its own copy of the initial KV
    # state, so that the first timed step can be checked afterwards
    outs = [sv.spec_verify_hier_rollback(*copies[0], w["draft_tokens"], w["temperature"],
                                         table0.clone(), lens0.clone(),
                                         block_size=w["block_size"], max_freed=1,
                                         window=w["window"], seed=0, offset=999999,
                                         workspace=ws)
            for _ in range(args.steps)]
    kvs = [(table0.clone(), lens0.clone()) for _ in range(args.steps)]
    scratch_kv = (table0.clone(), lens0.clone())
    torch.cuda.synchronize()

    def step(i, events=None, out=None, kv=None):
        # verification of both stages and the paged-KV rollback, one call
        ld, li, lf = copies[i % len(copies)]
        t, l = kv if kv is not None else scratch_kv
        return call(ld, li, lf, w["draft_tokens"], w["temperature"], t, l,
                    block_size=w["block_size"], max_freed=1, window=w["window"], seed=0,
                    offset=i, workspace=ws, events=events, out=out if out is not None else outs[-1],
                    **extra)

    def reset_scratch_kv():
        scratch_kv[0].copy_(table0)
        scratch_kv[1].copy_(lens0)

    settle_steps = 0
    if args.settle_ms > 0:
        def sync():
            torch.cuda.synchronize()
            reset_scratch_kv()     # the rollbacks of the settle steps must not run dry
        settle_steps = _settle(step, args.settle_ms, sync)
    for i in range(args.warmup):
        step(1000000 + i)
    torch.cuda.synchronize()
    ev = HipEvents(2 * args.steps + 2)
    hip = ev.hip
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    hip.hipEventRecord(ev.ev[-2], stream)
    t_host = time.perf_counter()
    for i in range(args.steps):
        step(i, events=(ev.ev[2 * i].value, ev.ev[2 * i + 1].value), out=outs[i], kv=kvs[i])
    t_host = time.perf_counter() - t_host
    hip.hipEventRecord(ev.ev[-1], stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(2 * args.steps, 2 * args.steps + 1)
    k1_ms = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)]
    # step i runs from its statistics kernel's start to the next step's (the
    # last one to the closing event)
    step_ms = [ev.elapsed_ms(2 * i, 2 * (i + 1)) for i in range(args.steps - 1)]
    step_ms.append(ev.elapsed_ms(2 * (args.steps - 1), 2 * args.steps + 1))
    ev.close()
    if args.calibration_copy:
        calibration_copy(dev)

    ms_step = total_ms / args.steps
    k1_avg = sum(k1_ms) / len(k1_ms)
    timing = {"step_us": _dist_us(step_ms), "stream_us": _dist_us(k1_ms),
              "settle_ms": args.settle_ms, "settle_steps": settle_steps}
    if lazy:
        # bytes actually read: the L_d / L_i rows of the first N_i positions;
        # L_f rows 0..a1 of a sequence that rejects a draft there; the rest of
        # the L_d / L_i rows and every L_f row of one that accepts all N_i
        a1 = outs[0]["accept_len_inter"].cpu()
        r0 = min(max(w["window"], 1), k)
        r1 = r0 + (1 if r0 == k else 0)
        open_ = (a1 >= r0) if r0 < k else torch.zeros_like(a1, dtype=torch.bool)
        n_open = int(open_.sum())
        di_rows = B * (r0 + r1) + n_open * (2 * (k - r0) + 1)
        lf_rows = int((a1 + 1)[~open_].sum()) + n_open * (k + 1)
        read_bytes = (di_rows + lf_rows) * V * 2
        line = {
            "metric": "verified draft tokens/s, hierarchical verify with lazy final exit, "
                      "B=256 k=8 V=128256 bf16",
            "value": round(B * k / (ms_step / 1e3), 1), "unit": "verified draft tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "hierarchical verify + KV rollback, L_f rows read only up "
                                   "to each sequence's stage-1 stop", "B": B, "k": k, "V": V,
                       "input_copies": len(copies)},
            "dense_bytes_per_step": launch_bytes, "read_bytes_per_step": read_bytes,
            "ld_li_rows_read": di_rows, "lf_rows_read": lf_rows,
            "hbm_gbps_read": round(read_bytes / (ms_step / 1e3) / 1e9, 1),
            "stats_phase_us": round(k1_avg * 1e3, 2),
            "host_enqueue_us_per_step": round(t_host / args.steps * 1e6, 1), **timing,
        }
        print(json.dumps(line), flush=True)
        return
    if byp:
        k1_gbps = launch_bytes / (k1_avg / 1e3) / 1e9
        name = {"entropy": "row entropies", "outcome": "outcome export (top 8)",
                "all": "row entropies and outcome export (top 8)"}[args.byproducts]
        line = {
            "metric": f"verified draft tokens/s with {name}, hierarchical verify + KV "
                      "rollback, B=256 k=8 V=128256 bf16",
            "value": round(B * k / (ms_step / 1e3), 1), "unit": "verified draft tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"hierarchical verify + KV rollback with {name}",
                       "B": B, "k": k, "V": V, "input_copies": len(copies)},
            "roofline": {"bound": "hbm",
                         "kernel": "rowstats_kernel<bf16, entropy>" if extra["entropy"]
                         else "rowstats_kernel<bf16>",
                         "achieved": round(k1_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(k1_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                         "bytes_per_launch": launch_bytes,
                         "avg_launch_us": round(k1_avg * 1e3, 2)},
            "host_enqueue_us_per_step": round(t_host / args.steps * 1e6, 1), **timing,
        }
        print(json.dumps(line), flush=True)
        return

    value = B * k / (ms_step / 1e3)
    step_gbps = launch_bytes / (ms_step / 1e3) / 1e9
    k1_gbps = launch_bytes / (k1_avg / 1e3) / 1e9
    traffic = _traffic(launch_bytes)
    reread, seq_bound = _draw_and_sequential_bytes(outs[-1], w, B, k, V)
    cpu, parity = None, None
    if pool is not None:
        print("[bench] oracle leg", file=sys.stderr, flush=True)
        res, cpu = oracle_leg(pool, procs, B, k, 0, min(B, args.cpu_p1_seqs))
        kv = (table0.cpu().numpy(), lens0.cpu().numpy(), kvs[0][0].cpu().numpy(),
              kvs[0][1].cpu().numpy(), outs[0]["freed_blocks"].cpu().numpy(),
              outs[0]["num_freed"].cpu().numpy())
        parity = parity_of_step(pool, res, outs[0], 0, kv)
        pool.close()
        pool.join()
        print(f"[bench] oracle: {cpu['value']:.1f} tokens/s on {procs} processes, "
              f"{cpu['p1_value']:.1f} on one; parity {parity}", file=sys.stderr, flush=True)
    others = None
    if not args.no_other_workloads:
        others = other_workloads(dev, parity=not args.no_cpu_baseline)
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
                   "block_size": w["block_size"], "input_copies": len(copies)},
        "host_enqueue_us_per_step": round(t_host / args.steps * 1e6, 1),
        "hbm_gbps_step": round(step_gbps, 1),
        "hbm_frac_of_peak_step": round(step_gbps / HBM_PEAK_GBPS, 4),
        **timing,
        "draw_reread_bytes_last_step": reread,
        "sequential_lower_bound_bytes_last_step": seq_bound,
        "parity": parity,
        "roofline": {"bound": "hbm", "kernel": "rowstats_kernel<bf16>",
                     "achieved": round(k1_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k1_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": launch_bytes, "avg_launch_us": round(k1_avg * 1e3, 2)},
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)
    if parity is not None and (parity["n_mismatched"] or not parity["kv_state_equal"]):
        print("[bench] the first timed step differs from the oracle", file=sys.stderr)
        sys.exit(1)
    bad = [n for n, m in (others or {}).items() if m.get("parity", {}).get("n_mismatched")]
    if bad:
        print(f"[bench] outputs differ from the oracle on: {', '.join(bad)}", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
