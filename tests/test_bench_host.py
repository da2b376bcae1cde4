"""Host logic of bench.py (CPU, no GPU needed): the one-GPU guard, the step
time distribution, the conversion of rocprofv3 counter files into HBM bytes,
the check that ties the stored traffic to the kernel's sources, and the
comparison of a step's outputs with the oracle (the same code the benchmark
runs on its first timed step), each with a planted difference."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import workloads
from oracle import blocktable, verify

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                         capture_output=True, text=True, timeout=300,
                         env={**os.environ, **env}, cwd=ROOT)
    assert out.returncode == 2, out.stderr[-2000:]
    assert "one GPU" in out.stderr
    assert out.stdout == ""


def test_step_time_distribution():
    d = bench._dist_us([0.001 * (i + 1) for i in range(20)])   # 1..20 us
    assert d["first5"] == [1.0, 2.0, 3.0, 4.0, 5.0]
    assert d["last5"] == [16.0, 17.0, 18.0, 19.0, 20.0]
    assert (d["median"], d["p10"], d["p90"]) == (11.0, 3.0, 19.0)
    one = bench._dist_us([0.25])
    assert one["median"] == one["p10"] == one["p90"] == 250.0


def _counter_dir(path, counter, stats_kib, copy_kib):
    """A rocprofv3-style counter_collection.csv: two unrelated dispatches, the
    row-statistics kernel, the three calibration copies, then the runtime's
    read-back copy."""
    os.makedirs(path)
    rows, i = [], 0

    def add(name, value):
        nonlocal i
        i += 1
        rows.append({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                     "Counter_Value": value})

    add("void at::native::normal_kernel(...)", 12345.0)
    add("void sv::(anonymous namespace)::verify_kernel<1>(sv::VerifyArgs)", 777.0)
    for v in stats_kib:
        add("void sv::(anonymous namespace)::rowstats_kernel<1, false>(sv::StatsArgs)", v)
    for v in copy_kib:
        add("void at::native::vectorized_elementwise_kernel<4, MulFunctor>(...)", v)
    add("__amd_rocclr_copyBuffer", 1.0)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_traffic_from_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gib_kib = bench.COPY_ELEMS * 4 / 1024.0
    # the copy reads 1 GiB but FETCH_SIZE counts half of it; writes count in full
    _counter_dir(tmp_path / "f", "FETCH_SIZE", [800000.0, 800002.0], [gib_kib / 2] * 3)
    _counter_dir(tmp_path / "w", "WRITE_SIZE", [834.0, 834.0], [gib_kib] * 3)
    bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["dispatches"] == [2, 2]
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["hbm_fetch_bytes_per_launch"] == int(800001.0 * 1024 * 2.0)
    assert t["hbm_write_bytes_per_launch"] == int(834.0 * 1024)
    assert t["hbm_bytes_per_launch"] == int(800001.0 * 1024 * 2.0 + 834.0 * 1024)
    assert t["rowstats_source_sha256"] == bench._rowstats_sha()
    # reported while the kernel's sources are unchanged, and only then
    assert bench._traffic(1) == t["hbm_bytes_per_launch"]
    t["rowstats_source_sha256"] = "0" * 64
    json.dump(t, open(tmp_path / "traffic.json", "w"))
    assert bench._traffic(1) is None


def test_traffic_from_needs_the_calibration_copy_last(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    _counter_dir(tmp_path / "f", "FETCH_SIZE", [800000.0], [1.0, 1.0])   # two copies only
    _counter_dir(tmp_path / "w", "WRITE_SIZE", [834.0], [1.0, 1.0])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))
    assert not os.path.exists(tmp_path / "traffic.json")


def test_committed_traffic_file_matches_the_sources():
    """The committed counter summary was taken on the current row-statistics
    sources (otherwise the benchmark reports no traffic)."""
    t = json.load(open(bench.TRAFFIC_FILE))
    assert t["rowstats_source_sha256"] == bench._rowstats_sha()
    assert 1.0 <= t["hbm_bytes_per_launch"] / 1707343872 < 1.01


def test_single_parity_counts_a_planted_difference():
    w = workloads.make_single(12, 3, 3000, dtype="bf16", temps=(1.0, 0.0), seed=(91, 1))
    d = workloads.to_numpy_raw(w["draft_logits"])
    t = workloads.to_numpy_raw(w["target_logits"])
    ref = verify.spec_verify_single(d, t, w["draft_tokens"].numpy(), w["temperature"].numpy(),
                                    0, 5)
    gpu = {k: torch.from_numpy(ref[k].copy()) for k in bench.SINGLE_KEYS}
    p = bench._single_parity(w, gpu, 5)
    assert p["n_mismatched"] == 0 and p["sequences"] == 12
    assert p["exact"] + p["near_tie_as_oracle"] == 12
    b = next(b for b in range(12) if verify.near_tie_event(ref["infos"][b]) is None)
    gpu["out_tokens"][b, 0] = (gpu["out_tokens"][b, 0] + 1) % 3000
    p = bench._single_parity(w, gpu, 5)
    assert p["n_mismatched"] == 1 and p["mismatched"] == [b]


def test_step_parity_with_the_oracle_pool():
    """The benchmark's oracle leg on a small hierarchical batch: forked
    workers, the CPU baseline record, and the step comparison (outputs and the
    rolled-back KV state), clean and with planted differences."""
    B, k = 6, 4
    host = workloads.make_hier(B, k, 2000, temps=(1.0, 0.0), window=4, seed=(92, 1),
                               ctx=(16, 64))
    pool = bench.oracle_pool(host, 2)
    try:
        res, cpu = bench.oracle_leg(pool, 2, B, k, 3, 2)
        assert sorted(res) == list(range(B))
        assert cpu["kind"] == "oracle" and cpu["cores"] == 2 and cpu["p1_sequences"] == 2
        assert cpu["value"] > 0 and cpu["p1_value"] > 0
        keys = ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop")
        gpu = {kk: torch.from_numpy(np.stack([res[b][0][kk] for b in range(B)])) for kk in keys}
        t0, l0 = host["block_table"].numpy(), host["seq_lens"].numpy()
        t1, l1, f1, n1 = blocktable.kv_blocktable_truncate(t0, l0, gpu["num_drop"].numpy(), 16, 1)
        gpu["freed_blocks"], gpu["num_freed"] = torch.from_numpy(f1), torch.from_numpy(n1)
        kv = (t0, l0, t1, l1, f1, n1)
        p = bench.parity_of_step(pool, res, gpu, 3, kv)
        assert p["n_mismatched"] == 0 and p["kv_state_equal"] and p["sequences"] == B
        # a wrong KV state is caught on its own
        bad_len = l1.copy()
        bad_len[0] += 1
        p = bench.parity_of_step(pool, res, gpu, 3, (t0, l0, t1, bad_len, f1, n1))
        assert p["n_mismatched"] == 0 and not p["kv_state_equal"]
        # and so is a wrong accepted length of a sequence without a near tie
        b = next(b for b in range(B) if verify.near_tie_event(res[b][1]) is None)
        gpu["accept_len_inter"][b] += 1
        p = bench.parity_of_step(pool, res, gpu, 3, kv)
        assert p["n_mismatched"] == 1 and p["mismatched"] == [b]
    finally:
        pool.close()
        pool.join()
