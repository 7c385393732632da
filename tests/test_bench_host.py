"""Host logic of bench.py, on the CPU: the one-GPU refusal, the algorithmic
byte counts (checked against the sizes of the arrays each call reads and
writes, taken from the oracle's own layout of a random batch), and the
HBM-counter ingestion (copy calibration, per-launch averages, the source-hash
guard that drops stale counters)."""
import csv
import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr and "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_are_the_arrays_each_call_touches():
    rng = np.random.default_rng(5)
    T, H, E, R, k = 300, 64, 24, 4, 3
    ids = pins.rand_ids(rng, T, E, k)
    lay = oracle.layout(ids, E, R)
    C, P = int(lay["rank_offsets"][-1]), int(lay["expert_offsets"][-1])
    # copies and pairs as the definitions state them
    assert C == sum(len({int(e) // (E // R) for e in row}) for row in ids)
    assert P == T * k
    row = np.zeros((1, H), np.uint16).nbytes
    hidden = T * row
    ids_b = ids.nbytes
    slots_b = lay["token_rank_slot"].nbytes
    pair_b = lay["pair_row"].nbytes
    src_b = np.zeros(C, np.int32).nbytes
    esrc_b = np.zeros(P, np.int32).nbytes
    meta_b = sum(lay[key].nbytes for key in
                 ("rank_counts", "rank_offsets", "expert_counts", "expert_offsets"))
    weights_b = np.zeros((T, k), np.float32).nbytes
    got = bench.algorithmic_bytes(T, H, E, R, k, C, P)
    assert got["layout"] == ids_b + slots_b + pair_b + meta_b
    assert got["pack"] == hidden + C * row + slots_b + src_b
    assert got["permute"] == C * row + P * row + src_b + ids_b + pair_b + esrc_b
    assert got["combine"] == P * row + hidden + pair_b + weights_b
    ts = bench.two_stage_bytes(T, H, R, k, C, P)
    offsets_b = lay["rank_offsets"].nbytes
    assert ts["partial"] == P * row + C * row + src_b + ids_b + pair_b + weights_b + offsets_b
    assert ts["ranks"] == C * row + hidden + slots_b
    for fmt, bits, per in (("mxfp8", 8, 32), ("mxfp4", 4, 32), ("nvfp4", 4, 16)):
        qrow = H * bits // 8 + H // per  # codes + one scale byte per 32 (16) values
        mx = bench.mx_bytes(T, H, R, k, C, P, fmt)
        assert mx["pack"] == hidden + C * qrow + slots_b + src_b
        assert mx["permute"] == C * qrow + P * qrow + src_b + ids_b + pair_b + esrc_b


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for name, grid, value in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": value})


def test_step_bytes_are_the_four_calls():
    """The bench line's bytes per step are the four calls' algorithmic bytes:
    at the prefill shape with C = 18,016 copies and P = 24,576 pairs,
    957,267,784 bytes (the one-call dispatch's own count, also kept by the
    bench, is an alternative to three of them and is not added)."""
    T, H, E, R, k, C, P = 4096, 5120, 384, 8, 6, 18016, 24576
    nb = bench.algorithmic_bytes(T, H, E, R, k, C, P)
    nb.update(bench.whole_dispatch_bytes(T, H, E, R, k, C, P))
    assert bench.path_bytes(nb) == 957267784
    # one launch: the layout's bytes, the hidden rows once, copies and expert rows once
    row = 2 * H
    assert nb["dispatch"] == nb["layout"] + T * row + C * row + 4 * C + P * row + 4 * P
    assert nb["dispatch"] < nb["layout"] + nb["pack"] + nb["permute"]


def test_counter_ingestion_and_stale_source_guard(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    mib = 512.0
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the calibration copy (largest grid) reads half its bytes on FETCH_SIZE;
    # a small copy of another grid size must be ignored
    _counter_csv(fetch, "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", 1 << 20, 262144.0),
        ("__amd_rocclr_copyBuffer", 1024, 7.0),
        ("void (anonymous namespace)::permute_rows<10, false>(...)", 4096, 90000.0),
        ("void (anonymous namespace)::permute_rows<10, false>(...)", 4096, 92000.0),
        ("void (anonymous namespace)::pack_rows<10>(...)", 4096, 20000.0),
    ])
    _counter_csv(write, "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", 1 << 20, 524288.0),
        ("void (anonymous namespace)::permute_rows<10, false>(...)", 4096, 246000.0),
        ("void (anonymous namespace)::pack_rows<10>(...)", 4096, 180000.0),
    ])
    rec = bench.ingest_counters(str(fetch), str(write), mib, "prefill")
    cal = rec["copy_calibration"]
    assert abs(cal["fetch_scale"] - 2.0) < 1e-12 and abs(cal["write_scale"] - 1.0) < 1e-12
    perm = rec["prefill"]["permute"]
    assert perm["fetch_kib_per_launch"] == 91000.0
    assert perm["bytes_per_launch"] == (91000.0 * 2.0 + 246000.0) * 1024
    assert perm["source_sha256_16"] == bench.source_digest()
    assert "combine" not in rec["prefill"]  # no counters, no entry
    assert bench.measured_traffic("permute", "prefill") == perm["bytes_per_launch"]
    assert bench.measured_traffic("permute", "decode") is None
    # counters taken on another version of the kernels are not reported
    stale = json.loads((tmp_path / "traffic.json").read_text())
    stale["prefill"]["permute"]["source_sha256_16"] = "0" * 16
    (tmp_path / "traffic.json").write_text(json.dumps(stale))
    assert bench.measured_traffic("permute", "prefill") is None


def test_trace_passes_split(tmp_path):
    """The per-pass split of a kernel trace: every library kernel's dispatches,
    in dispatch order, cut into the bench's passes (the combine has no
    placement dispatches, the permute none in the pass through moe_dispatch,
    pack_expand_rows runs only there); a count that does not fit is reported,
    not split."""
    steps, warmup, sets = 4, 2, 3
    path = tmp_path / "run_kernel_trace.csv"
    fields = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows, did, t = [], 0, 0

    def add(name, us):
        nonlocal did, t
        did += 1
        rows.append({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": did, "Kernel_Name": name,
                     "Start_Timestamp": t, "End_Timestamp": t + int(us * 1000)})
        t += 10 ** 6

    perm = "void (anonymous namespace)::permute_rows<10, false>(unsigned int const*, int)"
    comb = "void (anonymous namespace)::combine_rows<5, false>(unsigned int const*)"
    expand = "void (anonymous namespace)::pack_expand_rows<1, false, false>(unsigned int const*)"
    size = dict(placement=sets, warmup=warmup)
    for p_i, pas in enumerate(bench.RUN_PASSES):
        for _ in range(size.get(pas, steps)):
            if pas in bench.ONE_CALL_PASSES:
                add(expand, 50)
            else:
                add(perm, 10 + p_i)
            add("void at::native::fill_kernel<int>(int)", 1)
            if pas != "placement":
                add(comb, 100 + p_i)
    add("void (anonymous namespace)::pack_rows<10>(unsigned int const*)", 5)  # one stray dispatch
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)
    out = bench.trace_passes(str(path), steps, warmup, sets)
    assert set(out) == {"permute_rows<10, false>", "combine_rows<5, false>", "pack_rows<10>",
                        "pack_expand_rows<1, false, false>"}
    for p_i, pas in enumerate(bench.RUN_PASSES):
        if pas not in bench.ONE_CALL_PASSES:
            assert out["permute_rows<10, false>"][pas]["mean_us"] == 10 + p_i
        if pas != "placement":
            assert out["combine_rows<5, false>"][pas]["mean_us"] == 100 + p_i
    assert "placement" not in out["combine_rows<5, false>"]
    assert "one_call" not in out["permute_rows<10, false>"]
    assert out["pack_expand_rows<1, false, false>"] == {
        p: {"mean_us": 50.0, "min_us": 50.0, "max_us": 50.0, "n": steps}
        for p in bench.ONE_CALL_PASSES}
    assert out["permute_rows<10, false>"]["roofline"]["n"] == steps
    assert "error" in out["pack_rows<10>"]
