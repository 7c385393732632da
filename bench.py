"""Benchmark: one step = one pass of the whole hot path (layout, pack,
permute, combine) over one batch of seeded synthetic input already resident in
HBM, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill] [--sets 3]
    python bench.py --sweep [tiny,decode,prefill,skew,adv]

The default mode prints ONE JSON line: dispatch+combine throughput in GB/s of
algorithmic bytes (what the method must move, with the measured copy count C
and pair count P) and its fraction of the 8 TB/s HBM peak. The value comes
from steps that rotate through `--sets` complete buffer sets (inputs, expert
outputs and every output buffer), so that no step finds in L2 or the Infinity
Cache anything the step before it read or wrote, as consecutive layers or
batches would not; within a step the calls hand their results on as they do
in a layer. Beside it (`modes`): the same steps on one buffer set back to back
(warm), the rotated steps again right after a 1 GiB write by another kernel
(after_write: a large write changes how the Infinity Cache keeps the pack's
rows for the permute), and the sum of per-call times with L2 and the Infinity
Cache evicted before every call (cold). Also: per-call times, the load per destination rank
(max over mean), the roofline of the dominant kernel (permute: its algorithmic
bytes over its own duration, from a HIP event pair that the runtime records
with the kernel's dispatch on the stream it runs on), and the CPU oracle timed
on a bounded sample of the same workload.

--sweep measures every workload per call in the same three modes (warm,
rotated, cold; the cold eviction is a 1 GiB read, not a write, so that no dirty
lines of its own are written back inside the timed call): 5 warm-up steps,
then the median of 30 calls, repeated 3 times; next to it a plain 1 GiB device
copy as the achievable rate, and the oracle pinned to one core (median of 5
steps, 3 for the two large workloads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "dispatch+combine GB/s and % HBM peak, T=4096 H=5120 E=384 top-6 R=8"
KERNEL_SOURCE = os.path.join(ROOT, "combine_topk_ids_02_amd", "csrc", "moe_dispatch.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CALLS = ("layout", "pack", "permute", "combine")
TWO_STAGE_CALLS = ("partial", "ranks")


def algorithmic_bytes(T, H, E, R, k, C, P):
    """Bytes each call must move at least (each row read once, each copy
    written once, plus the index arrays it reads and writes)."""
    row = 2 * H
    return {
        "layout": 4 * T * k + 4 * T * R + 4 * T * k + 8 * (E + R + 1),
        "pack": T * row + C * row + 4 * T * R + 4 * C,
        "permute": C * row + P * row + 4 * C + 8 * T * k + 4 * P,
        "combine": P * row + T * row + 8 * T * k,
    }


def path_bytes(nbytes: dict) -> int:
    """Bytes of one step of the one-stage path: the four calls' algorithmic
    bytes (other entries, such as the one-call dispatch's, are alternatives to
    some of these calls and are not added)."""
    return sum(nbytes[c] for c in CALLS)


def whole_dispatch_bytes(T, H, E, R, k, C, P, fmt=None):
    """Bytes of moe_dispatch (or with fmt moe_dispatch_quantised) in its
    one-launch form: the layout's, each bf16 hidden row read once, each copy
    and each expert row written once (bf16, or codes and scales) with its
    source id (the packed rows are not read back, so this is less than the
    three calls' sum and is reported on its own)."""
    if fmt:
        bits, blk = WIRE[fmt]
        out_row = H * bits // 8 + H // blk
    else:
        out_row = 2 * H
    return {"dispatch": algorithmic_bytes(T, H, E, R, k, C, P)["layout"] + T * 2 * H
            + C * out_row + 4 * C + P * out_row + 4 * P}


# Quantised wire formats: name -> (code bits per value, values per scale byte).
WIRE = {"mxfp8": (8, 32), "mxfp4": (4, 32), "nvfp4": (4, 16)}


def mx_bytes(T, H, R, k, C, P, fmt="mxfp8"):
    """Bytes of the quantised dispatch: the fused quantise-and-pack reads each
    bf16 hidden row once and writes H*bits/8 code bytes + H/block scales per
    copy; the permute reads each quantised rank row once and writes it once
    per pair."""
    bits, blk = WIRE[fmt]
    qrow = H * bits // 8 + H // blk
    return {
        "pack": 2 * T * H + C * qrow + 4 * T * R + 4 * C,
        "permute": C * qrow + P * qrow + 4 * C + 8 * T * k + 4 * P,
    }


def two_stage_bytes(T, H, R, k, C, P):
    """Bytes of the two-stage combine: the per-rank partial rows (each expert
    row read once, each partial row written once, the token's ids, pair rows
    and weights read once) and the home sum (each partial row read once, each
    output row written once, the slots read once)."""
    row = 2 * H
    return {
        "partial": P * row + C * row + 4 * C + 12 * T * k + 4 * (R + 1),
        "ranks": C * row + T * row + 4 * T * R,
    }


def source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, only if the kernel source has not changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_sha256_16") != source_digest():
        return None
    return ent.get("bytes_per_launch")


OUR_KERNELS = ("layout_count", "layout_tiles", "pack_rows", "permute_rows", "combine_rows",
               "dispatch_small", "pack_expand_rows", "pack_expand_q")


# The passes of a default bench run, in order, in units of steps: each step
# of the four calls launches every library kernel of the path once. `sets`
# steps come first (layout, pack and permute once per buffer set, to place the
# expert outputs), then the warm-up and five passes of `steps` steps each, two
# passes of `steps` steps through moe_dispatch (layout, pack_expand_rows,
# combine; cold, then rotated) and the roofline pass.
RUN_PASSES = ("placement", "warmup", "rotated", "warm", "after_write", "per_call", "cold",
              "one_call_cold", "one_call", "roofline")
ONE_CALL_PASSES = ("one_call_cold", "one_call")


def passes_of(kernel: str) -> tuple:
    """The passes of a default bench run in which `kernel` is launched."""
    if kernel.startswith("pack_expand"):
        return ONE_CALL_PASSES
    if kernel.startswith(("pack_rows", "permute_rows")):
        return tuple(p for p in RUN_PASSES if p not in ONE_CALL_PASSES)
    if kernel.startswith("combine_rows"):
        return RUN_PASSES[1:]
    return RUN_PASSES


def trace_passes(trace_csv: str, steps: int, warmup: int, sets: int) -> dict:
    """Per library kernel and per pass of a default bench run, the mean, min
    and max duration (us) of its dispatches in a rocprofv3 kernel trace
    (run_kernel_trace.csv of `rocprofv3 --kernel-trace -- python3 bench.py`),
    so that the roofline pass can be compared with the bench line's own
    kernel time."""
    import csv
    import re

    durs = {}
    with open(trace_csv) as f:
        for row in csv.DictReader(f):
            name = re.sub(r"\(.*", "", row["Kernel_Name"].replace("void ", "").replace(
                "(anonymous namespace)::", ""))
            if not name.startswith(OUR_KERNELS):
                continue
            durs.setdefault(name, []).append(
                (int(row["Dispatch_Id"]), (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3))
    size = dict(placement=sets, warmup=warmup)
    out = {}
    for name, d in durs.items():
        d.sort()
        passes = passes_of(name)
        sz = [size.get(p, steps) for p in passes]
        if len(d) != sum(sz):
            out[name] = {"error": f"{len(d)} dispatches, expected {sum(sz)}"}
            continue
        res, i = {}, 0
        for pas, n in zip(passes, sz):
            v = [x for _, x in d[i:i + n]]
            i += n
            if v:
                res[pas] = {"mean_us": round(sum(v) / len(v), 2), "min_us": round(min(v), 2),
                            "max_us": round(max(v), 2), "n": len(v)}
        out[name] = res
    return out


def ingest_counters(fetch_csv: str, write_csv: str, calib_mib: float, workload: str) -> dict:
    """Per-launch HBM traffic of each kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), each scaled by what the same
    counter reads for the plain device copy of calib_mib MiB that
    --copy-calibration runs first. Writes profiles/traffic.json."""
    import csv

    def per_kernel(path, counter):
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        # the calibration copies: the runtime's copy kernel at its largest grid
        copies = [r for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        big = max(int(r["Grid_Size"]) for r in copies)
        acc = {"copy": [float(r["Counter_Value"]) for r in copies if int(r["Grid_Size"]) == big]}
        for r in rows:
            key = next((k for k in OUR_KERNELS if k in r["Kernel_Name"]), None)
            if key is not None:
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    nbytes = calib_mib * 2 ** 20
    f_fetch = nbytes / (fetch["copy"] * 1024)
    f_write = nbytes / (write["copy"] * 1024)
    rec = {"copy_calibration": {"bytes_each_way": nbytes, "fetch_kib": fetch["copy"],
                                "write_kib": write["copy"], "fetch_scale": f_fetch,
                                "write_scale": f_write}}
    out = {}
    for k in OUR_KERNELS:
        if k in fetch and k in write:
            rd = fetch[k] * 1024 * f_fetch
            wr = write[k] * 1024 * f_write
            out[k.replace("_rows", "").replace("_tiles", "")] = {
                "fetch_kib_per_launch": fetch[k], "write_kib_per_launch": write[k],
                "read_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr,
                "source_sha256_16": source_digest()}
    try:  # other workloads' entries are kept
        with open(TRAFFIC_FILE) as f:
            prev = json.load(f)
    except (OSError, ValueError):
        prev = {}
    prev.update(rec)
    prev[workload] = out
    rec = prev
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    return rec


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class one_core:
    """Pins the calling process to one host core for the duration."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(self.saved)})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)


def host_description() -> str:
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"1 thread of {len(os.sched_getaffinity(0))} host cores ({model})"


def oracle_step(w, hid, ids, wts, eo):
    import oracle

    T, k = ids.shape
    lay = oracle.layout(ids, w.E, w.R)
    rb, src, _ = oracle.pack(hid, lay["token_rank_slot"], T * min(k, w.R))
    oracle.permute(rb, src, lay, ids, w.E, T * k)
    oracle.combine(eo, lay["pair_row"], wts, want_f32=False)
    return int(lay["rank_offsets"][-1]), int(lay["expert_offsets"][-1])


def cpu_baseline(w, hid, ids, wts, y, budget_s: float):
    """The oracle as it stands, pinned to one core, on the same workload: whole
    steps (layout, pack, permute, combine) repeated until `budget_s` is used."""
    import oracle

    T, k = ids.shape
    lay = oracle.layout(ids, w.E, w.R)
    eo = oracle.place_slots(y, lay["pair_row"], T * k)
    reps, t_total = 0, 0.0
    C = P = 0
    with one_core():
        while t_total < budget_s or reps == 0:
            t0 = time.perf_counter()
            C, P = oracle_step(w, hid, ids, wts, eo)
            t_total += time.perf_counter() - t0
            reps += 1
    nbytes = sum(algorithmic_bytes(T, w.H, w.E, w.R, k, C, P).values())
    return {
        "value": round(nbytes * reps / t_total / 1e9, 3), "unit": "GB/s", "cores": 1,
        "kind": "oracle", "ms_per_step": round(1e3 * t_total / reps, 2),
        "sample": f"{reps} whole {w.name} steps (layout+pack+permute+combine), "
                  f"{t_total:.1f} s, {host_description()}",
    }


def oracle_median(w, hid, ids, wts, y, reps: int) -> dict:
    """Median wall time of `reps` whole oracle steps, pinned to one core."""
    import numpy as np

    import oracle

    T, k = ids.shape
    lay = oracle.layout(ids, w.E, w.R)
    eo = oracle.place_slots(y, lay["pair_row"], T * k)
    times = []
    with one_core():
        for _ in range(reps):
            t0 = time.perf_counter()
            C, P = oracle_step(w, hid, ids, wts, eo)
            times.append(time.perf_counter() - t0)
    ms = float(np.median(times)) * 1e3
    nbytes = sum(algorithmic_bytes(T, w.H, w.E, w.R, k, C, P).values())
    return {"ms_per_step": round(ms, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 3),
            "reps": reps, "host": host_description()}


class Rig:
    """One workload resident on the GPU with every buffer of a pass, in `sets`
    complete copies (inputs, expert outputs and every output buffer), and the
    four library calls on the current stream. Stepping through the copies in
    turn (rotate) gives each step a batch at addresses the previous steps did
    not touch, as consecutive layers or batches of a model would: nothing a
    step reads is still in L2 or the Infinity Cache from the step before."""

    def __init__(self, w, dev, two_stage: bool = False, align: int = 1, block: int = 0,
                 mx_bits=0, sets: int = 1):
        import torch

        import combine_topk_ids_02_amd as moe
        import synth
        from synth import staging

        self.w, self.dev, self.moe = w, dev, moe
        log(f"generating {w.describe()} ({sets} buffer set{'s' if sets > 1 else ''})")
        self.hid = synth.hidden(w)
        self.ids, self.wts = synth.routing(w)
        self.y = synth.expert_out_slots(w.seed, w.E, w.H, self.ids)
        self.shape = moe.Shape(w.T, w.H, w.E, w.R, w.k, align, block)
        # quantised dispatch: a format name of WIRE, or the bits 8 / 4 of an MX one
        self.wire = {8: "mxfp8", 4: "mxfp4", 0: None}.get(mx_bits, mx_bits)
        self.mx_bits = WIRE[self.wire][0] if self.wire else 0
        self.two_stage = two_stage
        y_d = staging.rows_to_device(self.y, dev)
        self.sets = [self._make_set(y_d) for _ in range(sets)]
        del y_d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.turn = 0
        self.cur = self.sets[0]
        b = self.cur.buf
        self.C = int(b.rank_offsets[-1].item())
        # pairs placed (a full block drops the rest) and padding rows marked
        counts = b.expert_counts.long()
        self.P = int((counts.clamp(max=block) if block else counts).sum().item())
        self.pad_rows = int(b.expert_offsets[-1].item()) - self.P
        self.nbytes = algorithmic_bytes(w.T, w.H, w.E, w.R, w.k, self.C, self.P)
        self.nbytes["permute"] += 4 * self.pad_rows + (8 * (w.E + 1) if self.pad_rows else 0)
        self.stream = torch.cuda.current_stream(dev)
        self.calls = CALLS
        if mx_bits:
            self.nbytes.update(mx_bytes(w.T, w.H, w.R, w.k, self.C, self.P, self.wire))
            self.nbytes["permute"] += 4 * self.pad_rows + (8 * (w.E + 1) if self.pad_rows else 0)
        if two_stage:
            self.nbytes.update(two_stage_bytes(w.T, w.H, w.R, w.k, self.C, self.P))
            self.calls = CALLS + TWO_STAGE_CALLS
        self.nbytes.update(whole_dispatch_bytes(w.T, w.H, w.E, w.R, w.k, self.C, self.P,
                                                self.wire))

    def _make_set(self, y_d):
        import types

        import torch

        from synth import staging

        moe, w, dev, sh = self.moe, self.w, self.dev, self.shape
        s = types.SimpleNamespace()
        s.buf = moe.Buffers(sh, dev)
        s.hid_d = staging.rows_to_device(self.hid, dev)
        s.ids_d = torch.from_numpy(self.ids).to(dev)
        s.wts_d = torch.from_numpy(self.wts).to(dev)
        # a first layout gives pair_row for placing the expert outputs
        moe.dispatch(s.buf, s.hid_d, s.ids_d)
        s.expert_out = staging.place_expert_outputs(y_d, s.buf.pair_row, sh.cap_expert)
        if self.mx_bits:
            # quantised dispatch: codes and scales replace the bf16 rank and expert rows
            u8 = torch.uint8
            bits, blk = WIRE[self.wire]
            qw = w.H * bits // 8
            s.rank_q = torch.empty((sh.cap_rank, qw), dtype=u8, device=dev)
            s.rank_s = torch.empty((sh.cap_rank, w.H // blk), dtype=u8, device=dev)
            s.exp_q = torch.empty((sh.cap_expert, qw), dtype=u8, device=dev)
            s.exp_s = torch.empty((sh.cap_expert, w.H // blk), dtype=u8, device=dev)
            s.buf.rank_buf = s.buf.expert_buf = None
        if self.two_stage:
            s.partial = torch.empty((sh.cap_rank, w.H), dtype=torch.bfloat16, device=dev)
            s.out2 = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
        return s

    def rotate(self) -> None:
        """Move on to the next buffer set (a no-op with one set)."""
        self.turn = (self.turn + 1) % len(self.sets)
        self.cur = self.sets[self.turn]

    def imbalance(self) -> dict:
        """Load per destination rank, max over mean: rank-buffer rows (token
        copies) and pairs (expert rows), as the pages measure the busiest GPU
        against the average ("A2A backends" page, section 1.3; "Beyond One
        GPU", section 6)."""
        b, R = self.cur.buf, self.w.R
        rows = b.rank_counts.double()
        pairs = b.expert_counts.double().reshape(R, -1).sum(dim=1)
        ratio = lambda x: round(float(x.max() / x.mean()), 4) if float(x.mean()) > 0 else None
        return {"rank_rows_max_over_mean": ratio(rows),
                "rank_pairs_max_over_mean": ratio(pairs),
                "rank_rows": [int(v) for v in b.rank_counts.tolist()],
                "rank_pairs": [int(v) for v in pairs.tolist()]}

    def call(self, name: str) -> None:
        moe, s, x = self.moe, self.shape, self.cur
        b = x.buf
        if name == "layout":
            moe.layout(x.ids_d, s.E, s.R, s.H, align=s.align, block=s.block, err=b.err,
                       out=b.layout_dict(), workspace=b.workspace)
        elif name == "pack" and self.mx_bits:
            moe.pack_mx(self.wire, x.hid_d, b.token_rank_slot, s.E, s.k, x.rank_q,
                        x.rank_s, b.rank_src_token, err=b.err)
        elif name == "pack":
            moe.pack(x.hid_d, b.token_rank_slot, s.E, s.k, b.rank_buf, b.rank_src_token,
                     err=b.err)
        elif name == "permute" and self.mx_bits:
            moe.permute_mx(self.wire, x.rank_q, x.rank_s, b.rank_src_token,
                           b.rank_offsets, x.ids_d, b.pair_row, s.E, x.exp_q, x.exp_s,
                           b.expert_src_pair, expert_counts=b.expert_counts,
                           expert_offsets=b.expert_offsets, align=s.align, block=s.block,
                           err=b.err)
        elif name == "permute":
            moe.permute(b.rank_buf, b.rank_src_token, b.rank_offsets, x.ids_d, b.pair_row,
                        s.E, b.expert_buf, b.expert_src_pair, expert_counts=b.expert_counts,
                        expert_offsets=b.expert_offsets, align=s.align, block=s.block,
                        err=b.err)
        elif name == "dispatch" and self.mx_bits:
            moe.dispatch_all_mx(self.wire, x.hid_d, x.ids_d, s.E, s.R, b.layout_dict(),
                                x.rank_q, x.rank_s, b.rank_src_token, x.exp_q, x.exp_s,
                                b.expert_src_pair, align=s.align, block=s.block,
                                workspace=b.workspace, err=b.err)
        elif name == "dispatch":
            moe.dispatch_all(x.hid_d, x.ids_d, s.E, s.R, b.layout_dict(), b.rank_buf,
                             b.rank_src_token, b.expert_buf, b.expert_src_pair,
                             align=s.align, block=s.block, workspace=b.workspace, err=b.err)
        elif name == "combine":
            moe.combine(x.expert_out, b.pair_row, x.wts_d, s.E, s.R, b.out, err=b.err)
        elif name == "partial":
            moe.combine_rank_partial(x.expert_out, b.rank_src_token, b.rank_offsets,
                                     x.ids_d, b.pair_row, x.wts_d, s.E, x.partial,
                                     err=b.err)
        else:
            moe.combine_ranks(x.partial, b.token_rank_slot, s.E, s.k, x.out2, err=b.err)

    def step(self, ev=None, evict=None, rotate: bool = True, calls=None) -> None:
        """One pass, on the next buffer set if `rotate` (else on the current
        one again); with `ev` (events) records between the calls; with `evict`
        (a callable that enqueues a cache-evicting read) runs it before every
        call, outside the events. calls: the rig's path, or those given."""
        if rotate:
            self.rotate()
        calls = self.calls if calls is None else calls
        for i, c in enumerate(calls):
            if evict is not None:
                evict()
            if ev is not None:
                ev[2 * i if evict is not None else i].record(self.stream)
            self.call(c)
            if ev is not None and evict is not None:
                ev[2 * i + 1].record(self.stream)
        if ev is not None and evict is None:
            ev[len(calls)].record(self.stream)

    def kernel_ms(self, call: str, n: int, rotate: bool = True) -> list:
        """Durations (ms) of the kernel that `call` launches, inside n whole
        steps: the library has the runtime record an event pair with that
        kernel's dispatch (moe_testing_time_next_launch), so the pair brackets
        the kernel alone, as a kernel trace measures it."""
        import torch

        import combine_topk_ids_02_amd as moe

        pairs = []
        for _ in range(n):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(self.stream)  # creates the events; the kernel records them again
            b.record(self.stream)
            pairs.append((a, b))
        torch.cuda.synchronize()
        for a, b in pairs:
            if rotate:
                self.rotate()
            for c in self.calls:
                if c == call:
                    moe.time_next_launch(a, b)
                self.call(c)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in pairs]

    def per_call_ms(self, n: int, evict=None, rotate: bool = True, calls=None) -> dict:
        """Per-call durations (ms) over n steps (of the rig's path, or of
        `calls`)."""
        import torch

        calls = self.calls if calls is None else calls
        nc = len(calls)
        nev = 2 * nc if evict is not None else nc + 1
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            self.step(evs[i], evict, rotate, calls)
        torch.cuda.synchronize()
        out = {c: [] for c in calls}
        for ev in evs:
            for j, c in enumerate(calls):
                a, b = (ev[2 * j], ev[2 * j + 1]) if evict is not None else (ev[j], ev[j + 1])
                out[c].append(a.elapsed_time(b))
        return out

    def graph_step_us(self, n: int = 200, calls=CALLS, per_graph: int = 20) -> float:
        """`per_graph` steps recorded in one HIP graph (as a decode loop records
        the MoE layers of a forward pass), replayed back to back: the step's GPU
        time without host launch gaps and without the fixed cost of submitting
        a graph, which for one short step alone is longer than the step (about
        13 us per replay here). calls: the one-stage path, layout, pack,
        permute and combine, or ("dispatch", "combine")."""
        import torch

        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                for c in calls:
                    self.call(c)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(steps: int) -> float:
            reps = max(1, steps // per_graph)
            torch.cuda.synchronize()
            a.record()
            for _ in range(reps):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / (reps * per_graph) * 1e3

        # The first replays of a new graph run slower, and an idle GPU takes a
        # while to raise its clocks: replay for about 30 ms before timing.
        est = timed(20)
        timed(min(20000, max(20, int(30e3 / max(est, 1.0)))))
        return timed(n)

    def check_err(self) -> None:
        for x in self.sets:
            e = int(x.buf.err.item())
            if e != 0:
                print(f"bench.py: device error word {e} on {self.w.name}", file=sys.stderr)
                sys.exit(1)


def copy_reference(dev, gib: float = 1.0, reps: int = 10) -> dict:
    """A plain device-to-device copy of `gib` GiB: the achievable rate."""
    import numpy as np
    import torch

    n = int(gib * 2 ** 30)
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    del src, dst
    return {"bytes": 2 * n, "us": round(ms * 1e3, 1), "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}


# Measurement modes: warm = the same buffers back to back; rotated = a
# different complete buffer set each step; cold = a 1 GiB read evicts L2 and
# the Infinity Cache before every call.
MODE_NAMES = ("warm", "rotated", "cold")


def sweep(names, dev, with_oracle: bool) -> None:
    import numpy as np
    import torch

    import synth

    # Cold calls: a 1 GiB read (a sum into a preallocated scalar) before each
    # call replaces L2 and the 256 MB Infinity Cache with clean lines.
    flush = torch.ones(2 ** 30, dtype=torch.uint8, device=dev)
    acc = torch.zeros((), dtype=torch.int32, device=dev)

    def evict() -> None:
        torch.sum(flush, dim=0, dtype=torch.int32, out=acc)

    modes = (("warm", None, False), ("rotated", None, True), ("cold", evict, False))
    copy = copy_reference(dev)
    log(f"1 GiB device copy: {copy['GB/s']} GB/s")
    print(json.dumps({"copy_1GiB": copy}), flush=True)
    rows = []
    for spec in names:
        # "name" or "name:align=128" / "name:block=128" (padded or masked expert layout)
        name, _, opt = spec.partition(":")
        opts = dict(kv.split("=") for kv in opt.split(",") if "=" in kv)
        align, block = int(opts.get("align", 1)), int(opts.get("block", 0))
        flags = opt.split(",")
        wire = next((f for f in flags if f in WIRE), 0)
        w = synth.WORKLOADS[name]
        rig = Rig(w, dev, two_stage=True, align=align, block=block, mx_bits=wire, sets=2)
        for _ in range(5):
            rig.step()
        res = {"workload": w.describe(), "layout_shape": {"align": align, "block": block},
               "dispatch_format": wire or "bf16",
               "C": rig.C, "P": rig.P, "padding_rows": rig.pad_rows,
               "copies_per_token": round(rig.C / max(w.T, 1), 4),
               "imbalance": rig.imbalance(), "calls": {}}
        for mode, fl, rot in modes:
            meds = {c: [] for c in rig.calls}
            for _ in range(3):
                ms = rig.per_call_ms(30, fl, rot)
                for c in rig.calls:
                    meds[c].append(float(np.median(ms[c])))
            for c in rig.calls:
                us = float(np.median(meds[c])) * 1e3
                ent = res["calls"].setdefault(c, {"bytes": rig.nbytes[c]})
                ent[mode] = {"us": round(us, 2),
                             "us_spread": [round(min(meds[c]) * 1e3, 2),
                                           round(max(meds[c]) * 1e3, 2)],
                             "GB/s": round(rig.nbytes[c] / (us * 1e-6) / 1e9, 1)}
                ent[mode]["pct_peak"] = round(100 * ent[mode]["GB/s"] / HBM_PEAK_GBS, 1)
            log(f"{name} {mode}: " + ", ".join(
                f"{c} {res['calls'][c][mode]['us']} us" for c in rig.calls))
        rig.check_err()
        tot = sum(rig.nbytes[c] for c in CALLS)
        path2 = ("layout", "pack", "permute") + TWO_STAGE_CALLS
        tot2 = sum(rig.nbytes[c] for c in path2)
        for mode in MODE_NAMES:
            us = sum(res["calls"][c][mode]["us"] for c in CALLS)
            res[mode] = {"us": round(us, 2), "GB/s": round(tot / (us * 1e-6) / 1e9, 1),
                         "pct_peak": round(100 * tot / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
            us2 = sum(res["calls"][c][mode]["us"] for c in path2)
            res["two_stage_" + mode] = {
                "us": round(us2, 2), "GB/s": round(tot2 / (us2 * 1e-6) / 1e9, 1),
                "pct_peak": round(100 * tot2 / (us2 * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
        warm = res["calls"]
        res["rows_per_s"] = {
            "pack_copies": round(rig.C / (warm["pack"]["warm"]["us"] * 1e-6)),
            "permute_pairs": round(rig.P / (warm["permute"]["warm"]["us"] * 1e-6)),
            "combine_tokens": round(w.T / (warm["combine"]["warm"]["us"] * 1e-6)),
            "combine_pairs": round(rig.P / (warm["combine"]["warm"]["us"] * 1e-6))}
        res["bytes"] = tot
        res["two_stage_bytes"] = tot2
        us_g = rig.graph_step_us()
        res["graph"] = {"us_per_step": round(us_g, 2),
                        "note": "layout, pack, permute, combine replayed from one HIP graph"}
        log(f"{name}: graph replay {us_g:.1f} us per step")
        us_d = rig.graph_step_us(calls=("dispatch", "combine"))
        one = w.T <= 64 or (w.T <= 256 and w.k in (1, 2, 4, 6, 8))
        form = "one launch" if one else "three calls" if wire else "pack+permute kernel"
        bytes_d = path_bytes(rig.nbytes) if form == "three calls" else \
            rig.nbytes["dispatch"] + rig.nbytes["combine"]
        res["graph_whole_dispatch"] = {
            "us_per_step": round(us_d, 2), "bytes": bytes_d,
            "GB/s": round(bytes_d / (us_d * 1e-6) / 1e9, 1),
            "one_launch": one, "form": form,
            "note": ("moe_dispatch_quantised" if wire else "moe_dispatch") +
                    " (one launch for a decode-sized batch; past it the layout "
                    "and one pack-and-permute kernel, or the three calls for a wire format) "
                    "and combine, replayed from a HIP graph"}
        log(f"{name}: graph replay with the one-call dispatch {us_d:.1f} us per step")
        if with_oracle and align == 1 and block == 0 and not wire:
            log(f"{name}: oracle")
            res["oracle"] = oracle_median(w, rig.hid, rig.ids, rig.wts, rig.y,
                                          3 if w.T * w.H > 2 ** 25 else 5)
        print(json.dumps(res), flush=True)
        rows.append((spec, res))
        del rig
        torch.cuda.empty_cache()
    # human-readable table
    print("\n| workload | mode | layout us | pack us | permute us | combine us | total us "
          "| GB/s | % of 8 TB/s | oracle ms/step |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for name, r in rows:
        for mode in MODE_NAMES:
            orc = r.get("oracle", {}).get("ms_per_step", "") if mode == "warm" else ""
            print(f"| {name} | {mode} | " + " | ".join(
                str(r["calls"][c][mode]["us"]) for c in CALLS) +
                f" | {r[mode]['us']} | {r[mode]['GB/s']} | {r[mode]['pct_peak']} | {orc} |")
    print("\nTwo-stage combine (per-rank partial rows, then the home sum), and the whole path "
          "with it in place of the one-stage combine:\n")
    print("| workload | mode | partial us | partial GB/s | ranks us | ranks GB/s | path us "
          "| path GB/s | % of 8 TB/s |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, r in rows:
        for mode in MODE_NAMES:
            a, b, p = r["calls"]["partial"][mode], r["calls"]["ranks"][mode], \
                r["two_stage_" + mode]
            print(f"| {name} | {mode} | {a['us']} | {a['GB/s']} | {b['us']} | {b['GB/s']} "
                  f"| {p['us']} | {p['GB/s']} | {p['pct_peak']} |")
    print("\nOne step (layout, pack, permute, combine) replayed from one HIP graph, back to "
          "back (no host launch gaps), next to the sum of the per-call warm times:\n")
    print("| workload | us per step (graph) | with moe_dispatch (graph) | sum of per-call warm us |")
    print("|---|---|---|---|")
    for name, r in rows:
        wd = r.get("graph_whole_dispatch")
        wds = "" if wd is None else f"{wd['us_per_step']} ({wd['form']})"
        print(f"| {name} | {r['graph']['us_per_step']} | {wds} | {r['warm']['us']} |")
    print(f"\n1 GiB device copy: {copy['us']} us, {copy['GB/s']} GB/s (read + write)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--sets", type=int, default=3,
                    help="complete buffer sets the timed steps rotate through")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", nargs="?",
                    const="tiny,decode,prefill,skew,adv,prefill:align=128,decode:align=128,"
                          "decode:block=128,"
                          "prefill:mxfp8,decode:mxfp8,adv:mxfp8,prefill:mxfp4,decode:mxfp4,"
                          "adv:mxfp4,prefill:nvfp4,decode:nvfp4,adv:nvfp4",
                    default=None,
                    metavar="WORKLOADS", help="per-call warm/rotated/cold table over workloads")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (for counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs into profiles/traffic.json")
    ap.add_argument("--trace-passes", metavar="TRACE_CSV",
                    help="per-pass kernel durations from the rocprofv3 kernel trace of a bench "
                         "run with the same --steps, --warmup and --sets")
    args = ap.parse_args()
    if args.trace_passes:
        print(json.dumps(trace_passes(args.trace_passes, args.steps, args.warmup, args.sets),
                         indent=1))
        return
    if args.ingest_counters:
        rec = ingest_counters(*args.ingest_counters, args.copy_calibration or 512.0, args.workload)
        print(json.dumps(rec, indent=1, sort_keys=True))
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this path runs one GPU's share "
              "of an expert-parallel layer, with the R ranks as logical buffers in its own HBM; "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import __graft_entry__ as ge
    ge.ensure_built()
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.sweep:
        sweep(args.sweep.split(","), dev, not args.no_cpu_baseline)
        return
    w = synth.WORKLOADS[args.workload]

    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 2 ** 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 x {args.copy_calibration} MiB")

    rig = Rig(w, dev, sets=args.sets)
    step_bytes = path_bytes(rig.nbytes)
    stream = rig.stream

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        rig.step()
    torch.cuda.synchronize()

    def timed_steps(rotate: bool):
        """K whole steps bracketed by events on the stream the kernels run on
        (and a host clock around the synchronisations): ms per step, wall s."""
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        t_begin.record(stream)
        for _ in range(args.steps):
            rig.step(rotate=rotate)
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_begin.elapsed_time(t_end) / args.steps, time.perf_counter() - t0

    # The timed region: every step on the next of the rotating buffer sets.
    ms_per_step, wall = timed_steps(rotate=True)
    log(f"timed {args.steps} steps (buffer sets rotating): {ms_per_step * 1e3:.1f} us/step")
    # The same steps on one buffer set, back to back (its inputs partly cached
    # by the step before).
    warm_ms, _ = timed_steps(rotate=False)
    log(f"timed {args.steps} steps (one buffer set): {warm_ms * 1e3:.1f} us/step")

    # Per-call durations: events between the calls (rotating sets), and with a
    # 1 GiB read that evicts L2 and the Infinity Cache before every call.
    flush = torch.ones(2 ** 30, dtype=torch.uint8, device=dev)
    acc = torch.zeros((), dtype=torch.int32, device=dev)

    def evict() -> None:
        torch.sum(flush, dim=0, dtype=torch.int32, out=acc)

    # The rotated steps again, right after that 1 GiB write by another kernel
    # (a large write changes how the Infinity Cache keeps the pack's rows for
    # the permute; the step should not depend on it).
    torch.cuda.synchronize()
    after_write_ms, _ = timed_steps(rotate=True)
    log(f"timed {args.steps} steps after a 1 GiB write: {after_write_ms * 1e3:.1f} us/step")
    per_call_ms = rig.per_call_ms(args.steps)
    cold_ms = rig.per_call_ms(args.steps, evict, rotate=False)
    one_cold_ms = rig.per_call_ms(args.steps, evict, rotate=False, calls=("dispatch", "combine"))
    del flush
    rig.check_err()

    # The same step with layout, pack and permute through the one call
    # moe_dispatch (rotating sets): the same outputs from fewer bytes, since
    # the packed rows are not read back.
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for _ in range(args.steps):
        rig.rotate()
        rig.call("dispatch")
        rig.call("combine")
    t_end.record(stream)
    torch.cuda.synchronize()
    one_call_ms = t_begin.elapsed_time(t_end) / args.steps
    rig.check_err()
    one_call_bytes = rig.nbytes["dispatch"] + rig.nbytes["combine"]
    one_cold_step_ms = sum(float(np.mean(v)) for v in one_cold_ms.values())
    log(f"timed {args.steps} steps through moe_dispatch: {one_call_ms * 1e3:.1f} us/step")

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    call_stats = {}
    for c in CALLS:
        ms = float(np.mean(per_call_ms[c]))
        cms = float(np.mean(cold_ms[c]))
        call_stats[c] = {"us": round(ms * 1e3, 2),
                         "us_median": round(float(np.median(per_call_ms[c])) * 1e3, 2),
                         "bytes": rig.nbytes[c],
                         "GB/s": round(rig.nbytes[c] / (ms * 1e-3) / 1e9, 1),
                         "cold_us": round(cms * 1e3, 2)}
    cold_step_ms = sum(float(np.mean(cold_ms[c])) for c in CALLS)

    def mode(ms):
        gbs = step_bytes / (ms * 1e-3) / 1e9
        return {"us_per_step": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}

    modes = {"rotated": dict(mode(ms_per_step), note="the value: a different buffer set each "
                             "step, nothing read is cached from the step before"),
             "warm": dict(mode(warm_ms), note="one buffer set back to back"),
             "after_write": dict(mode(after_write_ms), note="the rotated steps right after a "
                                 "1 GiB write by another kernel"),
             "cold": dict(mode(cold_step_ms), note="sum of per-call means, L2 and Infinity "
                          "Cache evicted by a 1 GiB read before every call"),
             "one_call_dispatch": {
                 "us_per_step": round(one_call_ms * 1e3, 2), "bytes": one_call_bytes,
                 "GB/s": round(one_call_bytes / (one_call_ms * 1e-3) / 1e9, 1),
                 "note": "moe_dispatch (the layout, then pack and permute in one kernel) and "
                         "moe_combine, rotating buffer sets: the same outputs, the packed rows "
                         "not read back, so fewer algorithmic bytes (its own count)"},
             "one_call_dispatch_cold": {
                 "us_per_step": round(one_cold_step_ms * 1e3, 2), "bytes": one_call_bytes,
                 "GB/s": round(one_call_bytes / (one_cold_step_ms * 1e-3) / 1e9, 1),
                 "note": "the same two calls, L2 and Infinity Cache evicted by a 1 GiB read "
                         "before each (sum of per-call means)"}}
    # The dominant kernel's own duration: a third pass of whole steps (rotating
    # sets) in which the library records an event pair with the permute's
    # dispatch.
    dom = "permute"
    dom_us = float(np.mean(rig.kernel_ms(dom, args.steps))) * 1e3
    rig.check_err()
    achieved = rig.nbytes[dom] / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(dom, w.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": "permute_rows",
                "algorithmic_bytes_per_launch": rig.nbytes[dom],
                "kernel_us": round(dom_us, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(w, rig.hid, rig.ids, rig.wts, rig.y, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.describe(), "T": w.T, "H": w.H, "E": w.E, "R": w.R, "k": w.k,
                   "seed": w.seed, "copies_C": rig.C, "pairs_P": rig.P,
                   "copies_per_token": round(rig.C / max(w.T, 1), 4),
                   "bytes_per_step": step_bytes, "buffer_sets": args.sets},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "modes": modes,
        "imbalance": rig.imbalance(),
        "calls": call_stats,
        "rows_per_s": {
            "step_tokens": round(w.T / (ms_per_step * 1e-3)),
            "pack_copies": round(rig.C / (call_stats["pack"]["us"] * 1e-6)),
            "permute_pairs": round(rig.P / (call_stats["permute"]["us"] * 1e-6)),
            "combine_tokens": round(w.T / (call_stats["combine"]["us"] * 1e-6))},
        "wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
