#!/usr/bin/env python3
"""Throughput of the KDA spec-verify core on one MI355X (gfx950).

One step is one kda_verify call over the whole batch: for R x L rows and 12
heads it runs the conv update, the decay gate (MFMA), beta, l2norm, the gated
delta rule with a state written per token, and the gated RMSNorm. Inputs are
seeded synthetic tensors at the pages' shapes (12 heads x 128 channels per
tensor-parallel rank, f_a rank 128, width-4 conv), resident in HBM before the
timed region starts.

The headline workload is the large spec-verify batch: R = 64 requests x L = 8
tokens (S = 512 rows), a pool of 1024 slots addressed through a [64, 16] block
table, accepted counts ~ U{1..8}. Successive steps alternate between the two
8-column halves of the block table, so that a step's reads come from slots
written two steps earlier, with ~420 MB of other writes in between: the 256 MB
Infinity Cache cannot hold them, and the rate is the HBM rate.

Metric bytes per step (state + conv window, read once per request and written
once per token): (R + S) x H x 67,840 B, where a unit of 67,840 B is one
128 x 128 fp32 state tile plus one 3 x 384 bf16 conv window.

Prints one JSON line. Besides the headline it carries, under `configs`, every
one of the five workloads (tiny decode, decode 64, verify 16 x 4, verify 64 x 8,
decode 256): kernel time over back-to-back launches with slot sets rotating,
tokens/s, metric GB/s and fraction of the HBM peak, the same kernel against the
ceiling of its own access pattern (the fastest replay of its state traffic
with no arithmetic, include/kda_probe.h; for decode also a plain device copy of
the same bytes), and per-launch times. The pools of the three small workloads
fit the 256 MB Infinity Cache, so for them the line adds a flushed figure: each
launch timed alone after 1 GiB of other writes.

`--trace-only` runs only the headline's rotated timed launches (for
rocprofv3 kernel traces and counters); `--config N` picks the headline
workload; `--layer` / `--proj` time the projections around the core.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA verify tokens/s and achieved HBM GB/s (state+conv R/W) at R x L"
UNIT_BYTES = 128 * 128 * 4 + 3 * 128 * 3 * 2        # state tile + conv window of one head
HBM_PEAK_GBPS = 8000.0                                # MI355X published HBM3E bandwidth
MALL_BYTES = 256 << 20                                # MI355X Infinity Cache
KERNEL_NAME = "kda_core_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_core_traffic.json")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="headline workload 0..4 (default 3)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the oracle baseline (0 disables it)")
    ap.add_argument("--rounding", choices=("fused", "bf16_handoff"), default="fused",
                    help="core rounding mode (default fused)")
    ap.add_argument("--no-probe", action="store_true", help="skip the plain HBM probes")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table (headline only)")
    ap.add_argument("--trace-only", action="store_true",
                    help="run only the headline's warm-up and rotated timed launches (for "
                         "rocprofv3 traces): no per-launch, pattern, probe, table or CPU legs")
    ap.add_argument("--probe-only", action="store_true",
                    help="run only the plain HBM probes (counter calibration)")
    ap.add_argument("--graph", type=int, default=0, metavar="CHAIN",
                    help="capture CHAIN consecutive launches (rotating slot sets) in one HIP "
                         "graph and time graph replays (steps rounded up to whole replays)")
    ap.add_argument("--layer", action="store_true",
                    help="time in_proj -> core -> o_proj per step instead (eager and one HIP graph)")
    ap.add_argument("--proj", action="store_true",
                    help="time the in_proj / o_proj projections at the workload's row count "
                         "instead of the core (prints one JSON line)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="(CPU only) record the core kernel's HBM bytes per launch for WORKLOAD "
                         "from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE; each run also "
                         "timing the 1 GiB copy probe that calibrates the counters) into "
                         "profiles/kda_core_traffic.json with the current kernel source digest")
    return ap.parse_args()


def counter_means(csv_path, counter):
    """Mean value per dispatch of `counter` for the core kernel and the 1 GiB
    grid-stride copy probe, from a rocprofv3 counter-collection CSV."""
    import csv
    sums = {}
    for row in csv.DictReader(open(csv_path)):
        if row.get("Counter_Name") != counter:
            continue
        name = row.get("Kernel_Name", "")
        key = "core" if "kda_core_kernel" in name else "copy" if "probe_copy(" in name or \
            name.split("(")[0].endswith("probe_copy") else None
        if key is None:
            continue
        v = float(row["Counter_Value"])
        n, tot = sums.get(key, (0, 0.0))
        sums[key] = (n + 1, tot + v)
    if "core" not in sums or "copy" not in sums:
        raise SystemExit(f"{csv_path}: no {counter} rows for both the core kernel and probe_copy")
    return {k: (tot / n, n) for k, (n, tot) in sums.items()}


def record_traffic(workload, fetch_csv, write_csv):
    """HBM bytes a launch: each counter (KiB a dispatch) scaled by what it reads
    for the copy probe, which moves exactly 1 GiB each way."""
    f = counter_means(fetch_csv, "FETCH_SIZE")
    w = counter_means(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    fetch_scale = gib_kib / f["copy"][0]
    write_scale = gib_kib / w["copy"][0]
    read_bytes = f["core"][0] * fetch_scale * 1024
    write_bytes = w["core"][0] * write_scale * 1024
    rec = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    rec[workload] = {"source_digest": source_digest(), "fetch_size_kib": round(f["core"][0], 1),
                     "write_size_kib": round(w["core"][0], 1), "dispatches": [f["core"][1], w["core"][1]],
                     "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
                     "read_bytes": int(read_bytes), "write_bytes": int(write_bytes),
                     "bytes_per_launch": int(read_bytes + write_bytes)}
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps({workload: rec[workload]}))


def source_digest() -> str:
    import hashlib
    path = os.path.join(ROOT, "kimi_delta_attention_conv_amd", "csrc", "kda_core.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def rotation_sets(case, torch):
    """Disjoint slot sets of the pool, each laid out like case.slots.

    Returns (flat int32 base, [(shape, stride, offset)]): every set is a view of
    the base, so a block-table slice keeps its row stride on the device."""
    S, L = case.S, case.L
    if case.slots.dim() == 2 and case.slots.stride(0) > L:
        cols = case.slots.stride(0)
        base = torch.as_strided(case.slots, (case.R * cols,), (1,), case.slots.storage_offset())
        views = [((case.R, L), (cols, 1), j * L) for j in range(cols // L)]
        return base.contiguous(), views
    first = case.slots.reshape(-1)
    used = set(first.tolist())
    perm = torch.randperm(case.num_slots, generator=torch.Generator().manual_seed(77)).tolist()
    rest = [x for x in perm if x not in used]
    chunks = [first]
    while len(rest) >= S:
        chunks.append(torch.tensor(rest[:S], dtype=torch.int32))
        rest = rest[S:]
    shape, stride = tuple(case.slots.shape), tuple(case.slots.contiguous().stride())
    views = [(shape, stride, k * S) for k in range(len(chunks))]
    return torch.cat(chunks).contiguous(), views


class Workload:
    """One workload's inputs on the device, its core handle and its launches."""

    def __init__(self, torch, kda, index, rounding="fused"):
        from kda_inputs import make_config

        self.torch = torch
        self.case = case = make_config(index)
        dev = "cuda"
        self.conv_storage = case.conv_storage.to(dev)
        conv = self.conv_storage if case.conv_dim_first else self.conv_storage.transpose(-1, -2)
        self.state = case.state.to(dev)
        self.core = kda.KdaCore(conv_weight=case.conv_weight.to(dev),
                                conv_bias=None if case.conv_bias is None else case.conv_bias.to(dev),
                                f_b=case.f_b.to(dev), A_log=case.A_log.to(dev),
                                dt_bias=case.dt_bias.to(dev), norm_weight=case.norm_weight.to(dev),
                                gate_lower_bound=case.gate_lower_bound, norm_eps=case.norm_eps,
                                l2_eps=case.l2_eps, conv=conv, state=self.state, rounding=rounding)
        self.projected = case.projected.to(dev)
        self.out = torch.empty(case.S, case.D, dtype=torch.bfloat16, device=dev)
        base, views = rotation_sets(case, torch)
        self.slot_base = base.to(dev)
        self.sets = [torch.as_strided(self.slot_base, sh, st, off) for sh, st, off in views]
        self.accepted = None if case.accepted is None else case.accepted.to(dev)
        self.lib = kda.load_library()
        self.metric_bytes = (case.R + case.S) * case.H * UNIT_BYTES
        # bytes of the slots one launch touches: the MALL holds them when small
        self.pool_bytes = case.num_slots * case.H * UNIT_BYTES

    def make_launch(self, s, sp):
        lib, c, h = self.lib, self.case, self.core.handle
        proj, out = self.projected.data_ptr(), self.out.data_ptr()
        if self.accepted is None:
            return lambda: lib.kda_decode(h, proj, c.pitch, c.R, s.data_ptr(), out, sp)
        acc = self.accepted.data_ptr()
        return lambda: lib.kda_verify(h, proj, c.pitch, c.R, c.L, s.data_ptr(), s.stride(0), acc,
                                      out, sp)

    def launches(self, sp):
        return [self.make_launch(s, sp) for s in self.sets]

    def check_errors(self):
        n = self.core.device_errors()
        if n:
            raise RuntimeError(f"{self.case.name}: {n} requests were skipped for invalid slots")

    def close(self):
        self.core.close()


def events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_back_to_back(torch, fns, steps, warmup, stream):
    """Average ms of one call over `steps` back-to-back calls (rotating through
    `fns`), HIP events on the launch stream."""
    for i in range(warmup):
        if fns[i % len(fns)]() != 0:
            raise RuntimeError("launch failed")
    torch.cuda.synchronize()
    e0, e1 = events(torch)
    e0.record(stream)
    failed = sum(fns[(warmup + i) % len(fns)]() != 0 for i in range(steps))
    e1.record(stream)
    torch.cuda.synchronize()
    if failed:
        raise RuntimeError(f"{failed} launches failed")
    return e0.elapsed_time(e1) / steps


def time_each(torch, fns, n, stream, before=None):
    """Per-launch µs of `n` calls, each between its own pair of events, with
    `before()` (e.g. a cache flush) enqueued ahead of each pair."""
    pairs = []
    for i in range(n):
        if before is not None:
            before()
        a, b = events(torch)
        a.record(stream)
        if fns[i % len(fns)]() != 0:
            raise RuntimeError("launch failed")
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    q = lambda f: us[min(len(us) - 1, int(f * len(us)))]
    return {"p10": round(q(0.1), 2), "p50": round(statistics.median(us), 2),
            "p90": round(q(0.9), 2), "launches": n}


def pattern_ceiling(torch, w, steps, stream):
    """The workload's state traffic alone (kda_probe_state_stream over the same
    rotating slot sets) in each probe variant, and for in-place decode a device
    copy of the same bytes; the fastest is the ceiling of the access pattern."""
    from kimi_delta_attention_conv_amd import probe as kprobe
    plib = kprobe.load_probe_library()
    c = w.case
    sp = stream.cuda_stream
    stride = c.H * 128 * 128
    acc = None if w.accepted is None else w.accepted.data_ptr()
    res = {}
    names = {0: "free", kprobe.BARRIER: "barrier", kprobe.CORE_OCCUPANCY: "core_occupancy",
             kprobe.BARRIER | kprobe.CORE_OCCUPANCY: "barrier_core_occupancy"}
    for opt, name in names.items():
        fns = [lambda s=s, o=opt: plib.kda_probe_state_stream(
            w.state.data_ptr(), stride, c.num_slots, s.data_ptr(),
            s.stride(0) if s.dim() == 2 else 1, acc, c.R, c.L, c.H, o, sp) for s in w.sets]
        res[name] = round(time_back_to_back(torch, fns, steps, 10, stream), 5)
    state_bytes = (c.R + c.S) * c.H * 128 * 128 * 4
    if c.L == 1:
        # in-place decode moves R H tiles in and out: a plain device copy of as many bytes
        n = c.R * c.H * 128 * 128
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(0.5)
        b = torch.empty_like(a)
        res["device_copy"] = round(time_back_to_back(torch, [lambda: (b.copy_(a), 0)[1]],
                                                     steps, 10, stream), 5)
        del a, b
    best = min(res, key=res.get)
    return {"variants_ms": res, "best": best, "kernel_ms": res[best], "state_bytes": state_bytes,
            "gbps": round(state_bytes / (res[best] * 1e-3) / 1e9, 1)}


def flush_fn(torch):
    """1 GiB of plain writes through the probe library: evicts the Infinity Cache."""
    from kimi_delta_attention_conv_amd import probe as kprobe
    plib = kprobe.load_probe_library()
    buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream

    def fn():
        if plib.kda_probe_write_runs(buf.data_ptr(), 1 << 30, 0.25, sp) != 0:
            raise RuntimeError("flush failed")
    fn.buf = buf
    return fn


def workload_row(torch, kda, index, steps, warmup, rounding, flush):
    """Everything the line reports for one workload."""
    w = Workload(torch, kda, index, rounding)
    stream = torch.cuda.current_stream()
    fns = w.launches(stream.cuda_stream)
    c = w.case
    print(f"[bench] {c.name}: {steps} rotated launches", file=sys.stderr, flush=True)
    ms = time_back_to_back(torch, fns, steps, warmup, stream)
    w.check_errors()
    gbps = w.metric_bytes / (ms * 1e-3) / 1e9
    row = {"workload": c.name, "requests": c.R, "tokens": c.L, "rows": c.S, "heads": c.H,
           "kernel_ms": round(ms, 5), "tokens_per_s": round(c.S / (ms * 1e-3), 1),
           "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
           "metric_bytes_per_step": w.metric_bytes, "slot_sets_rotated": len(w.sets),
           "pool_bytes": w.pool_bytes, "steps": steps, "warmup": warmup}
    row["launch_us"] = time_each(torch, fns, 50, stream)
    if w.pool_bytes <= MALL_BYTES:
        row["cache_resident"] = True
        fl = time_each(torch, fns, 30, stream, before=flush)
        row["flushed_launch_us"] = fl
        row["flushed_gbps"] = round(w.metric_bytes / (fl["p50"] * 1e-6) / 1e9, 1)
        row["flushed_frac"] = round(row["flushed_gbps"] / HBM_PEAK_GBPS, 4)
    w.check_errors()
    pat = pattern_ceiling(torch, w, min(steps, 100), stream)
    row["pattern"] = pat
    row["frac_of_pattern"] = round(pat["kernel_ms"] / ms, 4)
    w.close()
    del w
    torch.cuda.empty_cache()
    return row


def probe(torch):
    """Achievable HBM GB/s of plain read, write and copy streams (1 GiB buffers)."""
    from kimi_delta_attention_conv_amd import probe as kprobe
    lib = kprobe.load_probe_library()
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    sink = torch.empty(lib.kda_probe_sink_floats(), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    calls = {
        "read": lambda: lib.kda_probe_read(a.data_ptr(), nbytes, sink.data_ptr(), s),
        "write": lambda: lib.kda_probe_write(b.data_ptr(), nbytes, 2.0, s),
        "copy": lambda: lib.kda_probe_copy(b.data_ptr(), a.data_ptr(), nbytes, s),
        "write_runs": lambda: lib.kda_probe_write_runs(b.data_ptr(), nbytes, 2.0, s),
        "copy_runs": lambda: lib.kda_probe_copy_runs(b.data_ptr(), a.data_ptr(), nbytes, s),
    }
    moved = {"read": nbytes, "write": nbytes, "copy": 2 * nbytes, "write_runs": nbytes,
             "copy_runs": 2 * nbytes}
    res = {}
    stream = torch.cuda.current_stream()
    for name, fn in calls.items():
        ms = time_back_to_back(torch, [fn], 10, 3, stream)
        res[name] = dict(gbps=round(moved[name] / (ms * 1e-3) / 1e9, 1), ms=round(ms, 4),
                         bytes=moved[name])
    del a, b, sink
    return res


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def bench_projections(args, torch, kda):
    """in_proj [S, 7168] x [4D+128+H, 7168]^T and o_proj [S, D] x [7168, D]^T on MFMA."""
    from kda_inputs import CONFIGS, HIDDEN, make_linear
    cfg = CONFIGS[args.config]
    S, H = cfg["R"] * cfg["L"], cfg["H"]
    D = 128 * H
    lib = kda.load_library()
    sp = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, (N, K) in (("in_proj", (4 * D + 128 + H, HIDDEN)), ("o_proj", (HIDDEN, D))):
        x, w = make_linear(S, N, K, seed=7)
        # several weight copies rotate so that the timed launches stream from HBM
        copies = max(1, -(-(600 << 20) // (N * K * 2)))
        xs = x.cuda()
        ws = [w.cuda() for _ in range(copies)]
        y = torch.empty(S, N, dtype=torch.bfloat16, device="cuda")
        ws_bytes = int(lib.kda_linear_workspace_bytes(S, N, K))
        work = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

        def launch(i):
            return lib.kda_linear(xs.data_ptr(), xs.stride(0), ws[i % copies].data_ptr(),
                                  y.data_ptr(), N, S, N, K, work.data_ptr(), ws_bytes, sp)
        fns = [lambda i=i: launch(i) for i in range(copies)]
        ms = time_back_to_back(torch, fns, args.steps, args.warmup, torch.cuda.current_stream())
        flops = 2.0 * S * N * K
        nbytes = (N * K + S * K + S * N) * 2
        tflops = flops / (ms * 1e-3) / 1e12
        gbps = nbytes / (ms * 1e-3) / 1e9
        t_mfma, t_hbm = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBPS * 1e9)
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        out[name] = {"M": S, "N": N, "K": K, "split_k": ws_bytes > 0, "us": round(ms * 1e3, 2),
                     "tflops": round(tflops, 1), "gbps": round(gbps, 1),
                     "roofline": {"bound": bound,
                                  "achieved": round(tflops if bound == "mfma" else gbps, 1),
                                  "peak": MFMA_BF16_PEAK_TFLOPS if bound == "mfma" else HBM_PEAK_GBPS,
                                  "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                                  "frac": round((t_mfma if bound == "mfma" else t_hbm) / (ms * 1e-3), 4)}}
        del ws, xs, y, work
        torch.cuda.empty_cache()
    return out


def bench_layer(args, torch, kda):
    """One layer's attention-core step as a serving loop runs it: in_proj
    (hidden 7168 -> packed row), the core (decode or verify), o_proj (D -> 7168).
    Weight copies and slot sets rotate so that every step streams from HBM: each
    weight has enough copies (at least 600 MiB of them) that a kernel timed
    alone does not find its weights in the 256 MB Infinity Cache either."""
    from kda_inputs import HIDDEN, make_linear
    w = Workload(torch, kda, args.config)
    case = w.case
    S, H, D, pitch = case.S, case.H, case.D, case.pitch
    n_in = 4 * D + 128 + H
    lib = w.lib
    dev = "cuda"
    x, w_in = make_linear(S, n_in, HIDDEN, seed=21)
    _, w_o = make_linear(1, HIDDEN, D, seed=22)
    in_copies = max(4, -(-(600 << 20) // (n_in * HIDDEN * 2)))
    o_copies = max(4, -(-(600 << 20) // (HIDDEN * D * 2)))
    xs = x.to(dev)
    w_ins = [w_in.to(dev) for _ in range(in_copies)]
    w_os = [w_o.to(dev) for _ in range(o_copies)]
    projected = w.projected
    core_out = w.out
    out = torch.empty(S, HIDDEN, dtype=torch.bfloat16, device=dev)
    # one workspace serves both projections (they run in stream order)
    ws_bytes = max(int(lib.kda_linear_workspace_bytes(S, n_in, HIDDEN)),
                   int(lib.kda_linear_workspace_bytes(S, HIDDEN, D)))
    work = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def parts(i, sp):
        w1, w2 = w_ins[i % in_copies], w_os[i % o_copies]
        return [
            lambda: lib.kda_in_proj(xs.data_ptr(), HIDDEN, w1.data_ptr(), projected.data_ptr(),
                                    pitch, S, HIDDEN, H, work.data_ptr(), ws_bytes, sp),
            w.make_launch(w.sets[i % len(w.sets)], sp),
            lambda: lib.kda_o_proj(core_out.data_ptr(), D, w2.data_ptr(), out.data_ptr(), HIDDEN,
                                   S, H, HIDDEN, work.data_ptr(), ws_bytes, sp),
        ]

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    steps, warm = args.steps, args.warmup
    for i in range(warm):
        for f in parts(i, sp):
            assert f() == 0
    torch.cuda.synchronize()
    e0, e1 = events(torch)
    e0.record(stream)
    for i in range(steps):
        for f in parts(i, sp):
            f()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) / steps * 1e3
    # each kernel alone (its own events), same rotation
    names = ("in_proj", "core", "o_proj")
    alone = {}
    for k, name in enumerate(names):
        a, b = events(torch)
        a.record(stream)
        for i in range(steps):
            parts(i, sp)[k]()
        b.record(stream)
        torch.cuda.synchronize()
        alone[name] = round(a.elapsed_time(b) / steps * 1e3, 2)
    # one HIP graph holding `copies` whole steps (every in_proj weight copy once)
    copies = in_copies
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        spc = torch.cuda.current_stream().cuda_stream
        for i in range(copies):
            for f in parts(i, spc):
                if f() != 0:
                    raise RuntimeError("capture failed")
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    g0, g1 = events(torch)
    g0.record(stream)
    for _ in range(reps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_us = g0.elapsed_time(g1) / (reps * copies) * 1e3
    w.check_errors()
    w.close()
    return {"workload": case.name, "rows": S, "heads": H, "hidden": HIDDEN,
            "eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
            "tokens_per_s_graph": round(S / (graph_us * 1e-6), 1),
            "kernel_us_alone": alone, "weight_copies_rotated": {"in_proj": in_copies, "o_proj": o_copies},
            "note": "synthetic weights; the core's inputs are in_proj's outputs"}


def cpu_baseline(case, seconds):
    """The oracle, as it stands, timed on the host on the same workload."""
    import numpy as np

    import oracle
    orc = oracle.default()

    def u16(t):
        return t.detach().contiguous().view(__import__("torch").int16).numpy().view(np.uint16)

    conv = u16(case.conv_storage).copy()
    state = case.state.numpy().copy()
    out = np.zeros((case.S, case.D), np.uint16)
    s = case.slots
    span = (s.shape[0] - 1) * s.stride(0) + s.shape[1] if s.dim() == 2 else s.numel()
    flat = __import__("torch").as_strided(s, (span,), (1,), s.storage_offset()).contiguous().numpy()
    kw = dict(heads=case.H, width=case.W, requests=case.R, tokens=case.L,
              projected=u16(case.projected), pitch=case.pitch, slots=flat,
              slots_row_stride=case.slots_row_stride(),
              accepted=None if case.accepted is None else case.accepted.numpy(),
              num_slots=case.num_slots, conv=conv.reshape(-1), conv_strides=case.conv_strides(),
              state=state.reshape(-1), state_slot_stride=case.H * 128 * 128,
              conv_weight=u16(case.conv_weight),
              conv_bias=None if case.conv_bias is None else u16(case.conv_bias),
              f_b=u16(case.f_b), A_log=case.A_log.numpy(), dt_bias=case.dt_bias.numpy(),
              norm_weight=case.norm_weight.numpy(), norm_head_stride=0,
              gate_lower_bound=case.gate_lower_bound, norm_eps=case.norm_eps,
              l2_eps=case.l2_eps, core_out=out)
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.run(**kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    single = case.S * reps / el

    # The same oracle on contiguous chunks of requests, one host thread a chunk:
    # requests touch disjoint slots, the oracle keeps no global state, and
    # ctypes releases the interpreter lock during each call.
    import threading
    threads = max(1, min(16, os.cpu_count() or 1, case.R))
    bounds = [case.R * i // threads for i in range(threads + 1)]
    ss = case.slots_row_stride()
    done = [0] * threads
    stop = time.perf_counter() + seconds

    def worker(i):
        r0, r1 = bounds[i], bounds[i + 1]
        if r1 == r0:
            return
        sub = dict(kw, requests=r1 - r0, projected=kw["projected"][r0 * case.L: r1 * case.L],
                   slots=flat[r0 * ss: (r1 - 1) * ss + case.L],
                   accepted=None if kw["accepted"] is None else kw["accepted"][r0:r1],
                   core_out=out[r0 * case.L: r1 * case.L])
        while time.perf_counter() < stop:
            orc.run(**sub)
            done[i] += (r1 - r0) * case.L
    t1 = time.perf_counter()
    pool = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    el2 = time.perf_counter() - t1
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=round(sum(done) / el2, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"the same workload ({case.R} requests x {case.L} tokens x {case.H} "
                       f"heads): {threads} host threads on request chunks for {el2:.1f} s, "
                       f"and {reps} single-threaded full calls in {el:.1f} s; C oracle in double",
                single_thread_value=round(single, 2), cpu_model=model,
                host_cpus=os.cpu_count())


def main():
    args = parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the library "
              "has no multi-GPU path: the core shards by heads and requests with no exchange, "
              "and each GPU's share is what one process measures)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kimi_delta_attention_conv_amd as kda
    from kda_inputs import make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.probe_only:
        print(json.dumps({"hbm_probe": probe(torch)}), flush=True)
        return
    if args.layer:
        print(json.dumps({"layer": bench_layer(args, torch, kda)}), flush=True)
        return
    if args.proj:
        print(json.dumps({"projections": bench_projections(args, torch, kda),
                          "workload_rows_of": make_config(args.config).name}), flush=True)
        return

    w = Workload(torch, kda, args.config, args.rounding)
    case = w.case
    stream = torch.cuda.current_stream()
    launches = w.launches(stream.cuda_stream)
    if args.graph:
        chain = args.graph
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            sp_cap = torch.cuda.current_stream().cuda_stream
            for i in range(chain):
                rc = w.make_launch(w.sets[i % len(w.sets)], sp_cap)()
                if rc != 0:
                    raise RuntimeError(f"capture failed: {kda.kda_status_string(rc)}")
        args.warmup = -(-args.warmup // chain)
        args.steps = -(-args.steps // chain)
        launches = [lambda: (graph.replay(), 0)[1]]
    torch.cuda.synchronize()

    for i in range(args.warmup):
        rc = launches[i % len(launches)]()
        if rc != 0:
            raise RuntimeError(f"launch failed: {kda.kda_status_string(rc)}")
    torch.cuda.synchronize()
    print(f"[bench] {case.name}: warmup {args.warmup} done, timing {args.steps} steps",
          file=sys.stderr, flush=True)

    e0, e1 = events(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    failed = sum(launches[(args.warmup + i) % len(launches)]() != 0 for i in range(args.steps))
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if failed:
        raise RuntimeError(f"{failed} timed launches failed")
    gpu_ms = e0.elapsed_time(e1)
    w.check_errors()

    per_replay = args.graph if args.graph else 1
    steps_run = args.steps * per_replay
    ms_per_step = wall * 1e3 / steps_run
    kernel_ms = gpu_ms / steps_run           # one launch of the core kernel per step
    achieved = w.metric_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(case.name)
        if rec and rec.get("source_digest") == source_digest():
            traffic = rec.get("bytes_per_launch")
    result = {
        "metric": METRIC,
        "value": round(case.S / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps_run,
        "warmup": args.warmup * per_replay,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": case.name, "requests": case.R, "tokens": case.L,
                   "rows": case.S, "heads": case.H, "head_dim": 128, "pool_slots": case.num_slots,
                   "conv_layout": "dim_first" if case.conv_dim_first else "transposed",
                   "slot_sets_rotated": len(w.sets), "io": "bf16", "state": "f32",
                   "rounding": args.rounding,
                   "launch": f"hip_graph x{args.graph}" if args.graph else "eager"},
        "gbps": round(w.metric_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "metric_bytes_per_step": w.metric_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": KERNEL_NAME,
                     "kernel_ms": round(kernel_ms, 5)},
    }
    if args.trace_only:
        w.close()
        print(json.dumps(result), flush=True)
        return
    if not args.graph:
        result["launch_us"] = time_each(torch, launches, 50, stream)
        pat = pattern_ceiling(torch, w, min(args.steps, 100), stream)
        result["roofline"]["pattern"] = pat
        result["roofline"]["frac_of_pattern"] = round(pat["kernel_ms"] / kernel_ms, 4)
    w.check_errors()
    w.close()
    del w
    torch.cuda.empty_cache()
    if not args.no_probe:
        print("[bench] HBM probes", file=sys.stderr, flush=True)
        pr = probe(torch)
        result["hbm_probe"] = pr
        best = {"read": pr["read"]["gbps"],
                "write": max(pr["write"]["gbps"], pr["write_runs"]["gbps"]),
                "copy": max(pr["copy"]["gbps"], pr["copy_runs"]["gbps"])}
        result["roofline"]["frac_of_probe"] = {k: round(achieved / v, 4) for k, v in best.items()}
        torch.cuda.empty_cache()
    if not args.no_configs and not args.graph:
        flush = flush_fn(torch)
        table = {}
        for index in range(5):
            row = workload_row(torch, kda, index, 100, 10, args.rounding, flush)
            table[row["workload"]] = row
        del flush
        torch.cuda.empty_cache()
        result["configs"] = table
    if args.cpu_seconds > 0:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
