"""Benchmark of the causal SLAY forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one causal forward (slay_attn_chunked_fwd: feature map fused into
the chunked contraction, segment states, prefix scan) over B1 H16 L16384,
d = dv = 64, R = 4 Gauss-Laguerre nodes x m = 64 features (F = 256), chunk
64, bf16 in / fp32 accumulate / bf16 out, on seeded synthetic inputs already
resident in HBM.  Prints one JSON line.  Beside the forward it times the
standalone feature map on the same q and k (HBM-bound), the causal forward of
B4 H8 L2048 (F = 96), the non-causal, variable-length, backward and
long-sequence forwards, one recurrent decode step for 256 sequences x 16
heads (HBM-bound on the fp32 state), and the fp64 CPU oracle on bounded
samples of the workloads.

Warm-up: the W requested steps run first; then, if they amounted to less than
SETTLE_MS of GPU time, more untimed steps run until that much has passed
(the shader clock and the timings settle only after ~15 ms of sustained
work).  The extra steps are reported as "settle_steps".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

WORKLOAD = "h16_l16k_bf16"
SMALL = "b4h8_l2k_bf16"
DECODE = "decode_256x16_f32"
LONG = "h8_l128k_d128_bf16"
SETTLE_MS = 200.0  # minimum GPU time of untimed work before each timed loop
KERNEL_SOURCES = ("slay_chunked_fused.hip", "slay_chunked_generic.hip", "slay_chunked_wide.hip", "slay_featmap.hip",
                  "slay_decode.hip", "slay_backward.hip", "slay_backward_fused.hip", "slay_device.hpp")
# the sources whose kernels each measured unit launches (a counter summary is
# current while their digest matches the one it records)
_FWD = ("slay_chunked_fused.hip", "slay_chunked_generic.hip", "slay_device.hpp")
UNIT_SOURCES = {
    "fused_fwd_h16_l16k_bf16": _FWD,
    "fused_fwd_b4h8_l2k_bf16": _FWD,
    "noncausal_h16_l16k_bf16": _FWD,
    "varlen_h16_8seqs_16k_bf16": _FWD,
    "featmap_h16_l16k_bf16": ("slay_featmap.hip", "slay_device.hpp"),
    "backward_h16_l16k_bf16": ("slay_backward_fused.hip", "slay_chunked_generic.hip", "slay_device.hpp"),
    "long_h8_l128k_d128_bf16": ("slay_chunked_wide.hip", "slay_featmap.hip", "slay_chunked_generic.hip",
                                "slay_device.hpp"),
    "decode_256x16_f32": ("slay_decode.hip", "slay_featmap.hip", "slay_device.hpp"),
}


def fwd_flops_per_token_head(w) -> int:
    """Algorithmic flops of the causal forward per (token, head).

    feature map of q and k: 2 sides x 2 projections (anchor, PRF) x F columns x d x 2 = 8 d F;
    inter-chunk: phi(q).S and the state update 2 x 2 F dv, phi(q).z and z update 3 F;
    intra-chunk (causal half of each C x C block): (C+1)(F + dv) + (C+1)/2.
    """
    F, d, dv, C = w.F, w.d, w.dv, w.chunk
    return 8 * d * F + 4 * F * dv + 3 * F + (C + 1) * (F + dv) + (C + 1) // 2


def noncausal_flops_per_token_head(w) -> int:
    """Non-causal forward with Lq = Lk: q and k feature maps (4dF each), the
    state phi(k) [v | 1]^T (2F(dv+1)) and the readout phi(q)^T [S | z] (2F(dv+1))."""
    return 8 * w.d * w.F + 4 * w.F * (w.dv + 1)


def bwd_flops_per_token_head(w) -> int:
    """Algorithmic flops of the causal backward per (token, head), each product once.

    feature maps of q and k (8dF) and their VJPs dxh = P^T w (8dF);
    F x (dv+1) products per token: the chunk states phi(k) v'^T, the readout
    phi(q) S', dphi(q) = S' g', the reverse state phi(q) g'^T, dphi(k) = U v'
    (5 x 2F(dv+1)) and dv = U^T phi(k) (2F dv);
    causal halves of the C x C blocks: A = phi(Q) phi(K)^T, D^T phi(Q) and
    D phi(K) ((C+1)F each), A V' and D = G' V'^T ((C+1)(dv+1) each), A^T G ((C+1)dv).
    """
    F, d, dv, C = w.F, w.d, w.dv, w.chunk
    return 16 * d * F + 10 * F * (dv + 1) + 2 * F * dv + 3 * (C + 1) * F + 2 * (C + 1) * (dv + 1) + (C + 1) * dv


def fwd_bytes_per_token_head(w) -> int:
    """Algorithmic HBM bytes of the fused causal forward: q, k, v read and o written once (bf16)."""
    return 2 * (2 * w.d + 2 * w.dv)


def featmap_bytes_per_row(w) -> int:
    return 2 * w.d + 2 * w.F  # bf16 row in, bf16 features out


def decode_bytes_per_head(w) -> int:
    # fp32 state S (F x dv) and z (F) read and written, q, k, v read and o written (fp32)
    return 4 * 2 * (w.F * w.dv + w.F) + 4 * (2 * w.d + 2 * w.dv)


def sources_digest(names=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "kernelized_linear_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kind: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"^sources_sha256_16:\s*(\w+)", txt, re.M)
    m_val = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_src or not m_val or m_src.group(1) != sources_digest(UNIT_SOURCES[kind]):
        return None
    return float(m_val.group(1))


TRAFFIC_UNITS = {
    # summary name: (bench --only part, kernel-name fragments with their dispatches per launch of the unit,
    # description); the counters of each unit come from runs of that part alone
    "fused_fwd_h16_l16k_bf16": ("fwd", (("pass1s", 1), ("scan4_kernel", 1), ("pass2s", 1)),
                                "one causal forward, B1 H16 L16384 bf16 (segment states + scan + main pass)"),
    "fused_fwd_b4h8_l2k_bf16": ("small", (("pass1s", 1), ("scan4_kernel", 1), ("pass2s", 1)),
                                "one causal forward, B4 H8 L2048 F = 96 bf16 (segment states + scan + main pass)"),
    "featmap_h16_l16k_bf16": ("featmap", (("featmap_kernel<unsigned short, unsigned short", 1),),
                              "one feature-map launch over 262144 bf16 rows, F = 256"),
    "noncausal_h16_l16k_bf16": ("noncausal", (("pass1s", 1), ("scan4_kernel", 1), ("ncout_kernel", 1)),
                                "one non-causal forward, B1 H16 Lq = Lk = 16384 bf16"),
    "varlen_h16_8seqs_16k_bf16": ("varlen", (("vl_setup", 1), ("pass1s", 1), ("vl_scan", 1), ("pass2s", 1)),
                                  "one variable-length forward, 16 heads x 8 sequences (16384 tokens) bf16"),
    "backward_h16_l16k_bf16": ("backward", (("pb_state", 1), ("scan4_kernel", 2), ("pb_g", 1), ("pb_dq", 1),
                                            ("pb_dk", 1), ("vjp_kernel", 1)),
                               "one causal backward, B1 H16 L16384 bf16"),
    "long_h8_l128k_d128_bf16": ("long", (("featmap_kernel<unsigned short, unsigned short", 1), ("wstate", 1),
                                         ("scan4_kernel", 1), ("wout", 1)),
                                "one causal forward, B1 H8 L131072 d=dv=128 F=512 bf16 (wide path)"),
    "decode_256x16_f32": ("decode", (("featmap_kernel<float, float", 1), ("stream_kernel", 1)),
                          "one decode step for 4096 heads (q/k feature map + state stream)"),
}
CALIB_KERNEL = "copyBuffer"  # the device-to-device copy of --calib-copy-mib MiB


def traffic_summary(fetch_dir: str, write_dir: str, calib_mib: int, command: str, part: str) -> None:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of `bench.py --only part` into
    profiles/traffic_*.txt for the units of that part."""
    import collections
    import csv
    import glob

    def per_kernel(d, counter):
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        per_disp = collections.defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            per_disp[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        by_name = collections.defaultdict(list)
        for did, v in per_disp.items():
            by_name[names[did]].append(v)
        return {n: sum(v) / len(v) for n, v in by_name.items()}

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    calib_kib = calib_mib * 1024.0

    def pick(table, frag):
        vals = [v for n, v in table.items() if frag in n]
        return max(vals) if vals else None

    f_scale = calib_kib / pick(fetch, CALIB_KERNEL)
    w_scale = calib_kib / pick(write, CALIB_KERNEL)
    for name, (unit_part, frags, desc) in TRAFFIC_UNITS.items():
        if unit_part != part:
            continue
        f_kib = sum((pick(fetch, fr) or 0.0) * k for fr, k in frags)
        w_kib = sum((pick(write, fr) or 0.0) * k for fr, k in frags)
        total = (f_kib * f_scale + w_kib * w_scale) * 1024.0
        lines = [f"# HBM traffic per launch: {name}", "", f"unit: {desc}", "",
                 "commands (from the repository root, on the machine with the GPU):", "",
                 f"    {command.replace('COUNTER', 'FETCH_SIZE')}",
                 f"    {command.replace('COUNTER', 'WRITE_SIZE')}",
                 f"    python bench.py --only {part} --traffic-summary <FETCH_SIZE dir> <WRITE_SIZE dir> "
                 f"--calib-copy-mib {calib_mib}", "",
                 f"calibration: a {calib_mib} MiB device copy reads FETCH_SIZE x{1 / f_scale:.3f} and WRITE_SIZE "
                 f"x{1 / w_scale:.3f} of its bytes; factors {f_scale:.3f} and {w_scale:.3f}", "",
                 "| kernel | dispatches per launch | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch |",
                 "|---|---|---|---|"]
        for fr, k in frags:
            lines.append(f"| {fr} | {k} | {pick(fetch, fr) or 0.0:.0f} | {pick(write, fr) or 0.0:.0f} |")
        lines += ["", f"hbm_bytes_per_launch: {total:.6e}",
                  f"sources ({', '.join(UNIT_SOURCES[name])}):",
                  f"sources_sha256_16: {sources_digest(UNIT_SOURCES[name])}"]
        with open(os.path.join(ROOT, "profiles", f"traffic_{name}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print(name, f"{total / 1e6:.1f} MB per launch")


COUNTER_UNITS = {
    # bench --only part: (summary name, kernel-name fragments, description)
    "fwd": ("fused_fwd_h16_l16k_bf16", ("pass1s", "scan4_kernel", "pass2s"),
            "causal forward, B1 H16 L16384 d=dv=64 F=256 bf16"),
    "small": ("fused_fwd_b4h8_l2k_bf16", ("pass1s", "scan4_kernel", "pass2s"),
              "causal forward, B4 H8 L2048 d=dv=64 F=96 bf16"),
    "featmap": ("featmap_h16_l16k_bf16", ("featmap_kernel",), "feature map of 262144 bf16 rows, F = 256"),
    "backward": ("backward_h16_l16k_bf16", ("pb_state", "scan4_kernel", "pb_g", "pb_dq", "pb_dk", "vjp"),
                 "causal backward, B1 H16 L16384 bf16"),
    "varlen": ("varlen_h16_8seqs_16k_bf16", ("vl_setup", "pass1s", "vl_scan", "pass2s"),
               "variable-length causal forward, 16 heads x 8 sequences (16384 tokens) bf16"),
    "long": ("long_h8_l128k_d128_bf16", ("featmap_kernel", "wstate", "scan4_kernel", "wout"),
             "causal forward, B1 H8 L131072 d=dv=128 F=512 bf16 (wide path)"),
    "noncausal": ("noncausal_h16_l16k_bf16", ("pass1s", "scan4_kernel", "ncout"),
                  "non-causal forward, B1 H16 L16384 bf16"),
    "decode": ("decode_256x16_f32", ("featmap_kernel", "stream_kernel"), "decode step, 4096 heads, fp32"),
}


def counter_summary(pmc_dir: str, command: str, part: str) -> None:
    """profiles/counters_<unit>.md from one rocprofv3 --pmc run (with --kernel-trace) of `bench.py --only part`:
    per kernel, the averages over its dispatches of MFMA and VALU busy (% of the kernel's time on all SIMDs),
    LDS utilisation, LDS bank-conflict cycles per active LDS instruction cycle and the bf16 MFMA work executed."""
    import collections
    import csv
    import glob

    name, frags, desc = COUNTER_UNITS[part]
    path = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)[0]
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    kname = {}
    for r in csv.DictReader(open(path)):
        vals[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        kname[r["Dispatch_Id"]] = r["Kernel_Name"]
    dur = {}
    tr = glob.glob(os.path.join(pmc_dir, "**", "*kernel_trace.csv"), recursive=True)
    if tr:
        for r in csv.DictReader(open(tr[0])):
            dur[r["Dispatch_Id"]] = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3  # us
    per = collections.defaultdict(list)
    for did, cv in vals.items():
        kn = kname[did]
        if any(f in kn for f in frags):
            per[kn].append((cv, dur.get(did)))
    lines = [f"# rocprofv3 counters: {name}", "", f"unit: {desc}", "",
             "command (from the repository root, on the machine with the GPU):", "", f"    {command}",
             f"    python bench.py --only {part} --counter-summary <dir>", "",
             "Per kernel, averages over its dispatches.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs for the "
             "kernel's time (rocprofv3's MfmaUtil); VALU busy = rocprofv3's VALUBusy (SQ_ACTIVE_INST_VALU per CU "
             "over the kernel's time); LDS util = LdsUtil; LDS conflict ratio = SQ_LDS_BANK_CONFLICT / "
             "SQ_ACTIVE_INST_LDS (bank-conflict stall cycles per cycle of active LDS instructions); MFMA-VALU "
             "co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; bf16 MFMA work = "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops, executed (recomputation included), and its rate over "
             "the dispatch's traced duration (the counters serialise dispatches, so durations here run longer "
             "than in the timing runs).", "",
             "| kernel | dispatches | MFMA busy % | VALU busy % | LDS util % | LDS conflict ratio | MFMA-VALU co-issue |"
             " bf16 MFMA GFLOP / dispatch | executed TFLOP/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for kn, rows in sorted(per.items(), key=lambda kv: -len(kv[1])):
        n = len(rows)
        avg = lambda c: sum(r[0].get(c, 0.0) for r in rows) / n  # noqa: E731
        lds_act = avg("SQ_ACTIVE_INST_LDS")
        busy = avg("SQ_VALU_MFMA_BUSY_CYCLES")
        gflop = avg("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / 1e9
        ds = [r[1] for r in rows if r[1]]
        rate = gflop / (sum(ds) / len(ds)) * 1e3 if ds else float("nan")  # GFLOP per us -> TFLOP/s
        lines.append(f"| {kn[:70]} | {n} | {avg('MfmaUtil'):.1f} | {avg('VALUBusy'):.1f} | {avg('LdsUtil'):.1f} | "
                     f"{(avg('SQ_LDS_BANK_CONFLICT') / lds_act) if lds_act else 0.0:.2f} | "
                     f"{(avg('SQ_VALU_MFMA_COEXEC_CYCLES') / busy) if busy else 0.0:.2f} | {gflop:.2f} | "
                     f"{rate:.0f} |")
    lines += ["", f"sources ({', '.join(UNIT_SOURCES[name])}):",
              f"sources_sha256_16: {sources_digest(UNIT_SOURCES[name])}"]
    with open(os.path.join(ROOT, "profiles", f"counters_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_summary(trace_dir: str, command: str, part: str) -> None:
    """profiles/<unit>.md from one rocprofv3 --kernel-trace --stats run of `bench.py --only part` with as many
    warm-up steps as timed ones and no settle steps: per kernel, the average duration over all its dispatches
    and over the later half (the timed calls)."""
    import collections
    import csv
    import glob

    name, frags, desc = COUNTER_UNITS[part]
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if any(f in r["Kernel_Name"] for f in frags):
            per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
    lines = [f"# rocprofv3 kernel statistics: {name}", "", f"workload: {desc}", "",
             "command (from the repository root, on the machine with the GPU):", "", f"    {command}",
             f"    python bench.py --only {part} --stats-summary <dir>", "",
             "bench.py runs as many warm-up calls as timed ones here (it scales both per part) and no settle "
             "steps, so the later half of each kernel's dispatches are the timed calls. `average` is over every "
             "call, `timed average` over the timed calls only.", "",
             "| kernel | calls | average (us) | timed average (us) | min (us) | max (us) |", "|---|---|---|---|---|---|"]
    total = 0.0
    rows = []
    for kn, ds in per.items():
        ds.sort()
        d = [x[1] for x in ds]
        timed = d[len(d) // 2:]
        rows.append((sum(timed) / len(timed), kn, len(d), sum(d) / len(d), min(d), max(d)))
    n_units = None
    for ta, kn, n, avg, mn, mx in sorted(rows, reverse=True):
        short = re.sub(r"slay::\(anonymous namespace\)::", "", kn)
        short = re.sub(r"^void ", "", short)
        short = re.sub(r"\(.*\)$", "", short)
        lines.append(f"| {short[:80]} | {n} | {avg:.2f} | {ta:.2f} | {mn:.2f} | {mx:.2f} |")
        total += ta * n
        n_units = n if n_units is None else min(n_units, n)
    if n_units:
        lines += ["", f"sum of the timed averages per launch of the unit: {total / n_units:.1f} us"]
    lines += ["", f"sources ({', '.join(UNIT_SOURCES[name])}):",
              f"sources_sha256_16: {sources_digest(UNIT_SOURCES[name])}"]
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def event_time_ms(fn, steps: int, stream) -> float:
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def warm_up(fn, steps: int, stream) -> int:
    """Run `steps` untimed calls, then more until at least SETTLE_MS of GPU time
    has passed in this warm-up; returns the number of extra calls."""
    import torch

    settle_ms = SETTLE_MS  # set from --settle-ms

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    spent = start.elapsed_time(end) if steps > 0 else 0.0
    extra = 0
    while spent < settle_ms:
        n = 8 if extra == 0 else extra  # doubling batches
        start.record(stream)
        for _ in range(n):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        spent += start.elapsed_time(end)
        extra += n
    return extra


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Threads the oracle's OpenMP loops use (its own report)."""
    import oracle

    return int(oracle.max_threads())


def cpu_baseline(w, q, k, v, A, G, L_sample: int):
    import oracle

    oracle.build(force=False)
    qs, ks, vs = (x[:, :, :L_sample] for x in (q, k, v))
    t0 = time.perf_counter()
    oracle.slay_causal(qs, ks, vs, A, G, w.eps, w.R, w.m, form="recurrent")
    dt = time.perf_counter() - t0
    return {"value": w.B * L_sample / dt, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"fp64 recurrent form, all {w.B * w.H} heads x first {L_sample} of {w.L} tokens "
                      f"({dt:.2f} s wall); per-token cost is independent of L",
            "cpu_model": cpu_model()}


def cpu_baselines_other():
    """The oracle on bounded samples of the other workloads (reported beside the headline one)."""
    import oracle

    import slay_synth as ss

    out = []
    w2 = ss.WORKLOADS[SMALL]
    q, k, v = ss.make_qkv(w2)
    A, G = ss.make_draws(w2)
    t0 = time.perf_counter()
    oracle.slay_causal(q, k, v, A, G, w2.eps, w2.R, w2.m, form="recurrent")
    dt = time.perf_counter() - t0
    out.append({"workload": SMALL, "value": w2.B * w2.L / dt, "unit": "tokens/s", "wall_s": dt,
                "sample": "the whole workload (B4 H8 L2048, F = 96), fp64 recurrent form"})
    wl = ss.WORKLOADS[LONG]
    Ls = 2048
    q, k, v = ss.make_qkv(wl.with_(L=Ls))
    A, G = ss.make_draws(wl)
    t0 = time.perf_counter()
    oracle.slay_causal(q, k, v, A, G, wl.eps, wl.R, wl.m, form="recurrent")
    dt = time.perf_counter() - t0
    out.append({"workload": LONG, "value": wl.B * Ls / dt, "unit": "tokens/s", "wall_s": dt,
                "sample": f"all {wl.H} heads x first {Ls} of {wl.L} tokens (d = dv = 128, F = 512), fp64 recurrent "
                          "form; per-token cost is independent of L"})
    wd = ss.WORKLOADS[DECODE]
    n_steps = 16
    qs, ks, vs = zip(*(ss.make_decode_step(wd, t) for t in range(n_steps)))
    qd, kd, vd = (np.stack(x, 1) for x in (qs, ks, vs))  # [heads, steps, d]
    A, G = ss.make_draws(wd)
    t0 = time.perf_counter()
    oracle.slay_causal(qd, kd, vd, A, G, wd.eps, wd.R, wd.m, form="recurrent")
    dt = time.perf_counter() - t0
    out.append({"workload": DECODE, "value": wd.B * n_steps / dt, "unit": "tokens/s", "wall_s": dt,
                "sample": f"{n_steps} decode steps of all {wd.n_heads} heads (256 sequences x 16), fp64 recurrent "
                          "form (the state carried in memory as the GPU does)"})
    return out


def main():
    global SETTLE_MS
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # timings settle only after ~100 forwards (~15 ms of GPU work): the
    # default warm-up covers that; fewer warm-up steps measure a cold GPU
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--cpu-tokens", type=int, default=16384, help="tokens per head of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--only", choices=["all", "fwd", "small", "featmap", "noncausal", "varlen", "backward", "long",
                                       "decode"],
                    default="all")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run 3 plain device copies of this many MiB (scale for HBM byte counters)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_*.txt from two rocprofv3 --pmc runs and exit (no GPU)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="minimum GPU time of untimed work before each timed loop (0: only the warm-up steps)")
    ap.add_argument("--counter-summary", metavar="PMC_DIR",
                    help="write profiles/counters_*.md from one rocprofv3 --pmc run of this part and exit (no GPU)")
    ap.add_argument("--counter-command", default="rocprofv3 --pmc " + " ".join(
        ["MfmaUtil", "VALUBusy", "LdsUtil", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
         "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_COEXEC_CYCLES"]) +
        " --kernel-trace --output-format csv -d <dir> -o run -- python3 bench.py --only PART --steps 5 --warmup 1 "
        "--settle-ms 0 --decode-steps 32 --no-cpu")
    ap.add_argument("--traffic-command", default="rocprofv3 --pmc COUNTER --output-format csv -d <dir> -o run -- "
                    "python3 bench.py --only PART --steps 5 --warmup 1 --settle-ms 0 --decode-steps 32 --no-cpu "
                    "--calib-copy-mib 512")
    ap.add_argument("--stats-summary", metavar="TRACE_DIR",
                    help="write profiles/<unit>.md from one rocprofv3 --kernel-trace --stats run of this part and exit")
    ap.add_argument("--stats-command", default="rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                    "python3 bench.py --only PART --steps 100 --warmup 100 --settle-ms 0 --decode-steps 64 --no-cpu")
    args = ap.parse_args()
    SETTLE_MS = args.settle_ms
    if args.counter_summary:
        counter_summary(args.counter_summary, args.counter_command.replace("PART", args.only), args.only)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary, args.stats_command.replace("PART", args.only), args.only)
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.calib_copy_mib or 512,
                        args.traffic_command.replace("PART", args.only), args.only)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import slay_synth as ss
    from kernelized_linear_attention_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = ss.WORKLOADS[WORKLOAD]
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)

    def dev_bf16(a):
        return torch.from_numpy(a).to(dev).to(torch.bfloat16)

    fm = ops.FeatureMap(dev_bf16(A), dev_bf16(G), w.R, w.m, w.eps)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out = torch.empty_like(vd)
    ws_bytes = ops.chunked_fwd_workspace_size(fm, w.B, w.H, w.L, w.dv, w.chunk, torch.bfloat16)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def fwd():
        ops.chunked_fwd(fm, qd, kd, vd, w.chunk, out=out, workspace=ws)

    result = {}
    settle = {}
    if args.only in ("all", "fwd"):
        settle["fwd"] = warm_up(fwd, args.warmup, stream)
        t0 = time.perf_counter()
        ms = event_time_ms(fwd, args.steps, stream)
        wall = (time.perf_counter() - t0) / args.steps * 1e3
        flops = fwd_flops_per_token_head(w) * w.B * w.H * w.L
        achieved = flops / (ms * 1e-3) / 1e12
        result = {
            "metric": "SLAY causal fwd tokens/s at L=16k,H=16 on 1 GPU; % bf16 MFMA peak",
            "value": w.B * w.L / (ms * 1e-3),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": WORKLOAD, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "dv": w.dv, "R": w.R,
                       "m": w.m, "F": w.F, "chunk": w.chunk, "eps": w.eps, "parallelism": "single GPU"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_BF16_TFLOPS, "traffic": read_traffic("fused_fwd_h16_l16k_bf16"),
                         "kernel": "fused causal forward: segment-state pass + prefix scan + main pass, one stream",
                         "algorithmic_flops_per_launch": flops},
            "wall_ms_per_step": wall,
            "settle_steps": settle["fwd"],
        }
    also = []
    if args.only in ("all", "small"):
        # B4 H8 L2048, F = 96 (R = 3, m = 32), chunk 64: the fused kernels at a small feature count
        w2 = ss.WORKLOADS[SMALL]
        q2, k2, v2 = ss.make_qkv(w2)
        A2, G2 = ss.make_draws(w2)
        fm2 = ops.FeatureMap(dev_bf16(A2), dev_bf16(G2), w2.R, w2.m, w2.eps)
        q2d, k2d, v2d = dev_bf16(q2), dev_bf16(k2), dev_bf16(v2)
        o2 = torch.empty_like(v2d)
        ws2 = torch.empty(max(ops.chunked_fwd_workspace_size(fm2, w2.B, w2.H, w2.L, w2.dv, w2.chunk, torch.bfloat16),
                              16), dtype=torch.uint8, device=dev)

        def sfwd():
            ops.chunked_fwd(fm2, q2d, k2d, v2d, w2.chunk, out=o2, workspace=ws2)

        settle["small"] = warm_up(sfwd, args.warmup, stream)
        ms = event_time_ms(sfwd, args.steps, stream)
        nbytes = fwd_bytes_per_token_head(w2) * w2.B * w2.H * w2.L
        flops = fwd_flops_per_token_head(w2) * w2.B * w2.H * w2.L
        gbs = nbytes / (ms * 1e-3) / 1e9
        also.append({"name": "fwd_b4h8_l2k_bf16", "ms_per_step": ms, "tokens_per_s": w2.B * w2.L / (ms * 1e-3),
                     "config": {"B": w2.B, "H": w2.H, "L": w2.L, "d": w2.d, "dv": w2.dv, "R": w2.R, "m": w2.m,
                                "F": w2.F, "chunk": w2.chunk},
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": gbs / PEAK_HBM_GBS, "traffic": read_traffic("fused_fwd_b4h8_l2k_bf16"),
                                  "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                                  "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}})
        del q2d, k2d, v2d, o2, ws2
    if args.only in ("all", "featmap"):
        phi = torch.empty(w.B, w.H, w.L, w.F, dtype=torch.bfloat16, device=dev)

        def fmap():  # phi(q) then phi(k): two launches on the same stream
            for x in (qd, kd):
                ops.featmap(fm, x, torch.bfloat16, out=phi)

        settle["featmap"] = warm_up(fmap, args.warmup, stream)
        ms = event_time_ms(fmap, args.steps, stream) / 2  # per launch
        rows = w.B * w.H * w.L
        nbytes = rows * featmap_bytes_per_row(w)
        gbs = nbytes / (ms * 1e-3) / 1e9
        also.append({"name": "featmap_h16_l16k_bf16", "ms_per_launch": ms, "rows_per_launch": rows,
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": gbs / PEAK_HBM_GBS, "traffic": read_traffic("featmap_h16_l16k_bf16"),
                                  "algorithmic_bytes_per_launch": nbytes}})
    if args.only in ("all", "noncausal"):
        wsn = torch.empty(max(ops.noncausal_fwd_workspace_size(fm, w.B, w.H, w.L, w.L, w.dv, torch.bfloat16), 16),
                          dtype=torch.uint8, device=dev)

        def nc():
            ops.noncausal_fwd(fm, qd, kd, vd, out=out, workspace=wsn)

        settle["noncausal"] = warm_up(nc, args.warmup, stream)
        ms = event_time_ms(nc, args.steps, stream)
        flops = noncausal_flops_per_token_head(w) * w.B * w.H * w.L
        achieved = flops / (ms * 1e-3) / 1e12
        also.append({"name": "noncausal_h16_l16k_bf16", "ms_per_step": ms, "tokens_per_s": w.B * w.L / (ms * 1e-3),
                     "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                                  "traffic": read_traffic("noncausal_h16_l16k_bf16"),
                                  "algorithmic_flops_per_launch": flops}})
    if args.only in ("all", "varlen"):
        # eight sequences of mixed lengths packed per head (16384 tokens per head, 16 heads)
        lengths = [6144, 4096, 2048, 2048, 1024, 512, 256, 256]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device=dev)
        T = int(sum(lengths))
        qv, kv, vv = (x.reshape(w.H, T, -1) for x in (qd, kd, vd))  # the same values, read as a packed batch
        ov = torch.empty_like(vv)
        wsv = torch.empty(max(ops.varlen_fwd_workspace_size(fm, len(lengths), w.H, T, w.dv, torch.bfloat16), 16),
                          dtype=torch.uint8, device=dev)

        def vl():
            ops.varlen_fwd(fm, qv, kv, vv, cu, out=ov, workspace=wsv)

        settle["varlen"] = warm_up(vl, args.warmup, stream)
        ms = event_time_ms(vl, args.steps, stream)
        flops = fwd_flops_per_token_head(w) * w.H * T
        achieved = flops / (ms * 1e-3) / 1e12
        also.append({"name": "varlen_h16_8seqs_16k_bf16", "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
                     "lengths": lengths,
                     "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                                  "traffic": read_traffic("varlen_h16_8seqs_16k_bf16"),
                                  "algorithmic_flops_per_launch": flops}})
    if args.only in ("all", "backward"):
        dout = dev_bf16(ss.make_grads(w)[0])
        dq, dk, dvv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        wsb = torch.empty(max(ops.chunked_bwd_workspace_size(fm, w.B, w.H, w.L, w.dv, w.chunk, torch.bfloat16), 16),
                          dtype=torch.uint8, device=dev)

        def bwd():
            ops.chunked_bwd(fm, qd, kd, vd, dout, w.chunk, workspace=wsb, dq=dq, dk=dk, dv=dvv)

        settle["backward"] = warm_up(bwd, max(1, args.warmup // 5), stream)
        ms = event_time_ms(bwd, max(1, args.steps // 5), stream)
        flops = bwd_flops_per_token_head(w) * w.B * w.H * w.L
        achieved = flops / (ms * 1e-3) / 1e12
        also.append({"name": "backward_h16_l16k_bf16", "ms_per_step": ms, "tokens_per_s": w.B * w.L / (ms * 1e-3),
                     "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                                  "traffic": read_traffic("backward_h16_l16k_bf16"),
                                  "algorithmic_flops_per_launch": flops}})
        del wsb
    if args.only in ("all", "long"):
        # B1 H8 L131072, d = dv = 128, F = 512: feature maps in HBM, state on chip
        wl = ss.WORKLOADS[LONG]
        ql, kl, vl_ = ss.make_qkv(wl)
        Al, Gl = ss.make_draws(wl)
        fml = ops.FeatureMap(dev_bf16(Al), dev_bf16(Gl), wl.R, wl.m, wl.eps)
        qld, kld, vld = dev_bf16(ql), dev_bf16(kl), dev_bf16(vl_)
        del ql, kl, vl_
        oll = torch.empty_like(vld)
        wsl = torch.empty(max(ops.chunked_fwd_workspace_size(fml, wl.B, wl.H, wl.L, wl.dv, wl.chunk, torch.bfloat16),
                              16), dtype=torch.uint8, device=dev)

        def lfwd():
            ops.chunked_fwd(fml, qld, kld, vld, wl.chunk, out=oll, workspace=wsl)

        settle["long"] = warm_up(lfwd, max(1, args.warmup // 2), stream)
        ms = event_time_ms(lfwd, max(1, args.steps // 2), stream)
        flops = fwd_flops_per_token_head(wl) * wl.B * wl.H * wl.L
        achieved = flops / (ms * 1e-3) / 1e12
        also.append({"name": "long_h8_l128k_d128_bf16", "ms_per_step": ms,
                     "tokens_per_s": wl.B * wl.L / (ms * 1e-3),
                     "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                                  "traffic": read_traffic("long_h8_l128k_d128_bf16"),
                                  "algorithmic_flops_per_launch": flops}})
        del qld, kld, vld, oll, wsl
    if args.only in ("all", "decode"):
        wd = ss.WORKLOADS[DECODE]
        nh = wd.n_heads
        Ad, Gd = ss.make_draws(wd)
        fmd = ops.FeatureMap(torch.from_numpy(Ad).to(dev), torch.from_numpy(Gd).to(dev), wd.R, wd.m, wd.eps)
        n_in = 32
        steps_in = [ss.make_decode_step(wd, t) for t in range(n_in)]
        qs = torch.from_numpy(np.stack([s[0] for s in steps_in])).to(dev)
        ks_ = torch.from_numpy(np.stack([s[1] for s in steps_in])).to(dev)
        vs = torch.from_numpy(np.stack([s[2] for s in steps_in])).to(dev)
        S = torch.zeros(nh, wd.F, wd.dv, device=dev)
        z = torch.zeros(nh, wd.F, device=dev)
        o = torch.empty(nh, wd.dv, device=dev)
        wsd = torch.empty(ops.recurrent_step_workspace_size(fmd, nh, wd.dv, torch.float32), dtype=torch.uint8,
                          device=dev)
        # n_in consecutive steps (two launches each: feature map of all heads,
        # streaming state update) captured once as a HIP graph and replayed, so
        # host-side launch cost does not starve the GPU between short steps
        def steps():
            for t in range(n_in):
                ops.recurrent_step(fmd, qs[t], ks_[t], vs[t], S, z, out=o, workspace=wsd)

        steps()  # warm-up, eager
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            steps()
        reps = max(1, args.decode_steps // n_in)
        settle["decode"] = n_in * warm_up(graph.replay, max(1, args.warmup // n_in), stream)
        ms = event_time_ms(graph.replay, reps, stream) / n_in
        nbytes = nh * decode_bytes_per_head(wd)
        gbs = nbytes / (ms * 1e-3) / 1e9
        also.append({"name": "decode_256x16_f32", "ms_per_step": ms, "tokens_per_s": wd.B / (ms * 1e-3),
                     "heads": nh, "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                               "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                               "traffic": read_traffic("decode_256x16_f32"),
                                               "algorithmic_bytes_per_launch": nbytes}})
    if also:
        result["also"] = also
    if args.only in ("all", "fwd") and not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, A, G, min(args.cpu_tokens, w.L))
        if args.only == "all":
            result["cpu_baseline_other"] = cpu_baselines_other()
    result["settle_steps"] = settle
    result["sources_sha256_16"] = sources_digest()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
