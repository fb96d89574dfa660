"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  `value` is prefill throughput in tokens/s on the one-layer K3 KDA prefill
(B=1, T=4096, H=96, dk=dv=128, bf16 inputs, float32 state, 16-token tiles), inputs resident in HBM
before the timed region.  A `decode` object reports the batched single-token decode step
(256 sequences, H=96, float32 states read and written in place) the same way, and a `snapshots`
object the prefill that also saves the state every 64 tokens (kda_chunk_fwd_snapshots; 64 KiB per
head and snapshot, the stride at which saved states cost as much as the per-token cache they
replace).  An `output_gate` object times the output stage (per-head RMSNorm times a sigmoid
gate; 3 x 256 B per (token, head) in bf16) on the same [4096, 96, 128] shape, and
`decode.gated` the decode step with that stage fused; `decode.layer` the whole mixer's decode
step in one launch (input stage, decode, output stage: kda_decode_step_layer) on the same batch;
`decode.serving_graph` that step for 4 sequences, as three launches and as one, each eager and as
a captured HIP graph replayed per token.  A `frontend` object times the input stage
(short convolution, Swish, L2 norm, sigmoid beta, bounded log-decay: reads 3 dk + dv values and
beta's logit, writes as many per (token, head)) on the same token and head count.  A `varlen`
object times the prefill on the variable-length batch (16 sequences of 1,024-16,384 tokens with
initial states, packed with cu_seqlens); `varlen.gated` the prefill with the output stage fused
(kda_chunk_fwd_gated) against the prefill and the output-stage kernel, and `varlen.layer` the
whole token mixer (the input stage, then the gated prefill) against three separate passes.  A
`long` object times the long-context prefill (one sequence of 131,072 tokens, H=96: the same work
per token over a 32 times longer chain of tiles).  A `head_share` object times one GPU's share of
the heads under 8-way head sharding (12 of 96 heads, T = 4096, batch 1) with kda_chunk_fwd and with
kda_chunk_fwd_split (each sequence also cut into token ranges that run concurrently).

Roofline: algorithmic bytes per launch divided by the kernel's average duration, measured with
HIP events recorded on the stream the kernels are launched on, against MI355X's 8 TB/s HBM.
  prefill bytes / (token, head) = q, k, g (3 x 256) + v (256) + o (256) + beta (2) = 1282 B,
                                  plus 64 KiB per (sequence, head) for each of h0 (when given)
                                  and hT;
  prefill flops / (token, head) = 6 dk dv + d (5C - 1) = 108,416 at d = 128, C = 16;
  decode bytes / (sequence, head) = 2 x 65,536 (state in and out) + 4 x 256 (q, k, v, g)
                                    + 256 (o) + 2 (beta) = 132,354 B.
`cpu_baseline` times the float64 CPU oracle on the host cores on a bounded sample of the same
workload (rank 0, N = 1).  `traffic` is the HBM traffic per launch from rocprofv3 FETCH_SIZE +
WRITE_SIZE counters recorded in profiles/, used only while the kernel sources are unchanged.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6   # MI355X dense bf16 matrix peak (256 CU x 4096 flop/clk x 2.4 GHz)
CHUNK = 16

PREFILL_WORKLOADS = ("prefill_T4096_H96_d128_bf16", "varlen_16seq_H96_d128_bf16",
                     "long_T131072_H96_d128_bf16", "tiny_T64_H2_d32_f32")
DECODE_WORKLOAD = "decode_N256_H96_d128_bf16"
VARLEN_WORKLOAD = "varlen_16seq_H96_d128_bf16"
LONG_WORKLOAD = "long_T131072_H96_d128_bf16"


def _esize(dtype):
    return 2 if dtype == "bf16" else 4


def prefill_bytes(x) -> int:
    es = _esize(x.dtype)
    per_tok_head = (3 * x.dk + 2 * x.dv) * es + es
    state = x.dk * x.dv * 4
    n_states = x.num_seqs * x.H * (2 if x.h0 is not None else 1)
    return x.total_tokens * x.H * per_tok_head + n_states * state


def prefill_flops(x) -> int:
    d = x.dk
    return x.total_tokens * x.H * (6 * x.dk * x.dv + d * (5 * CHUNK - 1))


def decode_layer_bytes(N, H) -> int:
    """kda_decode_step_layer (dk = dv = 128, bf16): per (sequence, head) the state in and out, the
    pre-activations, the saved inputs in and out, gate and y; the taps, bias, A and gain once."""
    per_unit = 2 * 128 * 128 * 4 + (3 * 128 + 128) * 2 + 2 + 2 * 3 * 384 * 2 + 2 * 128 * 2
    return N * H * per_unit + H * (384 * 16 + 128 * 4 + 4) + 128 * 4


def decode_bytes(d) -> int:
    es = _esize(d.dtype)
    per = 2 * d.dk * d.dv * 4 + (3 * d.dk + 2 * d.dv) * es + es
    return d.B * d.H * per


# The sources that make each measured kernel's code: its own file, the shared device helpers and
# the build script (which holds the code-generation options).
KERNEL_SOURCES = {
    "kda_chunk_fwd": "kda_prefill_mfma.hip",
    "kda_chunk_fwd_split": ("kda_prefill_mfma.hip", "kda_prefill_split.hip"),
    "kda_chunk_fwd_chunk64": "kda_prefill_c64_mfma.hip",
    "kda_decode": "kda_decode.hip",
    "kda_output_gate": "kda_output_gate.hip",
    "kda_frontend": "kda_frontend.hip",
}


def kernel_source_digest(kernel_tag: str) -> str:
    """sha256 over the sources of the kernel a summary tag names: identifies the code measured."""
    pkg = os.path.join(ROOT, "linear_attention_recurrence_08_amd")
    src = next(f for prefix, f in sorted(KERNEL_SOURCES.items(), key=lambda kv: -len(kv[0]))
               if kernel_tag.startswith(prefix))
    srcs = (src,) if isinstance(src, str) else src
    h = hashlib.sha256()
    for path in tuple(os.path.join(pkg, "csrc", f) for f in srcs) + (
            os.path.join(pkg, "csrc", "kda_internal.h"), os.path.join(pkg, "csrc", "kda_mfma.h"),
            os.path.join(pkg, "build.py")):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_tag: str):
    """HBM bytes per launch from the committed counter summary for this kernel, if its recorded
    source digest matches the current sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_hbm_traffic.md")  # noqa: E501
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_d = re.search(r"source_digest:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_d or not m_b or m_d.group(1) != kernel_source_digest(kernel_tag):
        return None
    return float(m_b.group(1))


CALIB_BYTES = 1 << 30   # calibration copy: reads and writes exactly this many bytes


def traffic_pass(dev, workload=None):
    """A plain copy of known size (y = x * 1 over 1 GiB of float32), then 3 launches of each
    entry point the bench line times, on its benchmark workload.  With `workload` (a prefill
    workload other than the bench line's), 3 launches of kda_chunk_fwd on it alone."""
    import torch
    from linear_attention_recurrence_08_amd import (inputs, kda_chunk_fwd, kda_chunk_fwd_snapshots,
                                                    kda_decode_step, kda_decode_step_gated,
                                                    kda_frontend, kda_output_gate)
    if workload is not None:
        w = inputs.make_workload(workload).to(dev)
        for _ in range(3):
            kda_chunk_fwd(*w.call_views(), h0=w.h0, cu_seqlens=w.cu_seqlens)
        torch.cuda.synchronize()
        print("traffic pass done", file=sys.stderr)
        return
    x = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    del x, y
    w = inputs.make_workload("prefill_T4096_H96_d128_bf16").to(dev)
    for _ in range(3):
        kda_chunk_fwd(*w.call_views(), h0=w.h0, cu_seqlens=w.cu_seqlens)
    from linear_attention_recurrence_08_amd import kda_chunk_fwd_chunk64
    for _ in range(3):
        kda_chunk_fwd_chunk64(*w.call_views(), h0=w.h0, cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    del w
    d = inputs.make_workload(DECODE_WORKLOAD)
    qd, kd, vd, gd, bd, S = (t.to(dev) for t in (d.q, d.k, d.v, d.g, d.beta, d.h0))
    for _ in range(3):
        kda_decode_step(qd, kd, vd, gd, bd, S)
    _, dz, dw = (t.to(dev) for t in inputs.make_output_gate_inputs(256, 96, 128, "bf16", 62))
    for _ in range(3):
        kda_decode_step_gated(qd, kd, vd, gd, bd, S, dz, dw, 1e-6)
    from linear_attention_recurrence_08_amd import kda_decode_step_layer
    fr = inputs.make_frontend_inputs([1] * 256, 96, 128, 128, "bf16", seed=653,
                                     with_state=True).to(dev)
    for _ in range(3):
        kda_decode_step_layer(fr.x_q, fr.x_k, fr.x_v, fr.x_z, fr.x_b, fr.w_q, fr.w_k, fr.w_v,
                              fr.z_bias, fr.A, fr.conv_in, S, dz, dw)
    torch.cuda.synchronize()
    del qd, kd, vd, gd, bd, S, dz, dw, fr
    og, gz, gw = (t.to(dev) for t in inputs.make_output_gate_inputs(4096, 96, 128, "bf16", 61))
    for _ in range(3):
        kda_output_gate(og, gz, gw, 1e-6)
    torch.cuda.synchronize()
    del og, gz, gw
    fr = inputs.make_frontend_inputs([4096], 96, 128, 128, "bf16", seed=93).to(dev)
    for _ in range(3):
        kda_frontend(fr.x_q, fr.x_k, fr.x_v, fr.x_z, fr.x_b, fr.w_q, fr.w_k, fr.w_v, fr.z_bias,
                     fr.A, cu_seqlens=fr.cu_seqlens, output_conv_state=True)
    torch.cuda.synchronize()
    print("traffic pass done", file=sys.stderr)


SUMMARY_KERNELS = {
    # kernel name fragment (as rocprofv3 records it) -> (summary tag, workload)
    "kda_prefill_mfma_kernel": ("kda_chunk_fwd_prefill_T4096_H96_d128_bf16",
                                "prefill_T4096_H96_d128_bf16"),
    # 64-token chunks: the state-independent prep kernel, then the carry (one head in two halves)
    "kda_c64_prep_kernel": ("kda_chunk_fwd_chunk64_prefill_T4096_H96_d128_bf16",
                            "prefill_T4096_H96_d128_bf16"),
    "kda_c64_carry_kernel<1>": ("kda_chunk_fwd_chunk64_prefill_T4096_H96_d128_bf16",
                                "prefill_T4096_H96_d128_bf16"),
    "kda_decode_d128_kernel<unsigned short, 2, false, false>": (
        "kda_decode_decode_N256_H96_d128_bf16", "decode_N256_H96_d128_bf16"),
    "kda_decode_d128_kernel<unsigned short, 2, true, false>": (
        "kda_decode_step_gated_decode_N256_H96_d128_bf16", "decode_gated_N256_H96_d128_bf16"),
    # the whole mixer's decode step in one launch (input stage, decode, output stage)
    "kda_decode_d128_kernel<unsigned short, 2, true, true>": (
        "kda_decode_step_layer_decode_N256_H96_d128_bf16", "decode_layer_N256_H96_d128_bf16"),
    "kda_output_gate_kernel<unsigned short>": ("kda_output_gate_T4096_H96_d128_bf16",
                                               "output_gate_T4096_H96_d128_bf16"),
    # the input stage: one kernel streams q, k, v and the gates, a second saves the conv state
    "kda_frontend_conv_kernel<unsigned short, true>": ("kda_frontend_T4096_H96_d128_bf16",
                                                       "frontend_T4096_H96_d128_bf16"),
    "kda_frontend_state_kernel<unsigned short>": ("kda_frontend_T4096_H96_d128_bf16",
                                                  "frontend_T4096_H96_d128_bf16"),
}


# Kernels that other timed entries of the same bench run launch at other sizes (the serving
# step's 4 sequences, the one-launch decode's three-launch comparison): their summaries keep the
# dispatches of their own workload, told apart by the grid (threads in x and y).
SUMMARY_GRIDS = {
    "kda_decode_d128_kernel<unsigned short, 2, false, false>": (256 * 96 // 2 * 256, 1),
    "kda_decode_d128_kernel<unsigned short, 2, true, false>": (256 * 96 // 2 * 256, 1),
    "kda_decode_d128_kernel<unsigned short, 2, true, true>": (256 * 96 // 2 * 256, 1),
    "kda_frontend_conv_kernel<unsigned short, true>": (4096 // 128 * 96 * 64, 4),
    "kda_frontend_state_kernel<unsigned short>": (96 * 384, 1),
}


def _dispatch_stats(trace_csvs, frag, grid):
    """Calls, mean, min, max and total duration (ns) of the dispatches of one kernel with the
    given grid, from rocprofv3 kernel-trace rows; None without any."""
    import csv
    durs = []
    for f in trace_csvs:
        for r in csv.DictReader(open(f)):
            if frag in r["Kernel_Name"] and (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"])) == grid:
                durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not durs:
        return None
    return {"Calls": str(len(durs)), "AverageNs": sum(durs) / len(durs), "MinNs": min(durs),
            "MaxNs": max(durs), "TotalDurationNs": sum(durs)}


def _algorithmic_bytes(workload):
    from linear_attention_recurrence_08_amd import inputs
    tok_head = 4096 * 96
    if workload == "decode_gated_N256_H96_d128_bf16":
        return 256 * 96 * (2 * 128 * 128 * 4 + (3 * 128 + 2 * 128) * 2 + 2 + 2 * 128 * 2) + 512
    if workload == "decode_layer_N256_H96_d128_bf16":
        return decode_layer_bytes(256, 96)
    if workload == "output_gate_T4096_H96_d128_bf16":
        return 3 * tok_head * 128 * 2 + 128 * 4
    if workload == "frontend_T4096_H96_d128_bf16":
        return 2 * tok_head * ((3 * 128 + 128) * 2 + 2)
    w = inputs.WORKLOADS[workload]
    if w["kind"] == "decode":
        return w["N"] * w["H"] * (2 * w["dk"] * w["dv"] * 4 + (3 * w["dk"] + 2 * w["dv"]) * 2 + 2)
    T = sum(w["seq_lens"])
    return T * w["H"] * ((3 * w["dk"] + 2 * w["dv"]) * 2 + 2) + len(w["seq_lens"]) * w["H"] * \
        w["dk"] * w["dv"] * 4


def summarize(dirs, command, workload=None):
    """profiles/<kernel>_<workload>_kernel_trace.md from a --kernel-trace --stats run and
    profiles/<kernel>_<workload>_hbm_traffic.md from FETCH_SIZE + WRITE_SIZE counter runs (each
    scaled by what the same counter reads for the 1 GiB calibration copy).  Where one entry point
    launches several kernels, the summary lists each and adds them up per call.  With `workload`,
    the runs timed kda_chunk_fwd alone on that prefill workload (bench.py --workload NAME)."""
    import csv
    import glob
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    kernels = SUMMARY_KERNELS
    if workload is not None:
        kernels = {"kda_prefill_mfma_kernel": ("kda_chunk_fwd_" + workload, workload)}
    tags = {}
    for frag, (tag, wl) in kernels.items():
        tags.setdefault(tag, (wl, []))[1].append(frag)
    trace = {}        # tag -> list of (fragment, stats row)
    counters = {}     # (fragment or "copy", counter) -> list of per-dispatch values (KiB)
    for d in dirs:
        per_dispatch = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
        for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                for frag, (tag, _) in kernels.items():
                    if frag in r["Name"]:
                        row = r
                        if frag in SUMMARY_GRIDS and workload is None:
                            row = _dispatch_stats(per_dispatch, frag, SUMMARY_GRIDS[frag])
                            if row is None:
                                continue
                        trace.setdefault(tag, []).append((frag, row))
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name = r["Kernel_Name"]
                key = None
                if "elementwise" in name or "vectorized" in name:
                    key = "copy"
                for frag in kernels:
                    if frag in name:
                        key = frag
                if key is None:
                    continue
                counters.setdefault((key, r["Counter_Name"]), []).append(
                    float(r["Counter_Value"]))
    for tag, rows in trace.items():
        wl, _ = tags[tag]
        path = os.path.join(out_dir, f"{tag}_kernel_trace.md")
        with open(path, "w") as fo:
            names = ", ".join(frag for frag, _ in rows)
            fo.write(f"# {names} on {wl}: rocprofv3 kernel trace\n\n")
            fo.write(f"command: `{command}`\n\n")
            fo.write("| kernel | calls | average ns | min ns | max ns | total ns |\n")
            fo.write("|---|---|---|---|---|---|\n")
            for frag, r in rows:
                fo.write(f"| {frag} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                         f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} | "
                         f"{float(r['TotalDurationNs']):.0f} |\n")
            if len(rows) > 1:
                fo.write(f"| sum per call | | "
                         f"{sum(float(r['AverageNs']) for _, r in rows):.0f} | | | |\n")
            fo.write(f"\nsource_digest: {kernel_source_digest(tag)}\n")
        print("wrote", path)
    if counters:
        cal = {}
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = counters.get(("copy", cn))
            if vals:
                cal[cn] = max(vals) * 1024.0 / CALIB_BYTES   # counter bytes per true byte
        for tag, (wl, frags) in tags.items():
            if "FETCH_SIZE" not in cal or "WRITE_SIZE" not in cal:
                continue
            fetch = write = 0.0
            ndisp = []
            for frag in frags:
                f_vals = counters.get((frag, "FETCH_SIZE"))
                w_vals = counters.get((frag, "WRITE_SIZE"))
                if not f_vals or not w_vals:
                    break
                fetch += sum(f_vals) / len(f_vals) * 1024.0 / cal["FETCH_SIZE"]
                write += sum(w_vals) / len(w_vals) * 1024.0 / cal["WRITE_SIZE"]
                ndisp.append(str(len(f_vals)))
            else:
                algo = _algorithmic_bytes(wl)
                path = os.path.join(out_dir, f"{tag}_hbm_traffic.md")
                with open(path, "w") as fo:
                    fo.write(f"# {', '.join(frags)} on {wl}: HBM traffic per call "
                             "(rocprofv3 counters)\n\n")
                    fo.write(f"command: `{command}`\n\n")
                    fo.write("Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each taken "
                             "in its own run and scaled by what the same counter reads for a copy "
                             f"of exactly {CALIB_BYTES} bytes read and {CALIB_BYTES} bytes "
                             f"written (factor FETCH {cal['FETCH_SIZE']:.4f}, WRITE "
                             f"{cal['WRITE_SIZE']:.4f} counter bytes per byte); the per-dispatch "
                             "means of the kernels of one call are added.\n\n")
                    fo.write("| dispatches | fetch bytes | write bytes | total bytes | "
                             "algorithmic bytes | total / algorithmic |\n"
                             "|---|---|---|---|---|---|\n")
                    fo.write(f"| {' + '.join(ndisp)} | {fetch:.4g} | {write:.4g} | "
                             f"{fetch + write:.4g} | {algo} | {(fetch + write) / algo:.3f} |\n\n")
                    fo.write(f"source_digest: {kernel_source_digest(tag)}\n")
                    fo.write(f"hbm_bytes_per_launch: {fetch + write:.6g}\n")
                print("wrote", path)


def _cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


SETTLE_S = 0.3   # untimed launches continue after the warm-up steps until this much wall time


def time_launches(fn, steps, warmup, stream, settle_s=None):
    """Mean time per launch of `steps` launches of fn on `stream` (HIP events), after `warmup`
    untimed launches; the untimed launches continue until settle_s seconds have passed, so that
    the timed ones run at the clocks the GPU holds under sustained load."""
    import torch
    settle_s = SETTLE_S if settle_s is None else settle_s
    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < settle_s:
        fn()
        done += 1
        if done % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return start.elapsed_time(end) / steps, wall  # ms per launch (one kernel per step), seconds


def serving_step_graph(dev, stream, steps, N=4):
    """The per-token serving step of the token mixer for a small batch, N sequences x 96 heads:
    the input stage (its convolution state updated in place), the decode (the recurrent state
    updated in place) and the output stage, as three launches (kda_frontend, then
    kda_decode_step_gated) and as one (kda_decode_step_layer).  Each is timed as eager calls and as
    one captured HIP graph replayed per token; at this size the launches cost more than the
    kernels."""
    import torch
    from linear_attention_recurrence_08_amd import (inputs, kda_decode_step_gated,
                                                    kda_decode_step_layer, kda_frontend)
    H = 96
    f = inputs.make_frontend_inputs([1] * N, H, 128, 128, "bf16", seed=650,
                                    with_state=True).to(dev)
    _, z, w = (t.to(dev) for t in inputs.make_output_gate_inputs(N, H, 128, "bf16", 651))
    S = inputs.make_decode_inputs(N, H, 128, 128, "bf16", seed=652).h0.to(dev)
    ones = torch.arange(N + 1, dtype=torch.int32, device=dev)
    conv = f.conv_in

    def step():
        q, k, v, g, b, _ = kda_frontend(f.x_q, f.x_k, f.x_v, f.x_z, f.x_b, f.w_q, f.w_k, f.w_v,
                                        f.z_bias, f.A, cu_seqlens=ones, conv_in=conv,
                                        conv_out=conv)
        kda_decode_step_gated(q, k, v, g, b, S, z, w)

    def step_fused():
        kda_decode_step_layer(f.x_q, f.x_k, f.x_v, f.x_z, f.x_b, f.w_q, f.w_k, f.w_v, f.z_bias,
                              f.A, conv, S, z, w)

    out = {"N": N, "H": H}
    for tag, fn, launches, entries in (
            ("three_kernels", step, 3, "kda_frontend + kda_decode_step_gated"),
            ("one_kernel", step_fused, 1, "kda_decode_step_layer")):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        eager_ms, _ = time_launches(fn, steps, 3, stream)
        graph_ms, _ = time_launches(graph.replay, steps, 3, stream)
        out[tag] = {"entries": entries, "launches_per_token": launches,
                    "eager_us_per_token": round(eager_ms * 1e3, 2),
                    "graph_us_per_token": round(graph_ms * 1e3, 2),
                    "graph_tokens_per_s": round(N / (graph_ms * 1e-3), 1),
                    "graph_vs_eager": round(eager_ms / graph_ms, 3)}
        del graph
    return out


def long_context(dev, stream, steps):
    """The long-context prefill (B = 1, T = 131,072, H = 96, bimodal per-channel decay): the same
    work per token as the 4,096-token layer, over a 32 times longer serial chain of tiles."""
    import torch
    from linear_attention_recurrence_08_amd import inputs, kda_chunk_fwd
    t0 = time.perf_counter()
    xl = inputs.make_workload(LONG_WORKLOAD)
    xld = xl.to(dev)
    gen_s = time.perf_counter() - t0
    lviews = xld.call_views()
    ol = torch.empty_like(lviews[2])
    hTl = torch.empty((xl.num_seqs, xl.H, xl.dk, xl.dv), dtype=torch.float32, device=dev)
    print(f"[bench] long context {LONG_WORKLOAD}: T={xl.total_tokens} H={xl.H} steps={steps} "
          f"(inputs drawn in {gen_s:.1f} s)", file=sys.stderr, flush=True)

    def prefill_long():
        kda_chunk_fwd(*lviews, h0=xld.h0, cu_seqlens=xld.cu_seqlens, o=ol, hT=hTl)

    lms, _ = time_launches(prefill_long, steps, 1, stream)
    lbytes = prefill_bytes(xl)
    lgbs = lbytes / (lms * 1e-3) / 1e9
    out = {
        "workload": LONG_WORKLOAD, "total_tokens": xl.total_tokens, "steps": steps,
        "ms_per_step": round(lms, 4), "value": round(xl.total_tokens / (lms * 1e-3), 1),
        "unit": "tokens/s",
        "roofline": {"bound": "hbm", "achieved": round(lgbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(lgbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("kda_chunk_fwd_" + LONG_WORKLOAD),
                     "kernel": "kda_prefill_mfma", "algorithmic_bytes_per_launch": lbytes},
    }
    del xl, xld, lviews, ol, hTl
    return out


def head_share(dev, stream, steps, warmup, unsplit=True):
    """Prefill of one GPU's share of K3's heads under 8-way head sharding (12 of 96, T = 4096,
    batch 1): kda_chunk_fwd beside kda_chunk_fwd_split with the library's segment count
    (unsplit=False: the split alone)."""
    import torch
    from linear_attention_recurrence_08_amd import (inputs, kda_chunk_fwd, kda_chunk_fwd_split,
                                                    kda_chunk_fwd_split_segments,
                                                    kda_chunk_fwd_split_workspace_bytes)
    Hs, Ts = 12, 4096
    xs = inputs.make_inputs([Ts], H=Hs, dk=128, dv=128, dtype="bf16", seed=1, packed=False)
    xsd = xs.to(dev)
    sviews = xsd.call_views()
    o_s = torch.empty_like(sviews[2])
    h_s = torch.empty((1, Hs, 128, 128), dtype=torch.float32, device=dev)
    P = kda_chunk_fwd_split_segments(xsd.q, 1, Ts, Hs, 128, 128, 0)
    sbytes = kda_chunk_fwd_split_workspace_bytes(xsd.q, 1, Ts, Hs, 128, 128, 0)
    ws_s = torch.empty(max(sbytes, 1), dtype=torch.uint8, device=dev)
    print(f"[bench] head share T={Ts} H={Hs}: {P} segments", file=sys.stderr, flush=True)

    def share_plain():
        kda_chunk_fwd(*sviews, o=o_s, hT=h_s)

    def share_split():
        kda_chunk_fwd_split(*sviews, segments=0, o=o_s, hT=h_s, workspace=ws_s)

    sp_ms = time_launches(share_plain, steps, warmup, stream)[0] if unsplit else float("nan")
    ss_ms, _ = time_launches(share_split, steps, warmup, stream)
    sb = prefill_bytes(xs)
    return {
        "workload": f"prefill_T{Ts}_H{Hs}_d128_bf16 (12 of 96 heads: one GPU under 8-way head "
                    "sharding)",
        "kernel": "kda_prefill_mfma (token-range split) + kda_split_compose + kda_split_fixup",
        "segments": P, "workspace_bytes": sbytes,
        "unsplit_ms_per_step": round(sp_ms, 5) if unsplit else None,
        "ms_per_step": round(ss_ms, 5),
        "value": round(Ts / (ss_ms * 1e-3), 1), "unit": "tokens/s",
        "vs_unsplit": round(sp_ms / ss_ms, 3) if unsplit else None,
        "roofline": {"bound": "hbm", "achieved": round(sb / (ss_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(sb / (ss_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": sb},
    }


DEFAULT_WORKLOAD = "prefill_T4096_H96_d128_bf16"   # the bench line's prefill
SQ_PASS1 = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
            "SQ_INSTS_SALU SQ_INSTS_VMEM")
SQ_PASS2 = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT "
            "SQ_INSTS_VALU_TRANS_F32 SQ_WAIT_INST_LDS SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_ANY")


def summarize_sq(dirs, command, wl=None):
    """profiles/kda_chunk_fwd_<workload>_sq_counters.md from two rocprofv3 --pmc runs of
    --traffic-pass (the SQ_PASS1 and SQ_PASS2 counter sets; for a workload other than the bench
    line's, runs of --traffic-pass --workload NAME).  The prefill kernel runs one workgroup of 12
    waves per (sequence, head, 64-column half) on a CU of its own (one per (sequence, head) from
    256 pairs up), each SIMD holding one wave of each of the three roles, and walks nsteps + 4
    pipeline periods (nsteps = the sequence's tile count rounded up to even); counts are given
    per SIMD and period, over all workgroups' periods."""
    import csv
    import glob
    from linear_attention_recurrence_08_amd import inputs
    wl = wl or DEFAULT_WORKLOAD
    w = inputs.WORKLOADS[wl]
    lens = (inputs.varlen_lengths(w["seed"], w["n_seqs"]) if w["kind"] == "varlen"
            else list(w["seq_lens"]))
    H = w["H"]
    pairs = len(lens) * H
    halves = 1 if pairs >= 256 else 2
    wgs = halves * pairs

    def walk(n):
        nt = (n + 15) // 16
        return nt + (nt & 1) + 4
    total_periods = halves * H * sum(walk(n) for n in lens)   # summed over workgroups
    periods = total_periods / wgs                              # per workgroup, mean
    simds, waves = 4 * wgs, 12 * wgs
    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if "kda_prefill_mfma_kernel" in r["Kernel_Name"]:
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    m = {k: sum(v) / len(v) for k, v in vals.items()}
    ndisp = len(vals.get("SQ_WAVES", []))
    assert round(m["SQ_WAVES"]) == waves, (m["SQ_WAVES"], waves)

    def per(k, x4=False):
        return m[k] * (4 if x4 else 1) / simds / periods
    rows = [(k, m[k], f"{per(k):.1f}") for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                                                  "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS",
                                                  "SQ_INSTS_SALU", "SQ_INSTS_VMEM")]
    for k in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
              "SQ_WAIT_INST_LDS"):
        rows.append((k + " (x4)", m[k], f"{per(k, True):.0f} cycles"))
    rows.append(("SQ_VALU_MFMA_BUSY_CYCLES", m["SQ_VALU_MFMA_BUSY_CYCLES"],
                 f"{per('SQ_VALU_MFMA_BUSY_CYCLES'):.0f} cycles"))
    rows.append(("SQ_LDS_BANK_CONFLICT", m["SQ_LDS_BANK_CONFLICT"],
                 f"{m['SQ_LDS_BANK_CONFLICT'] / wgs / periods:.0f} cycles per CU"))
    wave_cyc = m["SQ_WAVE_CYCLES"] * 4 / waves
    rows.append(("SQ_WAVE_CYCLES (x4)", m["SQ_WAVE_CYCLES"],
                 f"{wave_cyc:.0f} cycles per wave in all"))
    period = wave_cyc / periods
    other = (m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]) / simds / periods
    active = per("SQ_ACTIVE_INST_ANY", True) / period
    busy = per("SQ_VALU_MFMA_BUSY_CYCLES") / period
    path = os.path.join(ROOT, "profiles", f"kda_chunk_fwd_{wl}_sq_counters.md")
    with open(path, "w") as fo:
        fo.write(f"# kda_prefill_mfma_kernel on {wl}: SQ instruction counters\n\n")
        fo.write(f"command: `{command}`\n\n")
        fo.write(f"Means over the {ndisp} dispatches of the traffic pass; {waves} waves = {wgs} "
                 f"workgroups of 12 waves, {simds} SIMDs, {periods:.1f} pipeline periods per "
                 "workgroup (mean). Cycle counters marked (x4) count in units of four cycles.\n\n")
        fo.write("| counter | per launch | per SIMD and period |\n|---|---|---|\n")
        for k, v, dsc in rows:
            fo.write(f"| {k} | {v:.4g} | {dsc} |\n")
        fo.write(f"\nDerived: VALU instructions other than MFMA {other:.0f} per SIMD and period; a "
                 f"period of {period:.0f} cycles; instruction issue active {100 * active:.0f}% of "
                 f"a SIMD's cycles; MFMA unit busy {100 * busy:.0f}%.\n\n")
        fo.write(f"source_digest: {kernel_source_digest('kda_chunk_fwd')}\n")
    print("wrote", path)


def summarize_split(trace_dir, command):
    """profiles/kda_chunk_fwd_split_T4096_H12_d128_bf16_kernel_trace.md from a --kernel-trace
    --stats run of `bench.py --head-share-only` (every kernel of that run: the unsplit prefill, and
    the split's prefill, composition and correction)."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        rows += [r for r in csv.DictReader(open(f)) if "kda_" in r["Name"]]
    path = os.path.join(ROOT, "profiles", "kda_chunk_fwd_split_T4096_H12_d128_bf16_kernel_trace.md")
    with open(path, "w") as fo:
        fo.write("# kda_chunk_fwd_split on prefill_T4096_H12_d128_bf16 (12 of 96 heads, batch 1): "
                 "rocprofv3 kernel trace\n\n")
        fo.write(f"command: `{command}`\n\n")
        fo.write("Every kernel of one split call: the prefill launch (5 segments: 216 workgroups), "
                 "the composition of the entering states and the output correction.\n\n")
        fo.write("| kernel | calls | average ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in rows:
            name = re.sub(r"\(kda::PrefillArgs\)|void |kda::\(anonymous namespace\)::", "",
                          r["Name"])
            fo.write(f"| {name} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |\n")
        fo.write(f"\nsource_digest: {kernel_source_digest('kda_chunk_fwd_split')}\n")
    print("wrote", path)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=PREFILL_WORKLOADS)
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--snapshot-stride", type=int, default=64)
    ap.add_argument("--no-snapshots", action="store_true")
    ap.add_argument("--no-output-gate", action="store_true")
    ap.add_argument("--no-frontend", action="store_true")
    ap.add_argument("--no-chunk64", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-split", action="store_true")
    ap.add_argument("--head-share-only", action="store_true",
                    help="time only the 12-head prefill (kda_chunk_fwd beside kda_chunk_fwd_split)")
    ap.add_argument("--split-only", action="store_true",
                    help="with --head-share-only: time the split alone (for a kernel trace)")
    ap.add_argument("--summarize-split", metavar="DIR",
                    help="write the split prefill's kernel-trace summary from a rocprofv3 run of "
                         "--head-share-only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="run a 1 GiB calibration copy and 3 launches of each kernel (for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE); prints no JSON")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="write profiles/*.md from rocprofv3 output directories: a kernel-trace "
                         "--stats run and/or FETCH_SIZE and WRITE_SIZE counter runs")
    ap.add_argument("--command", default="", help="command line recorded in the summaries")
    ap.add_argument("--summarize-sq", nargs=2, metavar="DIR",
                    help="write the prefill kernel's SQ counter summary from two rocprofv3 --pmc "
                         "runs of --traffic-pass (counter sets SQ_PASS1 and SQ_PASS2)")
    ap.add_argument("--summary-workload", default=None, metavar="NAME",
                    help="with --summarize: the runs timed kda_chunk_fwd alone on this prefill "
                         "workload (bench.py --workload NAME)")
    args = ap.parse_args()
    if args.summarize_split:
        summarize_split(args.summarize_split, args.command)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.command, args.summary_workload)
        return
    if args.summarize:
        summarize(args.summarize, args.command, args.summary_workload)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads and sequences would shard across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_recurrence_08_amd import (inputs, kda_chunk_fwd, kda_chunk_fwd_snapshots,
                                                    kda_decode_step, kda_decode_step_gated,
                                                    kda_frontend, kda_output_gate)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.traffic_pass:
        traffic_pass(dev, None if args.workload == DEFAULT_WORKLOAD else args.workload)
        return
    if args.head_share_only:
        print(json.dumps(head_share(dev, stream, args.steps, args.warmup,
                                    unsplit=not args.split_only)))
        return

    # ---------------- prefill ----------------
    x = inputs.make_workload(args.workload)
    xd = x.to(dev)
    args_views = xd.call_views()
    o = torch.empty_like(args_views[2])
    hT = torch.empty((x.num_seqs, x.H, x.dk, x.dv), dtype=torch.float32, device=dev)
    print(f"[bench] prefill {args.workload}: Ttot={x.total_tokens} H={x.H} warmup={args.warmup} "
          f"steps={args.steps}", file=sys.stderr, flush=True)

    def prefill():
        kda_chunk_fwd(*args_views, h0=xd.h0, cu_seqlens=xd.cu_seqlens, o=o, hT=hT)

    ms, wall = time_launches(prefill, args.steps, args.warmup, stream)
    tokens = x.total_tokens
    value = tokens / (ms * 1e-3)
    nbytes = prefill_bytes(x)
    flops = prefill_flops(x)
    achieved_gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = recorded_traffic("kda_chunk_fwd_" + args.workload)
    roofline = {
        "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": "kda_prefill_mfma" if (x.dtype == "bf16" and x.dk == 128 and x.dv == 128)
        else "kda_prefill_general",
        "algorithmic_bytes_per_launch": nbytes,
        "algorithmic_flops_per_launch": flops,
        # per (token, head): this count, 6 dk dv + d (5 C - 1), and for context the fit
        # 6 d^2 + 3 C d + C^2 to the pages' "about 127,000 at chunk 64" (126,976 at C = 64)
        "flops_per_token_head": 6 * x.dk * x.dv + x.dk * (5 * CHUNK - 1),
        "pages_fit_flops_per_token_head": {"C16": 6 * x.dk * x.dk + 3 * 16 * x.dk + 16 * 16,
                                           "C64": 6 * x.dk * x.dk + 3 * 64 * x.dk + 64 * 64},
        "kernel_ms": round(ms, 5),
        "mfma_bf16_tflops": round(tflops, 2),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFS, 4),
        # fraction of the attainable roofline: the faster of the HBM and matrix-core bounds
        "attainable_frac": round(max(nbytes / (HBM_PEAK_GBS * 1e9),
                                     flops / (MFMA_BF16_PEAK_TFS * 1e12)) / (ms * 1e-3), 4),
        "source_digest": kernel_source_digest("kda_chunk_fwd"),
    }

    result = {
        "metric": "KDA prefill tokens/s & decode tokens/s (H=96,d=128), % of MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": x.B, "T": x.T, "H": x.H, "dk": x.dk,
                   "dv": x.dv, "chunk": CHUNK, "num_seqs": x.num_seqs,
                   "total_tokens": tokens, "state": "f32"},
        "roofline": roofline,
        "wall_s_timed": round(wall, 4),
    }

    # ---------------- 64-token chunks beside 16-token tiles ----------------
    if not args.no_chunk64:
        from linear_attention_recurrence_08_amd import kda_chunk_fwd_chunk64
        from linear_attention_recurrence_08_amd.kda import kda_chunk_fwd_chunk64_workspace_bytes

        o_c, hT_c = torch.empty_like(o), torch.empty_like(hT)   # leave the prefill's o intact
        q0 = args_views[0]
        cB, cT = (1, q0.shape[0]) if q0.dim() == 3 else (q0.shape[0], q0.shape[1])
        ws_bytes = kda_chunk_fwd_chunk64_workspace_bytes(q0, xd.cu_seqlens, x.num_seqs, cB, cT,
                                                         x.H, x.dk, x.dv)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

        def prefill_c64():
            kda_chunk_fwd_chunk64(*args_views, h0=xd.h0, cu_seqlens=xd.cu_seqlens, o=o_c, hT=hT_c,
                                  workspace=ws)

        def forced_float32(fn):
            def run():
                os.environ["KDA_FORCE_GENERAL"] = "1"
                try:
                    fn()
                finally:
                    del os.environ["KDA_FORCE_GENERAL"]
            return run

        def prefill_c16():
            kda_chunk_fwd(*args_views, h0=xd.h0, cu_seqlens=xd.cu_seqlens, o=o_c, hT=hT_c)

        c64ms, _ = time_launches(prefill_c64, max(5, args.steps // 2), 2, stream)
        fsteps = max(3, args.steps // 10)
        f64ms, _ = time_launches(forced_float32(prefill_c64), fsteps, 1, stream, settle_s=0)
        f16ms, _ = time_launches(forced_float32(prefill_c16), fsteps, 1, stream, settle_s=0)
        # the workspace round trip: every (chunk, head) record written once and read back
        ws_traffic = 2 * ws_bytes
        result["chunk64"] = {
            "kernel": "kda_c64_prep + kda_c64_carry (matrix cores)" if ws_bytes else
                      "kda_prefill_c64 (float32 vector ALUs)",
            "steps": max(5, args.steps // 2),
            "ms_per_step": round(c64ms, 4), "value": round(tokens / (c64ms * 1e-3), 1),
            "unit": "tokens/s", "vs_chunk16": round(ms / c64ms, 4),
            "workspace_bytes": ws_bytes,
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (c64ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nbytes / (c64ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": nbytes,
                         "with_workspace_bytes_per_launch": nbytes + ws_traffic,
                         "with_workspace_frac": round((nbytes + ws_traffic) / (c64ms * 1e-3) /
                                                      1e9 / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("kda_chunk_fwd_chunk64_" + args.workload)},
            "float32_vector_ms_per_step": round(f64ms, 4),
            "chunk16_float32_vector_ms_per_step": round(f16ms, 4),
        }
        del o_c, hT_c, ws

    # ---------------- one GPU's share of the heads: 12 of 96 (8-way head sharding), batch 1 ------
    if not args.no_split:
        result["head_share"] = head_share(dev, stream, args.steps, args.warmup)

    # ---------------- long context: one sequence of 131,072 tokens ----------------
    if not args.no_long and args.workload != LONG_WORKLOAD:
        result["long"] = long_context(dev, stream, max(3, args.steps // 4))
        torch.cuda.empty_cache()

    # ---------------- variable-length batch: 16 sequences of 1,024-16,384 tokens ----------------
    if not args.no_varlen and args.workload != VARLEN_WORKLOAD:
        xv = inputs.make_workload(VARLEN_WORKLOAD)
        xvd = xv.to(dev)
        vviews = xvd.call_views()
        ov = torch.empty_like(xvd.v)
        hTv = torch.empty((xv.num_seqs, xv.H, xv.dk, xv.dv), dtype=torch.float32, device=dev)

        def prefill_varlen():
            kda_chunk_fwd(*vviews, h0=xvd.h0, cu_seqlens=xvd.cu_seqlens, o=ov, hT=hTv)

        vsteps = max(3, args.steps // 10)
        vms, _ = time_launches(prefill_varlen, vsteps, 1, stream)
        vbytes = prefill_bytes(xv)
        lens = [e - s for s, e in xv.seq_bounds()]
        result["varlen"] = {
            "workload": VARLEN_WORKLOAD, "num_seqs": xv.num_seqs, "total_tokens": xv.total_tokens,
            "min_len": min(lens), "max_len": max(lens), "steps": vsteps,
            "ms_per_step": round(vms, 4), "value": round(xv.total_tokens / (vms * 1e-3), 1),
            "unit": "tokens/s",
            "roofline": {"bound": "hbm", "achieved": round(vbytes / (vms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(vbytes / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": vbytes},
        }
        # the prefill with the output stage (kda_chunk_fwd_gated, fused for these 1,536 pairs)
        # against the prefill followed by the output-stage kernel
        if not args.no_output_gate:
            from linear_attention_recurrence_08_amd import (kda_chunk_fwd_gated,
                                                            kda_chunk_fwd_gated_fuses)
            _, zv, wv = inputs.make_output_gate_inputs(xv.total_tokens, xv.H, xv.dv, "bf16", 61)
            zv, wv = zv.to(dev).reshape(vviews[2].shape), wv.to(dev)
            yv = torch.empty_like(ov)

            def gated_varlen():
                kda_chunk_fwd_gated(*vviews, zv, weight=wv, h0=xvd.h0, cu_seqlens=xvd.cu_seqlens,
                                    y=yv, hT=hTv)

            def unfused_varlen():
                prefill_varlen()
                kda_output_gate(ov, zv, wv, y=yv)

            gvms, _ = time_launches(gated_varlen, vsteps, 1, stream)
            uvms, _ = time_launches(unfused_varlen, vsteps, 1, stream)
            row = xv.total_tokens * xv.H * xv.dv * 2          # one [Ttot, H, dv] bf16 tensor
            gbytes = vbytes + row                              # + gate read; y written in o's place
            result["varlen"]["gated"] = {
                "entry": "kda_chunk_fwd_gated",
                "fused": kda_chunk_fwd_gated_fuses(xvd.q, xv.num_seqs, 1, xv.H, xv.dk, xv.dv,
                                                   True),
                "ms_per_step": round(gvms, 4),
                "value": round(xv.total_tokens / (gvms * 1e-3), 1), "unit": "tokens/s",
                "unfused_ms_per_step": round(uvms, 4), "vs_unfused": round(uvms / gvms, 3),
                "algorithmic_bytes_per_launch": gbytes,
                "unfused_algorithmic_bytes": vbytes + 3 * row,
                "hbm_bytes_removed": 2 * row,
                "roofline": {"bound": "hbm",
                             "achieved": round(gbytes / (gvms * 1e-3) / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbytes / (gvms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            }
            # the whole token mixer on the same batch: the input stage, then the gated prefill
            # on its outputs, against the input stage, the prefill and the output-stage kernel
            if not args.no_frontend:
                fr = inputs.make_frontend_inputs(lens, xv.H, xv.dk, xv.dv, "bf16",
                                                 seed=93).to(dev)
                fst = torch.empty((xv.num_seqs, 3, xv.H * (2 * xv.dk + xv.dv)),
                                  dtype=fr.x_q.dtype, device=dev)

                def front_varlen():
                    return kda_frontend(fr.x_q, fr.x_k, fr.x_v, fr.x_z, fr.x_b, fr.w_q, fr.w_k,
                                        fr.w_v, fr.z_bias, fr.A, cu_seqlens=fr.cu_seqlens,
                                        conv_out=fst)[:5]

                def layer_fused():
                    kda_chunk_fwd_gated(*front_varlen(), zv, weight=wv, h0=xvd.h0,
                                        cu_seqlens=xvd.cu_seqlens, y=yv, hT=hTv)

                def layer_three_passes():
                    kda_chunk_fwd(*front_varlen(), h0=xvd.h0, cu_seqlens=xvd.cu_seqlens, o=ov,
                                  hT=hTv)
                    kda_output_gate(ov, zv, wv, y=yv)

                lms, _ = time_launches(layer_fused, vsteps, 1, stream)
                l3ms, _ = time_launches(layer_three_passes, vsteps, 1, stream)
                fbytes = 2 * xv.total_tokens * xv.H * ((3 * xv.dk + xv.dv) * 2 + 2)
                result["varlen"]["layer"] = {
                    "entries": "kda_frontend + kda_chunk_fwd_gated",
                    "ms_per_step": round(lms, 4),
                    "value": round(xv.total_tokens / (lms * 1e-3), 1), "unit": "tokens/s",
                    "three_pass_ms_per_step": round(l3ms, 4),
                    "vs_three_passes": round(l3ms / lms, 3),
                    "algorithmic_bytes_per_launch": fbytes + gbytes,
                    "three_pass_algorithmic_bytes": fbytes + vbytes + 3 * row,
                    "hbm_bytes_removed": 2 * row,
                }
                del fr, fst
            del zv, wv, yv
        del xv, xvd, vviews, ov, hTv
        torch.cuda.empty_cache()

    # ---------------- prefill with state snapshots ----------------
    if not args.no_snapshots:
        stride = args.snapshot_stride
        _, _, snaps, offs = kda_chunk_fwd_snapshots(*args_views, stride, h0=xd.h0,
                                                    cu_seqlens=xd.cu_seqlens, o=o, hT=hT)
        print(f"[bench] prefill with snapshots every {stride} tokens: {snaps.shape[0]} saved",
              file=sys.stderr, flush=True)

        def prefill_snap():
            kda_chunk_fwd_snapshots(*args_views, stride, h0=xd.h0, cu_seqlens=xd.cu_seqlens,
                                    snap_offsets=offs, o=o, hT=hT, snaps=snaps)

        sms, _ = time_launches(prefill_snap, args.steps, args.warmup, stream)
        sbytes = nbytes + snaps.numel() * 4
        result["snapshots"] = {
            "stride": stride, "saved": int(snaps.shape[0]), "ms_per_step": round(sms, 5),
            "value": round(tokens / (sms * 1e-3), 1), "unit": "tokens/s",
            "overhead_vs_prefill": round(sms / ms - 1.0, 4),
            "roofline": {"bound": "hbm", "achieved": round(sbytes / (sms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": sbytes},
        }
        del snaps, offs
        torch.cuda.empty_cache()

    # ---------------- output stage on the layer's output shape ----------------
    if not args.no_output_gate:
        og, gz, gw = (t.to(dev) for t in inputs.make_output_gate_inputs(
            x.total_tokens, x.H, x.dv, x.dtype, seed=61))
        gy = torch.empty_like(og)

        def out_gate():
            kda_output_gate(og, gz, gw, 1e-6, y=gy)

        gms, _ = time_launches(out_gate, args.steps, args.warmup, stream)
        gbytes = 3 * og.numel() * og.element_size() + gw.numel() * 4
        ggbs = gbytes / (gms * 1e-3) / 1e9
        result["output_gate"] = {
            "shape": list(og.shape), "ms_per_step": round(gms, 5),
            "value": round(x.total_tokens / (gms * 1e-3), 1), "unit": "tokens/s",
            "roofline": {"bound": "hbm", "achieved": round(ggbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(ggbs / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("kda_output_gate_T4096_H96_d128_bf16")
                         if (x.total_tokens, x.H, x.dv, x.dtype) == (4096, 96, 128, "bf16")
                         else None,
                         "kernel": "kda_output_gate", "algorithmic_bytes_per_launch": gbytes},
        }
        del og, gz, gw, gy
        torch.cuda.empty_cache()

    # ---------------- input stage on the same token and head count ----------------
    if not args.no_frontend:
        fr = inputs.make_frontend_inputs([e - s for s, e in x.seq_bounds()], x.H, x.dk, x.dv,
                                         x.dtype, seed=93).to(dev)
        fst = torch.empty((x.num_seqs, 3, x.H * (2 * x.dk + x.dv)), dtype=fr.x_q.dtype,
                          device=dev)

        def front():
            kda_frontend(fr.x_q, fr.x_k, fr.x_v, fr.x_z, fr.x_b, fr.w_q, fr.w_k, fr.w_v,
                         fr.z_bias, fr.A, cu_seqlens=fr.cu_seqlens, conv_out=fst)

        fms, _ = time_launches(front, args.steps, args.warmup, stream)
        es = fr.x_q.element_size()
        fbytes = 2 * x.total_tokens * x.H * ((3 * x.dk + x.dv) * es + es)
        fgbs = fbytes / (fms * 1e-3) / 1e9
        result["frontend"] = {
            "ms_per_step": round(fms, 5), "value": round(x.total_tokens / (fms * 1e-3), 1),
            "unit": "tokens/s",
            "roofline": {"bound": "hbm", "achieved": round(fgbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(fgbs / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("kda_frontend_T4096_H96_d128_bf16")
                         if (x.total_tokens, x.H, x.dv, x.dtype) == (4096, 96, 128, "bf16")
                         else None,
                         "kernel": "kda_frontend", "algorithmic_bytes_per_launch": fbytes},
        }
        del fr, fst
        torch.cuda.empty_cache()

    # ---------------- decode ----------------
    if not args.no_decode:
        d = inputs.make_workload(DECODE_WORKLOAD)
        qd, kd, vd, gd, bd = (t.to(dev) for t in (d.q, d.k, d.v, d.g, d.beta))
        S = d.h0.to(dev)
        od = torch.empty_like(vd)
        del d
        ksteps = args.decode_steps or args.steps
        print(f"[bench] decode {DECODE_WORKLOAD}: N=256 H=96 steps={ksteps}", file=sys.stderr,
              flush=True)

        def decode():
            kda_decode_step(qd, kd, vd, gd, bd, S, o=od)

        dms, _ = time_launches(decode, ksteps, args.warmup, stream)
        dbytes = 256 * 96 * (2 * 128 * 128 * 4 + 5 * 128 * 2 + 2)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        result["decode"] = {
            "workload": DECODE_WORKLOAD, "value": round(256 / (dms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(dms, 5),
            "roofline": {"bound": "hbm", "achieved": round(dgbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(dgbs / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("kda_decode_" + DECODE_WORKLOAD),
                         "kernel": "kda_decode_d128", "algorithmic_bytes_per_launch": dbytes},
        }
        if not args.no_output_gate:
            _, dz, dw = (t.to(dev) for t in inputs.make_output_gate_inputs(256, 96, 128, "bf16",
                                                                            seed=62))
            dy = torch.empty_like(od)

            def decode_gated():
                kda_decode_step_gated(qd, kd, vd, gd, bd, S, dz, dw, 1e-6, o=od, y=dy)

            gdms, _ = time_launches(decode_gated, ksteps, args.warmup, stream)
            gdbytes = dbytes + 256 * 96 * 128 * 2 * 2 + 128 * 4   # + gate in, y out, gain
            result["decode"]["gated"] = {
                "ms_per_step": round(gdms, 5), "value": round(256 / (gdms * 1e-3), 1),
                "unit": "tokens/s", "overhead_vs_decode": round(gdms / dms - 1.0, 4),
                "roofline": {"bound": "hbm",
                             "achieved": round(gdbytes / (gdms * 1e-3) / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gdbytes / (gdms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": recorded_traffic(
                                 "kda_decode_step_gated_decode_N256_H96_d128_bf16"),
                             "kernel": "kda_decode_d128 (gated)",
                             "algorithmic_bytes_per_launch": gdbytes},
            }
            # the whole mixer's decode step in one launch (input stage, decode, output stage)
            # against the input-stage kernel followed by the gated decode
            if not args.no_frontend:
                from linear_attention_recurrence_08_amd import kda_decode_step_layer
                fr = inputs.make_frontend_inputs([1] * 256, 96, 128, 128, "bf16", seed=653,
                                                 with_state=True).to(dev)
                ones = torch.arange(257, dtype=torch.int32, device=dev)
                taps = (fr.w_q, fr.w_k, fr.w_v, fr.z_bias, fr.A)
                xs = (fr.x_q, fr.x_k, fr.x_v, fr.x_z, fr.x_b)

                def decode_layer():
                    kda_decode_step_layer(*xs, *taps, fr.conv_in, S, dz, dw, y=dy)

                def decode_three():
                    q5 = kda_frontend(*xs, *taps, cu_seqlens=ones, conv_in=fr.conv_in,
                                      conv_out=fr.conv_in)[:5]
                    kda_decode_step_gated(*q5, S, dz, dw, 1e-6, o=od, y=dy)

                lms, _ = time_launches(decode_layer, ksteps, args.warmup, stream)
                l3ms, _ = time_launches(decode_three, ksteps, args.warmup, stream)
                lbytes = decode_layer_bytes(256, 96)
                result["decode"]["layer"] = {
                    "entry": "kda_decode_step_layer", "ms_per_step": round(lms, 5),
                    "value": round(256 / (lms * 1e-3), 1), "unit": "tokens/s",
                    "three_kernel_ms_per_step": round(l3ms, 5),
                    "vs_three_kernels": round(l3ms / lms, 3),
                    "roofline": {"bound": "hbm",
                                 "achieved": round(lbytes / (lms * 1e-3) / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(lbytes / (lms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "traffic": recorded_traffic(
                                     "kda_decode_step_layer_decode_N256_H96_d128_bf16"),
                                 "kernel": "kda_decode_d128 (input and output stages)",
                                 "algorithmic_bytes_per_launch": lbytes},
                }
                del fr, ones, taps, xs
            del dz, dw, dy
        # the whole mixer's serving step for a small batch, eager and as a replayed HIP graph
        if not args.no_output_gate and not args.no_frontend:
            result["decode"]["serving_graph"] = serving_step_graph(dev, stream, ksteps)
        del qd, kd, vd, gd, bd, S, od
        torch.cuda.empty_cache()

    # ---------------- CPU baseline: the float64 oracle on the host cores ----------------
    if not args.no_cpu_baseline and x.num_seqs >= 1:
        import oracle
        oracle.build(force=False)
        to64 = lambda t: t.detach().cpu().double().numpy()
        # bounded sample: the first sequence, heads [0, nh) (all 96 heads of the 4096-token
        # prefill is ~30 s of single-core work)
        nh = min(x.H, 96)
        a, e = x.seq_bounds()[0]
        e = min(e, a + 4096)
        sl = slice(a, e)
        h0 = None if x.h0 is None else to64(x.h0[0:1, :nh])
        cores = oracle.default_threads()
        print(f"[bench] cpu baseline: oracle on tokens [{a},{e}) x {nh} heads, {cores} threads",
              file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        o_ref, _ = oracle.recurrence(to64(x.q[sl, :nh]), to64(x.k[sl, :nh]), to64(x.v[sl, :nh]),
                                     to64(x.g[sl, :nh]), to64(x.beta[sl, :nh]), h0,
                                     [0, e - a], nthreads=cores)
        cpu_s = time.perf_counter() - t0
        toks = e - a
        cpu_value = toks * nh / x.H / cpu_s  # tokens/s of full-width (all-head) layers
        result["cpu_baseline"] = {
            "value": round(cpu_value, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{args.workload}: sequence 0 tokens [{a},{e}), heads 0..{nh - 1} of "
                      f"{x.H}; float64 token loop; {cpu_s:.2f} s wall",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
        }
        if x.h0 is None and a == 0 and e == x.seq_bounds()[0][1]:
            o_gpu = to64(o.reshape(x.total_tokens, x.H, x.dv)[sl, :nh])
            result["parity_sample"] = {
                "max_norm_err_o": float(np.abs(o_gpu - o_ref).max() / np.abs(o_ref).max()),
                "heads": nh, "tokens": toks}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
