"""Host-side logic of bench.py (no GPU): the one-GPU contract, per-kernel source digests and the
rocprofv3 summaries it writes from counter CSVs."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_source_digests_are_per_kernel():
    tags = ["kda_chunk_fwd_prefill_T4096_H96_d128_bf16", "kda_decode_decode_N256_H96_d128_bf16",
            "kda_decode_step_gated_decode_N256_H96_d128_bf16",
            "kda_output_gate_T4096_H96_d128_bf16", "kda_frontend_T4096_H96_d128_bf16"]
    d = {t: bench.kernel_source_digest(t) for t in tags}
    # the gated decode is the decode kernel; the others are distinct sources
    assert d[tags[1]] == d[tags[2]]
    assert len({d[tags[0]], d[tags[1]], d[tags[3]], d[tags[4]]}) == 4
    assert all(len(v) == 16 for v in d.values())


def _write_counters(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summaries_scale_by_the_copy_and_add_kernels_of_a_call(tmp_path, monkeypatch):
    # counters in KiB per dispatch: the 1 GiB calibration copy reads 2 GiB worth of FETCH_SIZE
    # (factor 2) and 1 GiB of WRITE_SIZE (factor 1); the input stage's two kernels are summed
    gib_kib = (1 << 30) / 1024.0
    conv = "void kda::(anonymous namespace)::kda_frontend_conv_kernel<unsigned short, true>(x)"
    state = "void kda::(anonymous namespace)::kda_frontend_state_kernel<unsigned short>(x)"
    fetch = [{"Kernel_Name": "elementwise_kernel", "Counter_Name": "FETCH_SIZE",
              "Counter_Value": 2 * gib_kib}]
    fetch += [{"Kernel_Name": conv, "Counter_Name": "FETCH_SIZE", "Counter_Value": 2000.0}] * 3
    fetch += [{"Kernel_Name": state, "Counter_Name": "FETCH_SIZE", "Counter_Value": 20.0}] * 3
    write = [{"Kernel_Name": "elementwise_kernel", "Counter_Name": "WRITE_SIZE",
              "Counter_Value": gib_kib}]
    write += [{"Kernel_Name": conv, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0}] * 3
    write += [{"Kernel_Name": state, "Counter_Name": "WRITE_SIZE", "Counter_Value": 5.0}] * 3
    _write_counters(str(tmp_path / "f" / "fetch_counter_collection.csv"), fetch)
    _write_counters(str(tmp_path / "w" / "write_counter_collection.csv"), write)
    out = tmp_path / "repo"
    (out / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(out))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda tag: "0123456789abcdef")
    bench.summarize([str(tmp_path / "f"), str(tmp_path / "w")], "test command")
    txt = open(out / "profiles" / "kda_frontend_T4096_H96_d128_bf16_hbm_traffic.md").read()
    want = (2000.0 + 20.0) * 1024 / 2 + (500.0 + 5.0) * 1024 / 1
    line = [l for l in txt.splitlines() if l.startswith("hbm_bytes_per_launch:")][0]
    assert float(line.split(":")[1]) == pytest.approx(want, rel=1e-5)
    assert "command: `test command`" in txt
    # a summary is used only while its digest matches the current sources
    assert bench.recorded_traffic("kda_frontend_T4096_H96_d128_bf16") == pytest.approx(
        want, rel=1e-5)
    monkeypatch.setattr(bench, "kernel_source_digest", lambda tag: "fedcba9876543210")
    assert bench.recorded_traffic("kda_frontend_T4096_H96_d128_bf16") is None


def test_split_digest_covers_both_sources():
    # the split's digest changes with the prefill kernel and with its completion kernels
    d_split = bench.kernel_source_digest("kda_chunk_fwd_split_T4096_H12_d128_bf16")
    d_prefill = bench.kernel_source_digest("kda_chunk_fwd_prefill_T4096_H96_d128_bf16")
    assert len(d_split) == 16 and d_split != d_prefill


def test_split_summary_lists_every_kernel_of_the_call(tmp_path, monkeypatch):
    trace = tmp_path / "t" / "split_kernel_stats.csv"
    trace.parent.mkdir(parents=True)
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        for name, ns in (("void kda::(anonymous namespace)::kda_prefill_mfma_kernel<2, 64>"
                          "(kda::PrefillArgs)", 64000.0),
                         ("kda::(anonymous namespace)::kda_split_fixup_kernel(kda::PrefillArgs)",
                          17000.0),
                         ("kda::(anonymous namespace)::kda_split_compose_kernel"
                          "(kda::PrefillArgs)", 15000.0),
                         ("__amd_rocclr_copyBuffer", 3000.0)):
            w.writerow({"Name": name, "Calls": 23, "AverageNs": ns, "MinNs": ns, "MaxNs": ns})
    out = tmp_path / "repo"
    (out / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(out))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda tag: "0123456789abcdef")
    bench.summarize_split(str(tmp_path / "t"), "split command")
    txt = open(out / "profiles" / "kda_chunk_fwd_split_T4096_H12_d128_bf16_kernel_trace.md").read()
    rows = [l for l in txt.splitlines() if l.startswith("| kda_")]
    assert [r.split("|")[1].strip() for r in rows] == [
        "kda_prefill_mfma_kernel<2, 64>", "kda_split_fixup_kernel", "kda_split_compose_kernel"]
    assert "command: `split command`" in txt and "source_digest: 0123456789abcdef" in txt


def test_cpu_model_is_read():
    m = bench._cpu_model()
    assert isinstance(m, str) and m


def test_trace_summary_keeps_its_workloads_dispatches(tmp_path, monkeypatch):
    """A kernel that other timed entries launch at other sizes in the same run (the decode at 4
    sequences in the serving step) is summarised from its own workload's dispatches only, told
    apart by the grid."""
    name = "void kda::(anonymous namespace)::kda_decode_d128_kernel<unsigned short, 2, true, true>(x)"
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs",
                                          "TotalDurationNs"])
        w.writeheader()
        w.writerow({"Name": name, "Calls": 4, "AverageNs": 300, "MinNs": 10, "MaxNs": 600,
                    "TotalDurationNs": 1200})
    big = bench.SUMMARY_GRIDS[name.split("::")[-1].split("(")[0]]
    with open(d / "t_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp",
                                          "Grid_Size_X", "Grid_Size_Y"])
        w.writeheader()
        for start, dur, grid in ((0, 500, big), (1000, 600, big), (2000, 10, (49152, 1)),
                                 (3000, 90, (49152, 1))):
            w.writerow({"Kernel_Name": name, "Start_Timestamp": start,
                        "End_Timestamp": start + dur, "Grid_Size_X": grid[0],
                        "Grid_Size_Y": grid[1]})
    out = tmp_path / "repo"
    (out / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(out))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda tag: "0123456789abcdef")
    bench.summarize([str(d)], "test command")
    txt = open(out / "profiles" /
               "kda_decode_step_layer_decode_N256_H96_d128_bf16_kernel_trace.md").read()
    row = [l for l in txt.splitlines() if l.startswith("| kda_decode_d128_kernel")][0]
    assert [c.strip() for c in row.split("|")[2:7]] == ["2", "550", "500", "600", "1100"]


@pytest.mark.parametrize("wl,wgs,periods", [
    # one sequence of 256 tiles, 96 heads in two 64-column halves
    ("prefill_T4096_H96_d128_bf16", 192, 260.0),
    # 16 sequences x 96 heads, one 128-column workgroup each; each walks its own tile count
    # (rounded up to even) plus 4 periods
    ("varlen_16seq_H96_d128_bf16", 1536, None)])
def test_sq_summary_counts_each_workgroups_periods(tmp_path, monkeypatch, wl, wgs, periods):
    from linear_attention_recurrence_08_amd import inputs
    w = inputs.WORKLOADS[wl]
    lens = (inputs.varlen_lengths(w["seed"], w["n_seqs"]) if w["kind"] == "varlen"
            else w["seq_lens"])
    halves = wgs // (len(lens) * w["H"])
    total = halves * w["H"] * sum((n + 15) // 16 + ((n + 15) // 16) % 2 + 4 for n in lens)
    if periods is not None:
        assert total / wgs == periods
    # every wave lives 2,000 cycles per period of its workgroup (the counter counts by 4)
    counters = {"SQ_WAVES": 12 * wgs, "SQ_WAVE_CYCLES": 12 * total * 2000 / 4}
    for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS",
              "SQ_INSTS_SALU", "SQ_INSTS_VMEM", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
              "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_VALU_MFMA_BUSY_CYCLES",
              "SQ_LDS_BANK_CONFLICT"):
        counters[k] = 4 * total   # one per SIMD and period
    d = tmp_path / "c"
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, v in counters.items():
            wr.writerow({"Kernel_Name": "void kda::kda_prefill_mfma_kernel<1, 64, false>()",
                         "Counter_Name": k, "Counter_Value": v})
    out = tmp_path / "repo"
    (out / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(out))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda tag: "0123456789abcdef")
    bench.summarize_sq([str(d)], "sq command", wl)
    txt = open(out / "profiles" / f"kda_chunk_fwd_{wl}_sq_counters.md").read()
    assert f"{wgs} workgroups" in txt and f"{total / wgs:.1f} pipeline periods" in txt
    assert "a period of 2000 cycles" in txt
    assert "| SQ_INSTS_VALU | " in txt and "| 1.0 |" in txt
