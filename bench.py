#!/usr/bin/env python3
"""Throughput benchmark of the chunked gated delta rule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the whole hot path over one batch: the chained forward over the
pipeline chunks of the sequence (boundary state passed forward, Eq. 5 of the
StateFlow page) followed by the chained backward (state gradient passed
backward, Eq. 7).  The default workload is a 262,144-token sequence, 16 heads,
d_k = d_v = 128, bf16, split into 8 chunks by the hybrid-cost plan
c_i(alpha = 0.5) of Eq. 9 (a = 1, b = 0.25, literal token units).  Inputs are
synthetic and resident in HBM before timing starts.

The timed region replays one captured step as a HIP graph K times (every
launch of the step; the host's launch gaps removed); --eager times the
launches themselves.  Per-kernel times come from HIP events recorded around
every launch on its stream during K eager steps with the same inputs.

Prints one JSON line with the metric, a roofline for the dominant kernel and
for the whole path, and the fp64 CPU oracle timed on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "tokens/sec chunked GDN fwd+bwd (H=16,d=128,1 GPU); % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 MFMA / vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

C = 64  # kernel block
DEFAULT_WORKLOAD = "fwdbwd_h16_t262144_d128_8skew"


def kernel_flops_per_block(name, d):
    """Algorithmic MFMA flops per 64-token block of one head, per kernel:
    the sum of the matrix products the kernel's step of the method needs
    (2 m n k each)."""
    g = lambda m, n, k: 2.0 * m * n * k
    pre = g(C, C, d) + g(C, C, d) + g(C, d, C) + g(C, d, C)   # K K^T, (Q K^T), W, U
    if name in ("gdn_fwd_out", "gdn_fwd_out_save"):
        return pre + g(C, d, d) + g(C, d, d) + g(C, d, C) + g(d, d, C)   # Vn, QS^T, P Vn, S'
    if name in ("gdn_fwd_summary", "gdn_bwd_summary"):
        return (pre - g(C, C, d)) + g(C, d, d) + g(d, d, C) + g(C, d, d) + g(d, d, C)  # + M
    if name == "gdn_fwd_states":
        return (pre - g(C, C, d)) + g(C, d, d) + g(d, d, C)
    if name in ("gdn_bwd_dscan", "gdn_bwd_dscan_summary"):
        return (pre - g(C, d, C)) + g(d, d, C) + g(C, d, C) + g(C, d, d) + g(d, d, C)
    if name == "gdn_bwd_grads":
        return (g(C, C, d) + g(C, C, d)                # K K^T, Q K^T (Vn from the forward)
                + g(C, d, C) + g(C, d, d)              # dVn
                + g(C, d, C) + g(C, C, d)              # dV, dP
                + g(C, d, d) + g(C, d, C) + g(C, d, C)  # dQ, dK1
                + 2 * g(C, d, d)                       # dW, dK2
                + 2 * g(C, C, d)                       # dTp, dTpp
                + 2 * g(C, C, C)                       # dA = -T^T dT T^T
                + g(C, C, d) + 3 * g(C, d, C))         # kk, dK4 (two), dK3
    return None


def kernel_bytes_per_token_head(name, d, elem=2):
    """Algorithmic HBM bytes per token and head of the kernels that move the
    method's own inputs and outputs (bf16 activations, fp32 gates): the
    gradient kernel reads q, k, v, dO, alpha, beta and writes dq, dk, dv,
    dalpha, dbeta; the output kernel reads q, k, v, alpha, beta and writes o.
    Intermediate buffers of this design (Tp, Tpp, maps, per-block states) are
    not counted.  None for kernels that only move intermediates."""
    if name == "gdn_bwd_grads":
        return 7 * d * elem + 16
    if name in ("gdn_fwd_out", "gdn_fwd_out_save"):
        return 4 * d * elem + 8
    return None


def kernel_flops_per_launch(name, d, H, T, L, P, save=False):
    """Algorithmic flops of one launch for one chunk of T tokens (``save``:
    the saving forward, whose summary covers every segment)."""
    nblk = (T + C - 1) // C
    if name in ("gdn_chain_fwd", "gdn_chain_bwd"):
        return H * max(P - 1, 0) * 2.0 * d * d * d
    per = kernel_flops_per_block(name, d)
    if per is None:
        return None
    if name == "gdn_fwd_summary":      # segments 0 .. P-2, or all when saving
        return H * (nblk if save else min(nblk, (P - 1) * L)) * per
    if name == "gdn_bwd_dscan_summary":
        return H * max(nblk - min(L, nblk), 0) * per
    return H * nblk * per


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "linear_recurrence_chunked_gated_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, wl_name=None):
    """HBM bytes per launch of `kernel` in workload wl_name (the benchmark
    workload when None) recorded from rocprofv3 counter runs
    (profiles/traffic.json), or None when absent or taken on other sources."""
    p = os.path.join(HERE, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    if wl_name is not None and wl_name != DEFAULT_WORKLOAD:
        rec = rec.get("workloads", {}).get(wl_name, {})
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def _read_counter_csv(path):
    """Per-kernel mean of a rocprofv3 counter over dispatches: {kernel: value}."""
    import csv
    sums, counts = {}, {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or row.get("KernelName")
            val = row.get("Counter_Value") or row.get("Counter-Value")
            if name is None or val is None:
                continue
            disp = row.get("Dispatch_Id") or row.get("Dispatch-Id") or str(len(counts))
            key = (name, disp)
            sums[key] = sums.get(key, 0.0) + float(val)   # sum over counter instances
    per = {}
    for (name, _), v in sums.items():
        per.setdefault(name, []).append(v)
    return {n: sum(v) / len(v) for n, v in per.items()}


def kernel_label(name):
    """The library's launch label of a kernel as a profiler names it
    (demangled or mangled), or None for other kernels."""
    import re
    m = re.search(r"((?:gdn|conv)_\w+?)_kernel", name)
    if not m:
        return None
    base = m.group(1)
    d = re.search(r"_kernel<([^<>]*)>", name)
    if d:
        last = d.group(1).split(",")[-1].strip()
    else:
        mm = re.search(r"L[ib](\d+)EEE", name)
        last = mm.group(1) if mm else ""
    if base == "gdn_fwd_summary2":  # two-blocks-in-flight form
        return "gdn_fwd_summary"
    if base in ("gdn_fwd_out", "gdn_fwd_out2"):  # one- and two-blocks-in-flight forms
        return {"0": "gdn_fwd_out", "1": "gdn_fwd_states", "2": "gdn_fwd_out_save"}.get(
            last, "gdn_fwd_out")
    if base in ("gdn_bwd_dscan", "gdn_bwd_dscan2"):
        return "gdn_bwd_dscan" if last in ("1", "true") else "gdn_bwd_dscan_summary"
    if base == "gdn_chain":
        return "gdn_chain_bwd" if last in ("1", "true") else "gdn_chain_fwd"
    return base


def write_traffic(fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, calib_bytes,
                  wl_name=None, stats_csv=None):
    """HBM bytes per launch of every library kernel of workload wl_name (the
    benchmark workload when None) from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain device
    copy of calib_bytes, into profiles/traffic.json and a table under
    profiles/ (with each kernel's achieved rate when the kernel-trace
    statistics of the same workload are given)."""
    wl_name = wl_name or DEFAULT_WORKLOAD
    fetch = _read_counter_csv(fetch_csv)
    write = _read_counter_csv(write_csv)
    cf = _read_counter_csv(calib_fetch_csv)
    cw = _read_counter_csv(calib_write_csv)
    copy_f = max(cf.values())
    copy_w = max(cw.values())
    sf = calib_bytes / (copy_f * 1024.0)
    sw = calib_bytes / (copy_w * 1024.0)
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        short = kernel_label(name)
        if short is None:
            continue
        fb = fetch.get(name, 0.0) * 1024.0 * sf
        wb = write.get(name, 0.0) * 1024.0 * sw
        kernels[short] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    calib = {"copy_bytes_each_way": calib_bytes, "fetch_kib_per_copy": copy_f,
             "write_kib_per_copy": copy_w, "fetch_scale": sf, "write_scale": sw}
    path = os.path.join(HERE, "profiles", "traffic.json")
    rec = {}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        rec = {"source_hash": source_hash()}
    if wl_name == DEFAULT_WORKLOAD:
        rec["calibration"] = calib
        rec["kernels"] = kernels
    else:
        rec.setdefault("workloads", {})[wl_name] = {"calibration": calib, "kernels": kernels}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    stats = _read_stats_csv(stats_csv) if stats_csv else None
    _write_traffic_md(kernels, calib, rec["source_hash"], wl_name, stats,
                      [fetch_csv, write_csv, calib_fetch_csv, calib_write_csv] +
                      ([stats_csv] if stats_csv else []))


# Bytes per 64-token block that a kernel moves of the method's own tensors
# (q, k, v, dO in; o, dq, dk, dv out; the gates), bf16 activations at width d,
# counted every time a kernel moves them.  Everything else a kernel moves is
# this design's intermediates (Tpp, per-block states, V^new, dS', the
# segment maps).
def method_bytes_per_block(name, d, elem=2):
    tile, gates = C * d * elem, C * 4
    return {"gdn_prep": tile + 2 * gates,                       # k; alpha, beta
            "gdn_fwd_summary": 2 * tile + 2 * gates,            # k, v
            "gdn_fwd_out_save": 4 * tile + 2 * gates,           # q, k, v; o
            "gdn_fwd_out": 4 * tile + 2 * gates,
            "gdn_bwd_dscan_summary": 3 * tile + 2 * gates,      # q, k, dO
            "gdn_bwd_dscan": 3 * tile + 2 * gates,
            "gdn_bwd_grads": 7 * tile + 4 * gates,              # q, k, v, dO; dq, dk, dv; gates
            }.get(name, 0)


def _traffic_blocks(wl_name):
    """Blocks (of 64 tokens, one head) that one launch of each kernel covers in
    workload wl_name, averaged over its chunks, and the number of chunks."""
    from linear_recurrence_chunked_gated_amd import _lib
    import torch
    wl = workload(wl_name)
    H, d, chunks, save = wl["H"], wl["D"], wl["chunks"], wl["bwd"]
    nch = len(chunks)
    blocks = {}
    for n in chunks:
        L, P = _lib.segment_plan(_lib.make_shape(1, n, H, d, d, torch.bfloat16, 0))
        nb = (n + C - 1) // C
        last = nb - (P - 1) * L  # blocks of the last segment
        per = {"gdn_prep": nb, "gdn_bwd_dscan": nb, "gdn_bwd_grads": nb,
               "gdn_fwd_out_save" if save else "gdn_fwd_out": nb,
               # the saving forward maps every segment, the plain one all but the last
               "gdn_fwd_summary": nb if save else (nb - last if P > 1 else 0),
               # the reverse maps skip the first segment
               "gdn_bwd_dscan_summary": max(nb - min(L, nb), 0)}
        for k, v in per.items():
            if k.startswith("gdn_bwd") and not wl["bwd"]:
                continue
            blocks[k] = blocks.get(k, 0) + H * v / nch
    return blocks, nch


def _write_traffic_md(kernels, calib, src_hash, wl_name, stats, csvs):
    """The traffic table of a workload: per launch, the counters' bytes split
    into the method's tensors and this design's intermediates, the achieved
    rate (when kernel times are given), and per step (one launch of each
    kernel per chunk)."""
    wl = workload(wl_name)
    H, d, bwd = wl["H"], wl["D"], wl["bwd"]
    blocks, nch = _traffic_blocks(wl_name)
    by_th = 2840 if bwd else 1032  # algorithmic bytes per token-head (bf16, d = 128)
    rows, tot_step, meth_step = [], 0.0, 0.0
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["bytes_per_launch"]):
        m = method_bytes_per_block(k, d) * blocks.get(k, 0)
        t = v["bytes_per_launch"]
        tot_step += t * nch
        meth_step += m * nch
        rate = ""
        if stats and k in stats:
            rate = " | %.1f | %.2f" % (stats[k], t / (stats[k] * 1e-6) / 1e12)
        elif stats:
            rate = " | | "
        rows.append("| %s | %.1f | %.1f | %.1f | %.1f | %.1f%s | %.2f |" % (
            k, v["fetch_bytes"] / 1e6, v["write_bytes"] / 1e6, t / 1e6, m / 1e6, (t - m) / 1e6,
            rate, t * nch / 1e9))
    algo = wl["T"] * H * by_th
    wl_arg = "" if wl_name == DEFAULT_WORKLOAD else " --workload " + wl_name
    tag = "fwdbwd" if bwd else "fwd"
    cmds = ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/tr_%s_fetch -o fetch -- "
            "python -u bench.py%s --steps 1 --warmup 1 --no-cpu-baseline" % (tag, wl_arg),
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/tr_%s_write -o write -- "
            "python -u bench.py%s --steps 1 --warmup 1 --no-cpu-baseline" % (tag, wl_arg),
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/tr_cfetch -o tr_cfetch -- "
            "python -u bench.py --copy-calibration",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/tr_cwrite -o tr_cwrite -- "
            "python -u bench.py --copy-calibration",
            "python bench.py --write-traffic " + " ".join(csvs[:4]) + " " + wl_name
            + (" " + csvs[4] if len(csvs) > 4 else "")]
    head = ("| kernel | fetch (MB) | write (MB) | total (MB) | method tensors (MB) | "
            "intermediates (MB) |" + (" avg (us) | TB/s |" if stats else "") + " per step (GB) |")
    sep = "|---|---:|---:|---:|---:|---:|" + ("---:|---:|" if stats else "") + "---:|"
    text = ["# HBM traffic per launch: %s" % wl["desc"],
            "", "Commands (run from the repository root on one MI355X, with `TMPDIR=/tmp`), one "
            "counter per pass:", "", "```"] + cmds + ["```", "",
            "Calibration: a plain 1 GiB device copy (torch `copy_`) reads FETCH_SIZE = %.0f KiB and "
            "WRITE_SIZE = %.0f KiB, so fetch counts are scaled by %.4f and write counts by %.4f."
            % (calib["fetch_kib_per_copy"], calib["write_kib_per_copy"], calib["fetch_scale"],
               calib["write_scale"]),
            "", "Bytes are per launch, averaged over every launch of the run (the warm-up step, the "
            "captured step's replays and the eager step, over every chunk size). \"method "
            "tensors\" is what a kernel moves of q, k, v, dO, o, dq, dk, dv and the gates, counted "
            "each time a kernel moves them (`method_bytes_per_block` in `bench.py`, times the "
            "blocks one launch covers); \"intermediates\" is the rest: this design's Tpp, per-block "
            "states, V^new, state gradients and segment maps (and any re-read)."
            + (" \"avg\" is the kernel's average duration in the kernel trace of the same "
               "workload (the `--stats` summary given last on the `--write-traffic` line) and "
               "TB/s the counted bytes over it; a plain device copy reaches 4.7-5.4 TB/s on this "
               "part." if stats else "")
            + " `profiles/traffic.json` holds the same bytes with the hash of the kernel sources "
            "they were taken on; `bench.py` reports `roofline.traffic` only while that hash "
            "matches.", "", head, sep] + rows + ["",
            "Per step: %.2f GB, of which %.2f GB are the method's tensors and %.2f GB intermediates, "
            "against %.2f GB of algorithmic bytes (each tensor moved once: %s B per token-head); "
            "%.2fx." % (tot_step / 1e9, meth_step / 1e9, (tot_step - meth_step) / 1e9, algo / 1e9,
                        "{:,}".format(by_th), tot_step / algo), "", "Source hash: `%s`." % src_hash]
    path = os.path.join(HERE, "profiles", "traffic_%s.md" % wl_file_tag(wl_name))
    with open(path, "w") as f:
        f.write("\n".join(text) + "\n")


def _read_stats_csv(path):
    """{launch label: average duration in us} from a rocprofv3 --stats kernel
    table (one row per kernel name)."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Name") or row.get("KernelName") or row.get("Kernel_Name")
            avg = row.get("AverageNs") or row.get("Average_Ns") or row.get("AverageNS")
            lab = kernel_label(name or "")
            if lab is None or avg is None:
                continue
            calls = float(row.get("Calls", 1))
            tot, n = out.get(lab, (0.0, 0.0))
            out[lab] = (tot + float(avg) * calls, n + calls)
    return {k: t / n / 1e3 for k, (t, n) in out.items()}


def write_counters(out_md, stats_csv, pmc_csvs, title, commands, cus=256, simds=1024,
                   xcds=8):
    """Per-kernel hardware-counter table from rocprofv3 --pmc runs (counter
    values summed over a dispatch's instances, averaged over the dispatches
    of a kernel) and the average durations of a --kernel-trace --stats run:
      bf16 TFLOP/s     SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 / duration
      MFMA busy        SQ_VALU_MFMA_BUSY_CYCLES / (active cycles * SIMDs)
      LDS active       SQ_LDS_IDX_ACTIVE / (active cycles * CUs)
      bank conflict    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
    with active cycles = GRBM_GUI_ACTIVE / XCDs (the counter is per XCD)."""
    dur = _read_stats_csv(stats_csv)
    vals = {}
    import csv
    for path in pmc_csvs:
        sums = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name") or row.get("Kernel-Name") or row.get("KernelName")
                ctr = row.get("Counter_Name") or row.get("Counter-Name")
                val = row.get("Counter_Value") or row.get("Counter-Value")
                disp = row.get("Dispatch_Id") or row.get("Dispatch-Id")
                lab = kernel_label(name or "")
                if lab is None or ctr is None or val is None:
                    continue
                key = (lab, disp, ctr)
                sums[key] = sums.get(key, 0.0) + float(val)
        per = {}
        for (lab, _, ctr), v in sums.items():
            per.setdefault((lab, ctr), []).append(v)
        for (lab, ctr), v in per.items():
            vals.setdefault(lab, {})[ctr] = sum(v) / len(v)
    rows = []
    for lab in sorted(vals, key=lambda k: -dur.get(k, 0.0)):
        c = vals[lab]
        d_us = dur.get(lab)
        act = c.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        tf = mops * 512 / (d_us * 1e-6) / 1e12 if (mops is not None and d_us) else None
        mb = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        lds = c.get("SQ_LDS_IDX_ACTIVE")
        bc = c.get("SQ_LDS_BANK_CONFLICT")
        fmt = lambda x, f: "" if x is None else f % x
        rows.append("| %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            lab, fmt(d_us, "%.1f"), fmt(mops and mops * 512 / 1e9, "%.1f"), fmt(tf, "%.0f"),
            fmt(tf and tf / PEAK_BF16_TFLOPS * 100, "%.1f%%"),
            fmt(mb and act and mb / (act * simds) * 100, "%.1f%%"),
            fmt(lds and act and lds / (act * cus) * 100, "%.1f%%"),
            fmt(bc is not None and lds and bc / lds * 100, "%.1f%%"),
            fmt(c.get("SQ_INSTS_LDS"), "%.3g")))
    text = ["# " + title, "",
            "Commands (run from the repository root on one MI355X, with `TMPDIR=/tmp`):", "",
            "```"] + commands + ["```", "",
            "Counter values are summed over a dispatch's instances and averaged over the dispatches "
            "of a kernel; durations are the averages of the kernel-trace run. bf16 GFLOP = "
            "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (executed matrix-core work, padding included); "
            "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d x %d SIMDs); LDS active = "
            "SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / %d x %d CUs); bank conflict = "
            "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (share of LDS-active cycles stalled on bank "
            "conflicts)." % (xcds, simds, xcds, cus), "",
            "| kernel | avg (us) | bf16 GFLOP / launch | bf16 TFLOP/s | of 2.5 PF | MFMA busy | "
            "LDS active | bank conflict | LDS instr / launch |",
            "|---|---:|---:|---:|---:|---:|---:|---:|---:|"] + rows
    with open(out_md, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def copy_calibration(nbytes=1 << 30, reps=4):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": nbytes, "reps": reps}))


def wl_file_tag(name):
    """The workload part of a profile's file name."""
    return "fwdbwd_h16_t262144_d128" if name == DEFAULT_WORKLOAD else name


def workload(name):
    from linear_recurrence_chunked_gated_amd.plan import chunk_lengths
    if name == "fwdbwd_h16_t262144_d128_8skew":
        T = 262144
        return dict(T=T, H=16, D=128, chunks=chunk_lengths(T, 8, 0.5), bwd=True, s_in_std=None,
                    seed=20260004,
                    desc="T=262144, H=16, d=128, bf16, 8 chunks by c_i(0.5) of Eq. 9 "
                         "(a=1, b=0.25, token units), chained fwd then bwd")
    if name == "fwdbwd_h16_t16384_d128":
        return dict(T=16384, H=16, D=128, chunks=[16384], bwd=True, s_in_std=None, seed=20260003,
                    desc="T=16384, H=16, d=128, bf16, one chunk fwd+bwd")
    if name == "fwd_h16_t8192_d128_8x1024":
        return dict(T=8192, H=16, D=128, chunks=[1024] * 8, bwd=False, s_in_std=None,
                    seed=20260001,
                    desc="T=8192, H=16, d=128, bf16, 8 chunks of 1024 chained, fwd only "
                         "(launch-bound)")
    if name == "fwd_h16_t65536_d128":
        return dict(T=65536, H=16, D=128, chunks=[65536], bwd=False, s_in_std=0.1, seed=20260102,
                    desc="T=65536, H=16, d=128, bf16, one chunk fwd, S_in ~ N(0, 0.1)")
    if name == "fwd_h32_t65536_d128":
        return dict(T=65536, H=32, D=128, chunks=[65536], bwd=False, s_in_std=0.1, seed=20260002,
                    desc="T=65536, H=32, d=128, bf16, one chunk fwd, S_in ~ N(0, 0.1)")
    raise SystemExit("unknown workload %r" % name)


def measured_peaks(dev):
    """What this GPU delivers in practice, for the fractions beside the
    datasheet ones: a plain 1 GiB device-to-device copy (bytes read plus
    bytes written over its duration) and a dense 8192^3 bf16 matrix product
    through torch (2 m n k flop over its duration)."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    m = 8192
    x = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    y = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(x, y), 10)
    del x, y
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": round(2 * n / t_copy / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2.0 * m * m * m / t_mm / 1e12, 1),
            "how": "1 GiB device copy (read + write bytes); 8192^3 bf16 torch.matmul"}


def bench_conv(args):
    """The short causal convolution (the chunk's auxiliary local-convolution
    state) over q, k and v of a GDN layer: C = 3 * H * d channels, width 4,
    SiLU, chained through the 8 skewed chunks of the main workload, forward
    then backward.  Bound by HBM: per token, the forward reads x and writes y,
    the backward reads x and dy and writes dx (bf16 each)."""
    import torch
    from linear_recurrence_chunked_gated_amd import _lib
    from linear_recurrence_chunked_gated_amd.inputs import conv_inputs
    from linear_recurrence_chunked_gated_amd.plan import chunk_lengths
    T, H, D, W = 262144, 16, 128, 4
    C = 3 * H * D
    chunks = chunk_lengths(T, 8, 0.5)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = conv_inputs(1, T, C, W, "bf16", seed=20260104, state_std=None, grads=True, device=dev)
    x, w, dy = d["x"], d["w"], d["dy"]
    bounds = [0]
    for n in chunks:
        bounds.append(bounds[-1] + n)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    states = [None] + [torch.empty(1, W - 1, C, dtype=x.dtype, device=dev) for _ in chunks]
    gst = [torch.empty(1, W - 1, C, dtype=x.dtype, device=dev) for _ in range(len(chunks) + 1)]
    dws = [torch.empty_like(w) for _ in chunks]
    wsb = _lib.alloc_workspace(max(_lib.shortconv_bwd_workspace_bytes(
        _lib.conv_shape(1, n, C, W, x.dtype, 1)) for n in chunks), dev)
    stream = torch.cuda.current_stream()

    def step():
        stream = torch.cuda.current_stream()
        for i in range(len(chunks)):
            sl = slice(bounds[i], bounds[i + 1])
            _lib.shortconv_fwd(x[:, sl], w, states[i], 1, y=y[:, sl], conv_out=states[i + 1],
                               stream=stream)
        g = None
        for i in range(len(chunks) - 1, -1, -1):
            sl = slice(bounds[i], bounds[i + 1])
            _, _, g = _lib.shortconv_bwd(x[:, sl], w, states[i], dy[:, sl], g, 1, dx=dx[:, sl],
                                         dw=dws[i], workspace=wsb, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with _lib.profile(capacity=64 * args.steps * len(chunks) + 64) as prof:
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kern = {n: {"avg_us": tot / k * 1e3, "ms_per_step": tot / args.steps, "launches": k}
            for n, (k, tot) in prof.results.items()}
    dom = max(kern, key=lambda n: kern[n]["ms_per_step"])
    per_tok = {"conv_fwd": 4 * C, "conv_bwd": 6 * C}
    by = per_tok[dom] * T / len(chunks)  # average chunk
    achieved = by / (kern[dom]["avg_us"] * 1e-6) / 1e9
    Bytes = 10 * C * T
    t_roof = Bytes / (PEAK_HBM_GBS * 1e9)
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        from linear_recurrence_chunked_gated_amd.inputs import as_f64
        oracle.build(force=False)
        hd = conv_inputs(1, T, C, W, "bf16", seed=20260104, state_std=None, grads=True)
        n, el = 16, 0.0
        while True:
            xs, dys = as_f64(hd["x"][:, :n]), as_f64(hd["dy"][:, :n])
            ws = as_f64(hd["w"])
            t0 = time.perf_counter()
            oracle.shortconv_fwd(xs, ws, None, 1)
            oracle.shortconv_bwd(xs, ws, None, dys, None, 1)
            el = time.perf_counter() - t0
            if el >= 5.0 or 2 * n > T:
                break
            n *= 2
        cpu = {"value": round(n / el, 1), "unit": "tokens/s", "cores": 1,
               "nproc": os.cpu_count(), "kind": "oracle",
               "sample": "first %d tokens x %d channels of the workload, one chunk, fwd+bwd, "
                         "fp64 loop (%.1f s)" % (n, C, el)}
    line = {
        "metric": "tokens/sec short causal conv fwd+bwd over q,k,v (H=16,d=128,W=4,1 GPU); "
                  "% HBM roofline",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": 1, "T": T, "C": C, "W": W, "act": "silu",
                   "chunks": chunks, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": load_traffic(dom),
                     "bytes_per_launch": by},
        "path_roofline": {"bound": "hbm", "t_roof_ms": round(t_roof * 1e3, 4),
                          "t_step_ms": round(ms, 4), "frac": round(t_roof / (ms * 1e-3), 4),
                          "algorithmic_bytes": Bytes},
        "kernels": {n: {"avg_us": round(v["avg_us"], 2),
                        "launches_per_step": v["launches"] // args.steps,
                        "ms_per_step": round(v["ms_per_step"], 4)} for n, v in kern.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, seconds_target=7.0):
    """The fp64 oracle on a bounded sample: the first n tokens of the same
    sequence (all heads), one chunk forward and backward (or forward only)."""
    import numpy as np
    import oracle
    from linear_recurrence_chunked_gated_amd.inputs import gdn_inputs, as_f64
    oracle.build(force=False)
    H, D = wl["H"], wl["D"]
    n = 256
    while True:
        d = gdn_inputs(1, n, H, D, D, dtype="bf16", seed=wl["seed"], s_in_std=wl["s_in_std"],
                       grads=wl["bwd"], device="cpu")
        args = [as_f64(d[k]) for k in ("q", "k", "v", "alpha", "beta")] + [as_f64(d["S_in"])]
        t0 = time.perf_counter()
        _, _, nt = oracle.gdn_fwd(*args, return_threads=True)
        if wl["bwd"]:
            oracle.gdn_bwd(*args, as_f64(d["dO"]), as_f64(d["dS_out"]))
        dt = time.perf_counter() - t0
        if dt >= seconds_target or 2 * n > wl["T"]:
            break
        n *= 2
    return {"value": n / dt, "unit": "tokens/s", "cores": int(nt), "nproc": os.cpu_count(),
            "kind": "oracle",
            "sample": "first %d tokens x %d heads of the workload's sequence, one chunk, %s, "
                      "fp64 token loop (%.1f s)" % (n, H, "fwd+bwd" if wl["bwd"] else "fwd", dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="fwdbwd_h16_t262144_d128_8skew (default), fwdbwd_h16_t16384_d128, "
                         "fwd_h16_t65536_d128, fwd_h32_t65536_d128, fwd_h16_t8192_d128_8x1024, or "
                         "conv_qkv_h16_t262144_d128_8skew (the short convolution)")
    ap.add_argument("--seg-blocks", type=int, default=0)
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB scratch buffer before every timed step (outside the "
                         "timed events) so that no input is served from the last-level cache")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of one step captured as a HIP "
                         "graph (the default; per-kernel times always come from an eager pass)")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the copy and GEMM measurements of the achievable peaks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--recompute", action="store_true",
                    help="backward recomputes the forward's block states instead of reading the "
                         "saving forward's buffer")
    ap.add_argument("--overlap", action="store_true",
                    help="split-and-overlap: each chunk's state-independent launches run on a "
                         "second stream beside the previous chunk's chain (saved backward)")
    ap.add_argument("--split-fraction", type=float, default=None, metavar="F",
                    help="cut every chunk at fraction F into two parts run as chunks (with "
                         "--overlap: part b's state-independent launches beside part a's chain)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (for rocprofv3 counter scaling) and exit")
    ap.add_argument("--write-counters", nargs="+", metavar="ARG",
                    help="OUT_MD TITLE STATS_CSV PMC_CSV... [CMD COMMAND...]: per-kernel counter "
                         "table from rocprofv3 runs")
    ap.add_argument("--write-traffic", nargs="+", metavar="ARG",
                    help="FETCH_CSV WRITE_CSV CALIB_FETCH_CSV CALIB_WRITE_CSV [WORKLOAD "
                         "[STATS_CSV]]: turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs into "
                         "profiles/traffic.json and a table under profiles/")
    args = ap.parse_args()
    if args.write_traffic:
        a = args.write_traffic
        if len(a) not in (4, 5, 6):
            ap.error("--write-traffic takes 4 to 6 arguments")
        write_traffic(*a[:4], calib_bytes=1 << 30, wl_name=a[4] if len(a) > 4 else None,
                      stats_csv=a[5] if len(a) > 5 else None)
        return
    if args.write_counters:
        a = args.write_counters
        cmds = []
        if "CMD" in a:
            i = a.index("CMD")
            a, cmds = a[:i], a[i + 1:]
        write_counters(a[0], a[2], a[3:], a[1], cmds)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU; runs on several GPUs are not implemented "
              "(the chunk path shards by heads with no exchange, or along the sequence with one "
              "boundary-state exchange per chunk)", file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("conv_"):
        bench_conv(args)
        return

    import torch
    import linear_recurrence_chunked_gated_amd as gdn
    from linear_recurrence_chunked_gated_amd import _lib
    from linear_recurrence_chunked_gated_amd.inputs import gdn_inputs

    wl = workload(args.workload)
    T, H, D, chunks = wl["T"], wl["H"], wl["D"], wl["chunks"]
    plan_chunks = chunks
    if args.split_fraction:
        # the page's split at fraction f: every chunk runs as two parts
        from linear_recurrence_chunked_gated_amd.chain import split_lengths
        chunks = split_lengths(chunks, args.split_fraction)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = gdn_inputs(1, T, H, D, D, dtype="bf16", seed=wl["seed"], s_in_std=wl["s_in_std"],
                   grads=wl["bwd"], device=dev)
    q, k, v, al, be = d["q"], d["k"], d["v"], d["alpha"], d["beta"]
    bounds = [0]
    for n in chunks:
        bounds.append(bounds[-1] + n)
    # Preallocated outputs, boundary states and workspaces.
    o = torch.empty_like(v)
    states = [d["S_in"] if d["S_in"] is not None else torch.zeros(1, H, D, D, device=dev)]
    states += [torch.empty(1, H, D, D, device=dev) for _ in chunks]
    ws_f = max(_lib.workspace_bytes(_lib.make_shape(1, n, H, D, D, q.dtype, args.seg_blocks))
               for n in chunks)
    wsf = _lib.alloc_workspace(ws_f, dev)
    if wl["bwd"]:
        dO, dS_out = d["dO"], d["dS_out"]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dal, dbe = torch.empty_like(al), torch.empty_like(be)
        gst = [torch.empty(1, H, D, D, device=dev) for _ in range(len(chunks) + 1)]
        ws_b = max(_lib.workspace_bytes(_lib.make_shape(1, n, H, D, D, q.dtype, args.seg_blocks),
                                        backward=True) for n in chunks)
        wsb = _lib.alloc_workspace(ws_b, dev)
    save = wl["bwd"] and not args.recompute
    saved = [None] * len(chunks)
    if save:
        saved = [_lib.alloc_workspace(_lib.saved_bytes(_lib.make_shape(1, n, H, D, D, q.dtype,
                                                                       args.seg_blocks)), dev)
                 for n in chunks]
    stream = torch.cuda.current_stream()
    overlap = args.overlap and (save or not wl["bwd"])
    if overlap:
        from linear_recurrence_chunked_gated_amd import chain as gchain
        side = torch.cuda.Stream(device=dev)
        wsf2 = [wsf, _lib.alloc_workspace(ws_f, dev)]
        wsb2 = [wsb, _lib.alloc_workspace(ws_b, dev)] if wl["bwd"] else None

    def step_overlap():
        stream = torch.cuda.current_stream()  # the capture stream when graph-replayed
        gchain.chain_fwd(q, k, v, al, be, states[0], chunks, o=o, seg_blocks=args.seg_blocks,
                         stream=stream, save=save, overlap=True, side_stream=side,
                         workspaces=wsf2, saved=saved if save else None, states=states)
        if wl["bwd"]:
            gchain.chain_bwd(q, k, v, al, be, dO, dS_out, chunks, None,
                             grads=(dq, dk, dv, dal, dbe), seg_blocks=args.seg_blocks,
                             stream=stream, saved=saved, overlap=True, side_stream=side,
                             workspaces=wsb2, state_grads=gst[:len(chunks)])

    def step():
        if overlap:
            return step_overlap()
        stream = torch.cuda.current_stream()  # the capture stream under --graph
        for i in range(len(chunks)):
            sl = slice(bounds[i], bounds[i + 1])
            _lib.chunk_fwd(q[:, sl], k[:, sl], v[:, sl], al[:, sl], be[:, sl], states[i],
                           o=o[:, sl], S_out=states[i + 1], seg_blocks=args.seg_blocks,
                           workspace=wsf, stream=stream, saved=saved[i])
        if wl["bwd"]:
            G = dS_out
            for i in range(len(chunks) - 1, -1, -1):
                sl = slice(bounds[i], bounds[i + 1])
                _lib.chunk_bwd(q[:, sl], k[:, sl], v[:, sl], al[:, sl], be[:, sl],
                               None if save else states[i],
                               dO[:, sl], G, grads=(dq[:, sl], dk[:, sl], dv[:, sl], dal[:, sl],
                                                    dbe[:, sl], gst[i]),
                               seg_blocks=args.seg_blocks, workspace=wsb, stream=stream,
                               saved=saved[i])
                G = gst[i]

    # The timed region replays one captured step (every launch of the step,
    # none skipped) unless launches are to be timed one by one, the step spans
    # two streams (--overlap; captured, it measured slower than the plain
    # captured step) or a cache flush sits between steps (--cold).
    use_graph = not (args.eager or overlap or args.cold)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall_graph = time.perf_counter() - wall0
        ms_graph = e0.elapsed_time(e1) / args.steps
    if args.cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    with _lib.profile(capacity=256 * args.steps * len(chunks) + 64) as prof:
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        if args.cold:
            for i in range(args.steps):
                scratch.fill_(i & 255)
                ev[i][0].record(stream)
                step()
                ev[i][1].record(stream)
        else:
            e0.record(stream)
            for _ in range(args.steps):
                step()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    if args.cold:
        ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    elif graph is not None:
        ms, wall = ms_graph, wall_graph  # the eager pass above only supplies per-kernel times
    else:
        ms = e0.elapsed_time(e1) / args.steps
    tok_s = T / (ms * 1e-3)

    # Per-kernel times over the eager steps (the timed region itself with --eager).
    kern = {name: {"launches": n, "avg_us": tot / n * 1e3, "total_ms_per_step": tot / args.steps}
            for name, (n, tot) in prof.results.items()}
    dom = max(kern, key=lambda n: kern[n]["total_ms_per_step"])
    # Algorithmic flops of the dominant kernel per launch (averaged over the
    # chunk sizes of one step).
    L_of = {n: _lib.segment_plan(_lib.make_shape(1, n, H, D, D, q.dtype, args.seg_blocks))
            for n in chunks}
    fl = []
    for n in chunks:
        L, P = L_of[n]
        f = kernel_flops_per_launch(dom, D, H, n, L, P, save)
        if f is None:
            fl = None
            break
        fl.append(f)
    roofline = None
    if fl:
        # The dominant kernel against whichever of its two rooflines binds:
        # algorithmic flops at the bf16 MFMA peak, or algorithmic bytes at
        # the HBM peak; the other one is reported beside it.
        dur = kern[dom]["avg_us"] * 1e-6
        per_launch = sum(fl) / len(fl)
        mfma = {"bound": "mfma", "achieved": round(per_launch / dur / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(per_launch / dur / 1e12 / PEAK_BF16_TFLOPS, 4)}
        bth = kernel_bytes_per_token_head(dom, D)
        hbm = None
        if bth is not None:
            by = bth * H * sum(chunks) / len(chunks)
            hbm = {"bound": "hbm", "achieved": round(by / dur / 1e9, 1), "peak": PEAK_HBM_GBS,
                   "unit": "GB/s", "frac": round(by / dur / 1e9 / PEAK_HBM_GBS, 4)}
        if hbm is not None and hbm["frac"] >= mfma["frac"]:
            main, other = hbm, mfma
        else:
            main, other = mfma, hbm
        roofline = dict(kernel=dom, **main, traffic=load_traffic(dom, args.workload),
                        flops_per_launch=per_launch,
                        bytes_per_launch=None if hbm is None else by, other=other)
    # Whole-path roofline: algorithmic flops and bytes per token-head of the
    # method (fwd 182,955 flop and 1,032 B; fwd+bwd 726,358 flop and 2,840 B at
    # d = 128, block 64) plus the boundary states each chunk call moves.
    fl_th = 726358.0 if wl["bwd"] else 182955.0
    by_th = 2840.0 if wl["bwd"] else 1032.0
    nst = (5 if wl["bwd"] else 2) * len(chunks) * H * D * D * 4
    F = fl_th * T * H
    Bytes = by_th * T * H + nst
    t_roof = max(F / (PEAK_BF16_TFLOPS * 1e12), Bytes / (PEAK_HBM_GBS * 1e9))
    path = {"bound": "hbm" if Bytes / (PEAK_HBM_GBS * 1e9) >= F / (PEAK_BF16_TFLOPS * 1e12) else "mfma",
            "t_roof_ms": round(t_roof * 1e3, 4), "t_step_ms": round(ms, 4),
            "frac": round(t_roof / (ms * 1e-3), 4),
            "algorithmic_flops": F, "algorithmic_bytes": Bytes}

    peaks = None if args.no_measured_peaks else measured_peaks(dev)
    if peaks and roofline:
        key = "hbm_copy_GBs" if roofline["bound"] == "hbm" else "bf16_gemm_TFLOPs"
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / peaks[key], 4)
    if peaks:
        t_meas = max(F / (peaks["bf16_gemm_TFLOPs"] * 1e12), Bytes / (peaks["hbm_copy_GBs"] * 1e9))
        path["frac_of_measured_peaks"] = round(t_meas / (ms * 1e-3), 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    line = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": wl["desc"], "B": 1, "T": T, "H": H,
                   "d_k": D, "d_v": D, "block": C, "chunks": plan_chunks,
                   "split_fraction": args.split_fraction,
                   "parts": chunks if args.split_fraction else None,
                   "seg_blocks": args.seg_blocks or "auto", "parallelism": "single GPU",
                   "backward_states": "saved by the forward" if save else
                   ("recomputed" if wl["bwd"] else None),
                   "overlap": "state-independent launches of the next chunk on a second stream"
                              if overlap else None,
                   "launch": ("one captured step replayed as a HIP graph (per-kernel times from "
                              "an eager pass)") if graph is not None else "eager"},
        "roofline": roofline,
        "path_roofline": path,
        "kernels": {n: {"avg_us": round(x["avg_us"], 2), "launches_per_step": x["launches"] // args.steps,
                        "ms_per_step": round(x["total_ms_per_step"], 4)} for n, x in kern.items()},
        "wall_s_timed": round(wall, 3),
        "cold_cache": bool(args.cold),
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
