"""Summaries of rocprofv3 output for the profiles/ folder, and the HBM traffic figure
that bench.py reports beside its roofline.

    python -m exact_io_aware_20_amd.profile_summary trace  <trace_dir> <out.md> <warmup_launches> <command>
    python -m exact_io_aware_20_amd.profile_summary traffic <fetch_dir> <write_dir> <out.md> <calib_mib> <command>
    python -m exact_io_aware_20_amd.profile_summary mfma <pmc_dir> <out.md> <command>
    python -m exact_io_aware_20_amd.profile_summary states <pmc_dir> <out.md> <command>
    python -m exact_io_aware_20_amd.profile_summary lds <pmc_dir> <out.md> <command>
    python -m exact_io_aware_20_amd.profile_summary valu <pmc_dir> <out.md> <command>

`trace` turns a `--kernel-trace --stats` run into a table of per-kernel launch
counts and durations.  `traffic` reads two `--pmc` runs (FETCH_SIZE, then
WRITE_SIZE, both in KiB per dispatch) of `bench.py --calib-copy-mib M`, which also
launches one plain streaming kernel of known size (an elementwise negation of M MiB
of fp32 into another M MiB buffer).  Each counter is scaled by the ratio of that
kernel's true bytes to what the same counter reads for it, and the per-launch HBM
bytes of every attention kernel are written with a digest of the kernel sources;
bench.py uses the figure only while the sources still match the digest.  `mfma`
reads a `--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` run and reports the share
of SIMD cycles each attention kernel kept the matrix pipe busy.  `states` reads a
run of the wave-state counters (STATE_COUNTERS) and splits each kernel's wave time
into issuing, waiting at s_waitcnt or a barrier, and waiting for an issue slot or a
dependency.  `lds` reads a run of LDS_COUNTERS and reports how busy the LDS was and
the bytes per clock per CU it delivered to LDS loads.  `valu` reads a run of
VALU_COUNTERS and reports the share of each kernel's SIMD cycles that issuing its
vector instructions takes (the secondary roofline of the softmax work).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_fwd_tile.hpp", "fa_common.hpp",
                  "fa_launch.hpp")
TRAFFIC_TAG = "traffic-json:"


def code_text(src: str) -> str:
    """The source with comments removed and whitespace collapsed, so that edits to
    comments alone leave the digest (and the profiles it guards) valid."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "csrc", name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code_text(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    """'void fa::fa_bwd_dkdv_kernel<128>(fa::BwdParams)' -> 'fa_bwd_dkdv_kernel<128>'."""
    k = kernel.split("(")[0]
    k = re.sub(r"^void ", "", k)
    return k.replace("fa::", "")


def _find(pattern_dir: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {pattern_dir}")
    return sorted(hits)[0]


def trace_table(trace_dir: str) -> list[dict]:
    rows = []
    with open(_find(trace_dir, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def timed_means(trace_dir: str, skip: int) -> dict[str, tuple[int, float]]:
    """Per kernel: (launches kept, mean duration in us) over its dispatches in launch
    order, leaving out the first `skip` of each (the untimed warm-up launches)."""
    per = defaultdict(list)
    with open(_find(trace_dir, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            per[short_name(r["Kernel_Name"])].append(
                (int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    out = {}
    for k, v in per.items():
        kept = [d for _, d in sorted(v)[skip:]]
        if kept:
            out[k] = (len(kept), sum(kept) / len(kept))
    return out


def counter_means(pmc_dir: str, counter: str) -> dict[str, float]:
    """Mean value of `counter` per dispatch for each kernel name."""
    vals = defaultdict(list)
    with open(_find(pmc_dir, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def calibration(means: dict[str, float]) -> tuple[str, float]:
    hits = [(k, v) for k, v in means.items() if "neg_kernel" in k]
    if len(hits) != 1:
        raise RuntimeError("expected exactly one calibration (negation) kernel in the counter run")
    return hits[0]


def traffic(fetch_dir: str, write_dir: str, calib_mib: int) -> dict:
    fetch = counter_means(fetch_dir, "FETCH_SIZE")
    write = counter_means(write_dir, "WRITE_SIZE")
    calib_bytes = calib_mib * 2**20
    cname, cf = calibration(fetch)
    _, cw = calibration(write)
    f_scale = calib_bytes / (cf * 1024.0)
    w_scale = calib_bytes / (cw * 1024.0)
    out = {}
    for k in fetch:
        if "fa_" not in k:
            continue
        f_kib, w_kib = fetch[k], write.get(k, 0.0)
        out[short_name(k)] = {"fetch_kib": f_kib, "write_kib": w_kib,
                              "bytes": f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale}
    return {"calib_kernel": short_name(cname), "calib_mib": calib_mib, "fetch_scale": f_scale,
            "write_scale": w_scale, "kernels": out, "source_digest": source_digest()}


def committed_traffic(md_path: str, kernel: str):
    """HBM bytes per launch of `kernel` from a committed traffic summary, or None when
    the file is missing or the kernel sources changed since the counters were taken."""
    if not os.path.exists(md_path):
        return None
    with open(md_path) as f:
        for line in f:
            if line.startswith(TRAFFIC_TAG):
                data = json.loads(line[len(TRAFFIC_TAG):])
                if data.get("source_digest") != source_digest():
                    return None
                k = data["kernels"].get(kernel)
                return None if k is None else k["bytes"]
    return None


def _write_trace_md(rows, timed, skip, out, command):
    lines = [f"# Kernel trace: {os.path.splitext(os.path.basename(out))[0].replace('kernel_trace_', '')}", "",
             "Command (run from the repository root; `$R` is the repository path):", "",
             f"    {command}", "",
             f"Kernel sources digest: `{source_digest()}`.  `avg` is rocprofv3's own statistic over all "
             f"launches; `timed avg` leaves out each kernel's first {skip} (warm-up) launches, the "
             "figure comparable with bench.py's event timing of the timed steps.", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share | timed avg (us) |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        t = timed.get(r["kernel"])
        ta = f"{t[1]:.1f} (n={t[0]})" if t else "-"
        lines.append(f"| {r['kernel']} | {r['calls']} | {r['avg_us']:.1f} | {r['min_us']:.1f} | "
                     f"{r['max_us']:.1f} | {r['pct']:.1f} % | {ta} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _write_traffic_md(t, out, command):
    lines = [f"# HBM traffic per launch: {os.path.splitext(os.path.basename(out))[0].replace('hbm_traffic_', '')}", "",
             "Two counter runs of the same command, one with `--pmc FETCH_SIZE`, one with",
             "`--pmc WRITE_SIZE` (run from the repository root; `$R` is the repository path):", "",
             f"    {command}", "",
             f"Calibration: `{t['calib_kernel']}` streams {t['calib_mib']} MiB in and {t['calib_mib']} MiB out; "
             f"true bytes / counter bytes = {t['fetch_scale']:.3f} (FETCH_SIZE), {t['write_scale']:.3f} (WRITE_SIZE).",
             "", "| kernel | FETCH_SIZE (KiB/dispatch) | WRITE_SIZE (KiB/dispatch) | calibrated HBM bytes / launch |",
             "|---|---|---|---|"]
    for k, v in sorted(t["kernels"].items()):
        lines.append(f"| {k} | {v['fetch_kib']:.4g} | {v['write_kib']:.4g} | {v['bytes'] / 1e6:.1f} MB |")
    lines += ["", f"Kernel sources digest: `{t['source_digest']}` (bench.py reports the figure only "
              "while the sources match).", "", TRAFFIC_TAG + " " + json.dumps(t)]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
MFMA_TAG = "mfma-json:"


def gpu_agent(pmc_dir: str) -> dict:
    """SIMD count and XCD count of the GPU agent of a rocprofv3 run (its agent_info.csv);
    MI355X's figures (1024 SIMDs, 8 XCDs) when the file has no GPU row."""
    try:
        with open(_find(pmc_dir, "agent_info.csv")) as f:
            for r in csv.DictReader(f):
                if int(r.get("Simd_Count", "0") or 0) > 0:
                    return {"simds": int(r["Simd_Count"]), "xcc": max(1, int(r.get("Num_Xcc", "1") or 1))}
    except FileNotFoundError:
        pass
    return {"simds": 1024, "xcc": 8}


def mean_durations(trace_dir: str) -> dict[str, float]:
    """Mean dispatch duration (ns) per kernel from a kernel_trace.csv, or {} if none."""
    try:
        path = _find(trace_dir, "kernel_trace.csv")
    except FileNotFoundError:
        return {}
    per = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            per[short_name(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: sum(v) / len(v) for k, v in per.items() if v}


def mfma_busy(pmc_dir: str) -> dict:
    """Per attention kernel: the means per dispatch of SQ_VALU_MFMA_BUSY_CYCLES (summed
    over every SIMD) and GRBM_GUI_ACTIVE (GPU-busy cycles of the dispatch, which the
    profiler sums over the XCDs, each having its own counter), and the share of SIMD
    cycles the matrix pipe was busy: busy / (active / XCDs x SIMDs).  When the run also
    traced the kernels (--kernel-trace), the shader clock the kernel ran at follows as
    (active / XCDs) / mean duration."""
    agent = gpu_agent(pmc_dir)
    busy = counter_means(pmc_dir, MFMA_COUNTERS[0])
    active = counter_means(pmc_dir, MFMA_COUNTERS[1])
    dur = mean_durations(pmc_dir)
    out = {}
    for k, b in busy.items():
        if "fa_" not in k or k not in active or active[k] <= 0:
            continue
        cycles = active[k] / agent["xcc"]
        v = {"mfma_busy": b, "gui_active": active[k], "frac": b / (cycles * agent["simds"])}
        d = dur.get(short_name(k))
        if d:
            v["duration_us"] = d / 1e3
            v["clock_mhz"] = cycles / d * 1e3
        out[short_name(k)] = v
    return {"agent": agent, "kernels": out, "source_digest": source_digest()}


def _write_mfma_md(m, out, command):
    a = m["agent"]
    lines = [f"# MFMA busy: {os.path.splitext(os.path.basename(out))[0].replace('mfma_busy_', '')}", "",
             "One counter run (run from the repository root; `$R` is the repository path):", "",
             f"    {command}", "",
             f"`frac` = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {a['xcc']} XCDs x {a['simds']} SIMDs): the "
             "share of SIMD cycles in which the matrix pipe was busy during the kernel (means per dispatch; "
             "the profiler sums GRBM_GUI_ACTIVE over the XCDs). It counts executed MFMAs, so for dQ it "
             "includes the recomputed S and dP contractions, and it is measured against the clock the "
             f"kernel ran at, not the 2.4 GHz of the published peak. Kernel sources digest: `{source_digest()}`.",
             "`clock` = (GRBM_GUI_ACTIVE / XCDs) / mean dispatch duration of the same run (the shader clock "
             "under this kernel's load). Only dispatches of a millisecond or more give a usable figure: for "
             "shorter ones the counter also covers cycles outside the traced duration, and the quotient "
             "exceeds the 2.4 GHz maximum.",
             "", "| kernel | SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE | frac | duration (us) | clock (MHz) |",
             "|---|---|---|---|---|---|"]
    for k, v in sorted(m["kernels"].items()):
        dur = f"{v['duration_us']:.1f}" if "duration_us" in v else "-"
        clk = f"{v['clock_mhz']:.0f}" if "clock_mhz" in v else "-"
        lines.append(f"| {k} | {v['mfma_busy']:.4g} | {v['gui_active']:.4g} | {v['frac']:.3f} | {dur} | {clk} |")
    lines += ["", MFMA_TAG + " " + json.dumps(m)]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def committed_mfma(md_path: str, kernel: str):
    """The MFMA-busy figures (and clock) of `kernel` from a committed summary, or None
    when the file is missing or the kernel sources changed since."""
    if not os.path.exists(md_path):
        return None
    with open(md_path) as f:
        for line in f:
            if line.startswith(MFMA_TAG):
                data = json.loads(line[len(MFMA_TAG):])
                if data.get("source_digest") != source_digest():
                    return None
                return data["kernels"].get(kernel)
    return None


STATE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                  "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_MISC")
LDS_COUNTERS = ("SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_LDS_BANK_CONFLICT",
                "SQ_LDS_DATA_FIFO_FULL", "GRBM_GUI_ACTIVE")


def _kernel_counters(pmc_dir: str, counters) -> dict[str, dict[str, float]]:
    """Per attention kernel (short name): the mean per dispatch of every counter."""
    means = {c: counter_means(pmc_dir, c) for c in counters}
    out = {}
    for k in means[counters[0]]:
        if "fa_" in k and all(k in means[c] for c in counters):
            out[short_name(k)] = {c: means[c][k] for c in counters}
    return out


def wave_states(pmc_dir: str) -> dict:
    """Shares of SQ_WAVE_CYCLES (wave-resident time summed over waves): a wave is
    issuing (SQ_ACTIVE_INST_ANY), waiting at s_waitcnt or a barrier (SQ_WAIT_ANY), or
    ready but not issued for a dependency or a busy pipe (SQ_WAIT_INST_ANY); the three
    add up to about 1.  The VALU, LDS and misc rows are parts of the issuing share."""
    out = {}
    for k, v in _kernel_counters(pmc_dir, STATE_COUNTERS).items():
        w = v["SQ_WAVE_CYCLES"]
        if w > 0:
            out[k] = {c: v[c] / w for c in STATE_COUNTERS[1:]}
    return out


def lds_use(pmc_dir: str) -> dict:
    """LDS busy share SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / XCDs x CUs) (the
    profiler sums GRBM_GUI_ACTIVE over the XCDs; four SIMDs per CU) and the bytes per
    clock per CU that LDS loads returned (SQ_INSTS_LDS_LOAD_BANDWIDTH counts 64-byte
    units)."""
    agent = gpu_agent(pmc_dir)
    cus = agent["simds"] // 4
    out = {}
    for k, v in _kernel_counters(pmc_dir, LDS_COUNTERS).items():
        cycles = v["GRBM_GUI_ACTIVE"] / agent["xcc"]
        if cycles <= 0:
            continue
        out[k] = {"busy": v["SQ_LDS_IDX_ACTIVE"] / (cycles * cus),
                  "load_bytes_per_clk_cu": 64.0 * v["SQ_INSTS_LDS_LOAD_BANDWIDTH"] / (cycles * cus),
                  "bank_conflict": v["SQ_LDS_BANK_CONFLICT"],
                  "fifo_full": v["SQ_LDS_DATA_FIFO_FULL"] / (cycles * cus)}
    return {"agent": agent, "kernels": out}


def _write_states_md(m, out, command):
    name = os.path.splitext(os.path.basename(out))[0].replace("wave_states_", "")
    lines = [f"# Wave states: {name}", "", "One counter run (run from the repository root; `$R` is the repository path):",
             "", f"    {command}", "",
             "Shares of SQ_WAVE_CYCLES (means per dispatch): `issuing` = SQ_ACTIVE_INST_ANY, `waitcnt/barrier` = "
             "SQ_WAIT_ANY, `not issued` = SQ_WAIT_INST_ANY (ready, held by a dependency or a busy pipe); the "
             "VALU, LDS and misc columns are parts of the issuing share, `LDS wait` of the not-issued share. "
             f"Kernel sources digest: `{source_digest()}`.", "",
             "| kernel | issuing | waitcnt/barrier | not issued | VALU | LDS | LDS wait | misc |",
             "|---|---|---|---|---|---|---|---|"]
    for k, v in sorted(m.items()):
        lines.append(f"| {k} | {v['SQ_ACTIVE_INST_ANY']:.3f} | {v['SQ_WAIT_ANY']:.3f} | {v['SQ_WAIT_INST_ANY']:.3f} | "
                     f"{v['SQ_ACTIVE_INST_VALU']:.3f} | {v['SQ_ACTIVE_INST_LDS']:.3f} | {v['SQ_WAIT_INST_LDS']:.3f} | "
                     f"{v['SQ_ACTIVE_INST_MISC']:.3f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _write_lds_md(m, out, command):
    a = m["agent"]
    name = os.path.splitext(os.path.basename(out))[0].replace("lds_use_", "")
    lines = [f"# LDS use: {name}", "", "One counter run (run from the repository root; `$R` is the repository path):",
             "", f"    {command}", "",
             f"`busy` = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / {a['xcc']} XCDs x {a['simds'] // 4} CUs); `B/clk/CU` = "
             "64 x SQ_INSTS_LDS_LOAD_BANDWIDTH over the same cycles, the bytes LDS loads returned; `fifo full` = "
             "SQ_LDS_DATA_FIFO_FULL over the same cycles (means per dispatch). "
             f"Kernel sources digest: `{source_digest()}`.", "",
             "| kernel | busy | B/clk/CU | bank conflict cycles | fifo full |", "|---|---|---|---|---|"]
    for k, v in sorted(m["kernels"].items()):
        lines.append(f"| {k} | {v['busy']:.3f} | {v['load_bytes_per_clk_cu']:.1f} | {v['bank_conflict']:.4g} | "
                     f"{v['fifo_full']:.3f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


VALU_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU",
                 "GRBM_GUI_ACTIVE")
VALU_TAG = "valu-json:"
# Issue cycles of one wave64 vector instruction on its SIMD (16 lanes, four passes) and of
# one v_exp_f32 (measured back to back on gfx950 with a throughput probe: about 10).
VALU_ISSUE_CYCLES = 4.0
TRANS_ISSUE_CYCLES = 10.0


def valu_load(pmc_dir: str) -> dict:
    """Per attention kernel (means per dispatch): vector instructions other than MFMA,
    the transcendental ones among them, MFMAs, and the share of the kernel's SIMD cycles
    that issuing the vector instructions alone takes at the issue costs above:
    (other x 4 + transcendental x 10) / (GRBM_GUI_ACTIVE / XCDs x SIMDs).  A share near 1
    means the kernel is bound by vector issue, whatever its matrix work."""
    agent = gpu_agent(pmc_dir)
    out = {}
    for k, v in _kernel_counters(pmc_dir, VALU_COUNTERS).items():
        cycles = v["GRBM_GUI_ACTIVE"] / agent["xcc"]
        if cycles <= 0:
            continue
        vec = v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"]
        trans = v["SQ_INSTS_VALU_TRANS_F32"]
        need = ((vec - trans) * VALU_ISSUE_CYCLES + trans * TRANS_ISSUE_CYCLES) / agent["simds"]
        out[k] = {"valu": vec, "trans": trans, "mfma": v["SQ_INSTS_MFMA"], "cycles": cycles,
                  "valu_issue_frac": need / cycles, "valu_per_mfma": vec / max(1.0, v["SQ_INSTS_MFMA"])}
    return {"agent": agent, "kernels": out, "source_digest": source_digest()}


def _write_valu_md(m, out, command):
    a = m["agent"]
    name = os.path.splitext(os.path.basename(out))[0].replace("valu_load_", "")
    lines = [f"# Vector-ALU load: {name}", "", "One counter run (run from the repository root; `$R` is the repository path):",
             "", f"    {command}", "",
             "Means per dispatch. `vector` = SQ_INSTS_VALU - SQ_INSTS_MFMA (wave instructions), `exp` = "
             f"SQ_INSTS_VALU_TRANS_F32; `issue share` = (non-exp x {VALU_ISSUE_CYCLES:g} + exp x "
             f"{TRANS_ISSUE_CYCLES:g} cycles) / (GRBM_GUI_ACTIVE / {a['xcc']} XCDs x {a['simds']} SIMDs), the share "
             "of the kernel's SIMD cycles that issuing its vector instructions alone takes (the secondary, "
             f"vector-ALU roofline). Kernel sources digest: `{m['source_digest']}`.", "",
             "| kernel | vector | exp | MFMA | vector per MFMA | issue share |", "|---|---|---|---|---|---|"]
    for k, v in sorted(m["kernels"].items()):
        lines.append(f"| {k} | {v['valu']:.4g} | {v['trans']:.4g} | {v['mfma']:.4g} | {v['valu_per_mfma']:.2f} | "
                     f"{v['valu_issue_frac']:.3f} |")
    lines += ["", VALU_TAG + " " + json.dumps(m)]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def committed_valu(md_path: str, kernel: str):
    """The vector-ALU figures of `kernel` from a committed summary, or None when the file
    is missing or the kernel sources changed since the counters were taken."""
    if not os.path.exists(md_path):
        return None
    with open(md_path) as f:
        for line in f:
            if line.startswith(VALU_TAG):
                data = json.loads(line[len(VALU_TAG):])
                if data.get("source_digest") != source_digest():
                    return None
                return data["kernels"].get(kernel)
    return None


def main(argv):
    if len(argv) >= 5 and argv[0] == "trace":
        skip = int(argv[3])
        _write_trace_md(trace_table(argv[1]), timed_means(argv[1], skip), skip, argv[2], argv[4])
    elif len(argv) >= 6 and argv[0] == "traffic":
        _write_traffic_md(traffic(argv[1], argv[2], int(argv[4])), argv[3], argv[5])
    elif len(argv) >= 4 and argv[0] == "mfma":
        _write_mfma_md(mfma_busy(argv[1]), argv[2], argv[3])
    elif len(argv) >= 4 and argv[0] == "states":
        _write_states_md(wave_states(argv[1]), argv[2], argv[3])
    elif len(argv) >= 4 and argv[0] == "lds":
        _write_lds_md(lds_use(argv[1]), argv[2], argv[3])
    elif len(argv) >= 4 and argv[0] == "valu":
        _write_valu_md(valu_load(argv[1]), argv[2], argv[3])
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
