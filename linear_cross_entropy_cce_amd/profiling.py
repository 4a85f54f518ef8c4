"""Summaries of rocprofv3 output for profiles/.

Kernel statistics (`--kernel-trace --stats`, csv):

    python -m linear_cross_entropy_cce_amd.profiling stats --dir DIR --steps K \\
        --command "..." --out profiles/<kernel>_<workload>.md

HBM traffic of the forward logit kernel: two counter passes of the same
command (`bench.py --copy-probe BYTES`), one with `--pmc FETCH_SIZE` and one
with `--pmc WRITE_SIZE`, give KiB per dispatch.  The command also runs a plain
device-to-device copy of BYTES bytes (torch's copy kernel); what the counters
read for it against the bytes it moves is the calibration factor applied to
the logit kernel's reading.

    python -m linear_cross_entropy_cce_amd.profiling traffic --fetch DIR --write DIR \\
        --copy-bytes BYTES --out profiles/<kernel>_<workload>_traffic.md

The traffic summary records a hash of the kernel's sources; `bench.py`
reports the traffic only while the sources still hash the same.

HBM traffic per step of kernels launched several times a step (the
backward's pass kernels): the same two counter passes, summed over every
dispatch of each kernel and divided by the profiled steps.

    python -m linear_cross_entropy_cce_amd.profiling steptraffic --fetch DIR --write DIR \
        --copy-bytes BYTES --steps K --kernels NAME... --title "..." --out profiles/<...>_traffic.md

Core counters of the forward logit kernel (one pass, within the per-block
limits of a single rocprofv3 run):

    rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_LDS_BANK_CONFLICT \
        SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAVES GRBM_GUI_ACTIVE --output-format csv -d DIR -o p -- CMD
    python -m linear_cross_entropy_cce_amd.profiling counters --dir DIR --command "..." \
        --out profiles/<kernel>_<workload>_counters.md

MFMA-busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x
SIMDs); GRBM_GUI_ACTIVE is summed over the XCDs, so per XCD it is the
kernel's length in GPU clock cycles and, over the dispatch's duration, the
average clock.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL = "k_fwd4"
SOURCES = ("csrc/fwd.hip", "csrc/k4.hpp", "csrc/cce_device.hpp", "csrc/cce_internal.hpp")


def _code_only(text: str) -> str:
    """The source without comments and whitespace, so that only code changes
    count (string literals in these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def sources_hash() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(PKG, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _per_dispatch(directory: str, counter: str, match) -> list[float]:
    paths = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    vals = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
                    continue
                key = (path, r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def summarize(fetch_dir: str, write_dir: str, copy_bytes: int) -> dict:
    is_kernel = lambda n: KERNEL in n  # noqa: E731
    is_copy = lambda n: "copy" in n.lower() and "cce" not in n  # noqa: E731
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        k = _per_dispatch(d, name, is_kernel)
        c = [v for v in _per_dispatch(d, name, is_copy) if v > 0]
        if not k or not c:
            raise RuntimeError(f"{name}: kernel dispatches {len(k)}, copy dispatches {len(c)}")
        kib_k = sum(k) / len(k)
        kib_c = max(c)  # the copy of copy_bytes is the largest copy dispatch
        factor = copy_bytes / (kib_c * 1024.0)
        out[name] = {"kernel_kib": kib_k, "copy_kib": kib_c, "factor": factor, "bytes": kib_k * 1024.0 * factor}
    out["traffic_bytes"] = out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]
    return out


def write_md(path: str, s: dict, copy_bytes: int, command: str, fetch_dir: str = "pmc_FETCH_SIZE",
             write_dir: str = "pmc_WRITE_SIZE") -> None:
    lines = [
        f"# HBM traffic of `{KERNEL}`: Gemma-2-2B head (N=8192, D=2304, V=256000, bf16)",
        "",
        "Commands (on the MI355X box, from the repository root; one counter per pass):",
        "",
        f"    {command.replace('COUNTER', 'FETCH_SIZE')}",
        f"    {command.replace('COUNTER', 'WRITE_SIZE')}",
        "",
        "Summarised with:",
        "",
        f"    python -m linear_cross_entropy_cce_amd.profiling traffic --fetch {fetch_dir} "
        f"--write {write_dir} --copy-bytes {copy_bytes} --out {os.path.relpath(path, os.path.dirname(PKG))}",
        "",
        f"Calibration: torch's device copy of {copy_bytes} bytes in the same run (reads and writes that many bytes).",
        "FETCH_SIZE and WRITE_SIZE count the L2's requests to the memory fabric, so reads served by the",
        "Infinity Cache (MALL) in front of HBM are included.",
        "",
        "| counter | kernel KiB / dispatch | copy KiB | factor (bytes / counted byte) | kernel bytes / launch |",
        "|---|---|---|---|---|",
    ]
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        v = s[name]
        lines.append(f"| {name} | {v['kernel_kib']:.1f} | {v['copy_kib']:.1f} | {v['factor']:.4f} | {v['bytes']:.4g} |")
    lines += [
        "",
        f"traffic_bytes_per_launch: {s['traffic_bytes']:.6g}",
        f"sources_sha256_16: {sources_hash()}",
        "",
    ]
    with open(path, "w") as f:
        f.write("\n".join(lines))


def load(path: str):
    """(bytes per launch, sources hash) from a summary written by write_md, or None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^traffic_bytes_per_launch: (\S+)$", text, re.M)
    h = re.search(r"^sources_sha256_16: (\S+)$", text, re.M)
    if not m or not h:
        return None
    return float(m.group(1)), h.group(1)


COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_LDS_BANK_CONFLICT",
            "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_WAVES", "GRBM_GUI_ACTIVE")


def _agent(directory: str) -> dict:
    for path in glob.glob(os.path.join(directory, "**", "*agent_info.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Name", "").startswith("gfx"):
                    return r
    raise FileNotFoundError(f"no GPU agent in {directory}")


def write_counters_md(path: str, directory: str, command: str, title: str,
                      kernels=(KERNEL,), counters=COUNTERS) -> dict:
    """Per-dispatch averages of one --pmc pass for each kernel whose name
    contains one of `kernels`, side by side, with the derived MFMA busy
    fraction, cycles per MFMA and average clock where the counters allow."""
    paths = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    disp = {k: {} for k in kernels}
    names = {}
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                k = next((k for k in kernels if k in r["Kernel_Name"]), None)
                if k is None:
                    continue
                names.setdefault(k, r["Kernel_Name"].split("(")[0])
                d = disp[k].setdefault((p, r["Dispatch_Id"]),
                                       {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    missing = [k for k in kernels if not disp[k]]
    if missing:
        raise RuntimeError(f"no dispatch of {missing} in {directory}")
    ag = _agent(directory)
    n_xcc, n_simd = int(ag["Num_Xcc"]), int(ag["Simd_Count"])
    res = {}
    for k in kernels:
        dd = disp[k].values()
        avg = {c: sum(d.get(c, 0.0) for d in dd) / len(dd) for c in tuple(counters) + ("ns",)}
        r = {"dispatches": len(dd), "duration_us": avg["ns"] / 1e3, "avg": avg}
        if "GRBM_GUI_ACTIVE" in counters:
            cycles = avg["GRBM_GUI_ACTIVE"] / n_xcc
            r["clock_ghz"] = cycles / avg["ns"]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
                r["mfma_busy"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * n_simd)
        if "SQ_INSTS_MFMA" in counters and "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            r["cycles_per_mfma"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / max(avg["SQ_INSTS_MFMA"], 1.0)
        if "SQ_LDS_BANK_CONFLICT" in counters and "SQ_LDS_IDX_ACTIVE" in counters:
            r["lds_conflict_frac"] = avg["SQ_LDS_BANK_CONFLICT"] / max(avg["SQ_LDS_IDX_ACTIVE"], 1.0)
        res[k] = r
    cols = " | ".join(f"`{names[k]}`" for k in kernels)
    lines = [f"# {title}", "", "Command (on the MI355X box, from the repository root):", "", f"    {command}", "",
             "Summarised with:", "",
             f"    python -m linear_cross_entropy_cce_amd.profiling counters --dir {directory} --out {path}"
             + ("" if tuple(kernels) == (KERNEL,) else " --kernels " + " ".join(kernels))
             + ("" if tuple(counters) == COUNTERS else " --counters " + " ".join(counters)), "",
             f"Agent: {ag['Name']}, {n_xcc} XCDs, {n_simd} SIMDs; dispatches averaged: "
             + ", ".join(f"{res[k]['dispatches']} of `{k}`" for k in kernels) + ".", "",
             f"| counter (average per dispatch) | {cols} |", "|---" * (len(kernels) + 1) + "|"]
    for c in counters:
        lines.append(f"| {c} | " + " | ".join(f"{res[k]['avg'][c]:.6g}" for k in kernels) + " |")
    lines += ["", f"| derived | {cols} |", "|---" * (len(kernels) + 1) + "|",
              "| dispatch duration | " + " | ".join(f"{res[k]['duration_us']:.1f} us" for k in kernels) + " |"]
    for key, label, fmt in (("cycles_per_mfma", "MFMA busy cycles per instruction", "{:.2f}"),
                            ("mfma_busy", "MFMA busy (of all SIMD cycles)", "{:.1%}"),
                            ("clock_ghz", "average GPU clock over the dispatch", "{:.2f} GHz"),
                            ("lds_conflict_frac", "LDS bank-conflict cycles / LDS active cycles", "{:.2e}")):
        if all(key in res[k] for k in kernels):
            lines.append(f"| {label} | " + " | ".join(fmt.format(res[k][key]) for k in kernels) + " |")
    lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return res


def step_traffic(fetch_dir: str, write_dir: str, copy_bytes: int, kernels, steps: int) -> dict:
    """FETCH_SIZE and WRITE_SIZE of each kernel summed over all its dispatches
    and divided by `steps`, in bytes after the copy calibration."""
    is_copy = lambda n: "copy" in n.lower() and "cce" not in n  # noqa: E731
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        c = [v for v in _per_dispatch(d, name, is_copy) if v > 0]
        if not c:
            raise RuntimeError(f"{name}: no copy dispatch for the calibration")
        factor = copy_bytes / (max(c) * 1024.0)
        for k in kernels:
            v = _per_dispatch(d, name, lambda n, k=k: k in n)
            if not v:
                raise RuntimeError(f"{name}: no dispatch of {k}")
            out.setdefault(k, {})[name] = {"dispatches": len(v), "kib": sum(v), "factor": factor,
                                           "bytes_per_step": sum(v) * 1024.0 * factor / steps}
    for k in kernels:
        out[k]["traffic_bytes_per_step"] = out[k]["FETCH_SIZE"]["bytes_per_step"] + \
            out[k]["WRITE_SIZE"]["bytes_per_step"]
    return out


def write_step_traffic_md(path: str, s: dict, copy_bytes: int, steps: int, command: str, title: str,
                          fetch_dir: str, write_dir: str) -> None:
    kernels = list(s)
    lines = [f"# {title}", "", "Commands (on the MI355X box, from the repository root; one counter per pass):", "",
             f"    {command.replace('COUNTER', 'FETCH_SIZE')}", f"    {command.replace('COUNTER', 'WRITE_SIZE')}", "",
             "Summarised with:", "",
             f"    python -m linear_cross_entropy_cce_amd.profiling steptraffic --fetch {fetch_dir} --write {write_dir} "
             f"--copy-bytes {copy_bytes} --steps {steps} --kernels {' '.join(kernels)} --out "
             f"{os.path.relpath(path, os.path.dirname(PKG))}", "",
             f"Calibration: torch's device copy of {copy_bytes} bytes in the same run.  Sums over every dispatch",
             f"of each kernel in the {steps} profiled steps, per step.", "",
             "| kernel | dispatches | FETCH bytes / step | WRITE bytes / step | total bytes / step |",
             "|---|---|---|---|---|"]
    for k in kernels:
        v = s[k]
        lines.append(f"| `{k}` | {v['FETCH_SIZE']['dispatches']} | {v['FETCH_SIZE']['bytes_per_step']:.4g} | "
                     f"{v['WRITE_SIZE']['bytes_per_step']:.4g} | {v['traffic_bytes_per_step']:.4g} |")
    lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines))


def write_stats_md(path: str, directory: str, steps: int, command: str, title: str) -> None:
    paths = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no kernel_trace.csv under {directory}")
    per = {}
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"].split("(")[0].replace("void ", "")
                per.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = sorted(per.items(), key=lambda kv: -sum(kv[1]))
    total = sum(sum(v) for _, v in rows)
    lines = [f"# {title}", "", "Command (on the MI355X box, from the repository root):", "", f"    {command}", "",
             f"{steps} profiled steps; durations from the kernel trace, microseconds.", "",
             "| kernel | calls | avg us | min us | max us | ms / step | % |", "|---|---|---|---|---|---|---|"]
    for name, v in rows:
        lines.append(f"| `{name}` | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{sum(v) / 1e3 / steps:.3f} | {100 * sum(v) / total:.1f} |")
    lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", default="rocprofv3 --pmc COUNTER --output-format csv -d pmc_COUNTER -o p "
                                         "-- python -u bench.py --steps 1 --warmup 1 --no-cpu-baseline "
                                         "--copy-probe 1073741824")
    s2 = sub.add_parser("steptraffic")
    s2.add_argument("--fetch", required=True)
    s2.add_argument("--write", required=True)
    s2.add_argument("--copy-bytes", type=int, required=True)
    s2.add_argument("--steps", type=int, required=True)
    s2.add_argument("--kernels", nargs="+", required=True)
    s2.add_argument("--title", required=True)
    s2.add_argument("--out", required=True)
    s2.add_argument("--command", required=True)
    k = sub.add_parser("stats")
    k.add_argument("--dir", required=True)
    k.add_argument("--steps", type=int, required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--dir", required=True)
    c.add_argument("--command", default="rocprofv3 --pmc " + " ".join(COUNTERS) + " --output-format csv "
                                         "-d pmc_core -o p -- python -u bench.py --steps 1 --warmup 1 "
                                         "--no-cpu-baseline")
    c.add_argument("--title", default="Core counters of `k_fwd4`: Gemma-2-2B head (N=8192, D=2304, V=256000, bf16)")
    c.add_argument("--out", required=True)
    c.add_argument("--kernels", nargs="+", default=[KERNEL], help="kernel-name substrings, one column each")
    c.add_argument("--counters", nargs="+", default=list(COUNTERS))
    a = ap.parse_args()
    if a.what == "counters":
        write_counters_md(a.out, a.dir, a.command, a.title, tuple(a.kernels), tuple(a.counters))
    elif a.what == "steptraffic":
        s = step_traffic(a.fetch, a.write, a.copy_bytes, a.kernels, a.steps)
        write_step_traffic_md(a.out, s, a.copy_bytes, a.steps, a.command, a.title, a.fetch, a.write)
    elif a.what == "traffic":
        s = summarize(a.fetch, a.write, a.copy_bytes)
        write_md(a.out, s, a.copy_bytes, a.command, a.fetch, a.write)
    else:
        write_stats_md(a.out, a.dir, a.steps, a.command, a.title)
    print(open(a.out).read())


if __name__ == "__main__":
    main()
