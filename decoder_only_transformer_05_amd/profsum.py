"""Short text summaries of rocprofv3 output, for the measurement records kept with the code.

    python -m decoder_only_transformer_05_amd.profsum stats KERNEL_STATS_CSV OUT_MD "COMMAND" "TITLE"
    python -m decoder_only_transformer_05_amd.profsum traffic OUT_JSON KERNEL \\
        FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES "COMMANDS"
    python -m decoder_only_transformer_05_amd.profsum traffic-table OUT_MD \\
        FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES "COMMANDS" [KERNEL_TABLE]

``stats`` turns a ``--kernel-trace --stats`` kernel_stats.csv into a markdown table.

``mfma`` (python -m ...profsum mfma OUT_MD COUNTER_CSV "COMMAND") turns a ``--pmc
SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_*`` run into the MFMA busy
fraction and executed MFMA work per kernel.

``traffic`` turns two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of the benchmark
(counter_collection.csv, KiB per dispatch) into HBM bytes per launch of one kernel. The
counters are scaled by what they read for a plain device copy of COPY_BYTES bytes each way
(the calibration runs of ``bench.py --copy-calibrate``), so the result is in the bytes an
exact copy would report. The source hash of the kernel's translation unit is stored with it;
the benchmark reports the figure only while the source is unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))

# translation unit (plus the headers every kernel includes) that defines each kernel
KERNEL_SOURCES = {
    "gemm_kernel": ["csrc/gemm.hip", "csrc/common.h", "csrc/kernels.h"],
    "gemm_x6_kernel": ["csrc/gemm.hip", "csrc/common.h", "csrc/kernels.h"],
    "attn_": ["csrc/attention.hip", "csrc/common.h", "csrc/kernels.h"],
}


_SIMPLE_TYPES = {"f": "float", "t": "unsigned short", "DF16_": "_Float16", "DF16b": "__bf16",
                 "i": "int", "b": "bool"}


def _template_args(m: str, i: int) -> tuple[list[str], int]:
    """Template arguments of a mangled name starting at m[i] == 'I' (the few forms the
    library's kernels use); returns them and the index past the closing 'E'."""
    assert m[i] == "I"
    i += 1
    out = []
    while m[i] != "E":
        if m.startswith("Li", i) or m.startswith("Lb", i):
            j = m.index("E", i)
            out.append(m[i + 2:j])
            i = j + 1
            continue
        for k, v in _SIMPLE_TYPES.items():
            if m.startswith(k, i):
                out.append(v)
                i += len(k)
                break
        else:
            mm = re.match(r"NS0_(\d+)", m[i:])
            if not mm:
                raise ValueError(m[i:])
            i += len(mm.group(0))
            name = m[i:i + int(mm.group(1))]
            i += int(mm.group(1))
            if m[i] == "I":
                args, i = _template_args(m, i)
                name += "<" + ",".join(args) + ">"
            assert m[i] == "E"
            i += 1
            out.append(name)
    return out, i + 1


def demangle(n: str) -> str:
    """Kernel names the profiler left mangled (it does for some _Float16 instances):
    name<args> for the forms above, else the name unchanged."""
    mm = re.match(r"_ZN4gpt212_GLOBAL__N_1(\d+)", n)
    if not mm:
        return n
    i = len(mm.group(0))
    name = n[i:i + int(mm.group(1))]
    i += int(mm.group(1))
    try:
        if i < len(n) and n[i] == "I":
            args, _ = _template_args(n, i)
            name += "<" + ",".join(args) + ">"
    except (ValueError, AssertionError, IndexError):
        return n
    return name


def short_name(n: str) -> str:
    n = demangle(n)
    n = n.replace("void ", "").replace("gpt2::(anonymous namespace)::", "")
    n = re.sub(r"\(.*", "", n)
    return n.replace("true", "1").replace("false", "0").replace(", ", ",")


def source_hash(kernel: str) -> str | None:
    for prefix, files in KERNEL_SOURCES.items():
        if kernel.startswith(prefix):
            h = hashlib.sha256()
            for f in files:
                with open(os.path.join(PKG, f), "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()
    return None


def stats_md(src: str, dst: str, command: str, title: str) -> None:
    rows = list(csv.DictReader(open(src)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    with open(dst, "w") as f:
        f.write(f"# {title}\n\nCommand (from the repository root, on one MI355X):\n\n```\n"
                f"{command}\n```\n\nSource: rocprofv3 `--kernel-trace --stats` "
                "(kernel_stats.csv), all dispatches of the run (warmup and timed steps).\n\n")
        f.write("| kernel | calls | total ms | average us | min us | max us | % |\n"
                "|---|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {short_name(r['Name'])} | {r['Calls']} | "
                    f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                    f"{float(r['Percentage']):.2f} |\n")
        f.write(f"\nTotal kernel time: {tot / 1e6:.1f} ms\n")


def counter_per_kernel(path: str, counter: str) -> dict:
    """{short kernel name: (dispatches, summed counter value)} of one counter_collection.csv."""
    out: dict = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = short_name(r["Kernel_Name"])
        n, s = out.get(k, (0, 0.0))
        out[k] = (n + 1, s + float(r["Counter_Value"]))
    return out


def copy_kib(path: str, counter: str) -> float:
    """Mean counter value of the calibration copy's dispatches (the largest kernel)."""
    per = counter_per_kernel(path, counter)
    k = max(per, key=lambda k: per[k][1] / per[k][0])
    return per[k][1] / per[k][0]


def traffic_json(dst: str, kernel: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
                 copy_write_csv: str, copy_bytes: float, command: str) -> dict:
    f = counter_per_kernel(fetch_csv, "FETCH_SIZE")[kernel]
    w = counter_per_kernel(write_csv, "WRITE_SIZE")[kernel]
    cf_kib, cw_kib = copy_kib(copy_fetch_csv, "FETCH_SIZE"), copy_kib(copy_write_csv, "WRITE_SIZE")
    scale_f, scale_w = copy_bytes / (cf_kib * 1024.0), copy_bytes / (cw_kib * 1024.0)
    fetch_b = f[1] / f[0] * 1024.0 * scale_f
    write_b = w[1] / w[0] * 1024.0 * scale_w
    rec = {"kernel": kernel, "dispatches": f[0], "fetch_bytes_per_launch": round(fetch_b),
           "write_bytes_per_launch": round(write_b),
           "bytes_per_launch": round(fetch_b) + round(write_b),
           "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": cf_kib,
                                "write_kib": cw_kib, "fetch_scale": scale_f,
                                "write_scale": scale_w},
           "source_sha256": source_hash(kernel), "command": command}
    with open(dst, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


def algorithmic_bytes(kernel_table: str) -> dict:
    """Algorithmic bytes per launch by kernel, from a `bench.py --kernel-table` file (the
    library's launch profile: each launch's bytes as the method defines them)."""
    with open(kernel_table) as fh:
        t = json.load(fh)["kernels"]
    return {k: v["bytes"] / v["launches"] for k, v in t.items() if v.get("launches")}


def _lookup(alg: dict, kernel: str):
    """The launch-profile entry of a profiler kernel name: the same name, else the name
    without its template arguments (the profile names some kernels without them)."""
    if kernel in alg:
        return alg[kernel]
    base = kernel.split("<")[0]
    return alg.get(base)


def traffic_md(dst: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
               copy_write_csv: str, copy_bytes: float, command: str,
               kernel_table: str | None = None) -> None:
    """Calibrated HBM bytes per launch of every kernel of the run, largest total first; with
    a launch-profile table, also each kernel's algorithmic bytes and the measured/algorithmic
    ratio."""
    fe = counter_per_kernel(fetch_csv, "FETCH_SIZE")
    wr = counter_per_kernel(write_csv, "WRITE_SIZE")
    sf = copy_bytes / (copy_kib(copy_fetch_csv, "FETCH_SIZE") * 1024.0)
    sw = copy_bytes / (copy_kib(copy_write_csv, "WRITE_SIZE") * 1024.0)
    alg = algorithmic_bytes(kernel_table) if kernel_table else None
    rows = []
    for k in fe:
        n, f = fe[k]
        w = wr.get(k, (n, 0.0))[1]
        rows.append((k, n, f * 1024.0 * sf / n, w * 1024.0 * sw / n))
    rows.sort(key=lambda r: -(r[2] + r[3]) * r[1])
    with open(dst, "w") as fh:
        fh.write("# HBM traffic per kernel launch (FETCH_SIZE / WRITE_SIZE, calibrated)\n\n"
                 f"Commands (from the repository root, on one MI355X):\n\n```\n{command}\n```\n\n"
                 f"Scale factors from a plain {copy_bytes / 2**30:.0f} GiB device copy: fetch x{sf:.3f}, "
                 f"write x{sw:.3f} (the counters' KiB times these give bytes).\n\n")
        if alg is None:
            fh.write("| kernel | dispatches | fetch MB/launch | write MB/launch |\n"
                     "|---|---|---|---|\n")
            for k, n, f, w in rows:
                fh.write(f"| {k} | {n} | {f / 1e6:.2f} | {w / 1e6:.2f} |\n")
            return
        fh.write("Algorithmic bytes: what the method reads and writes per launch (the library's "
                 "launch profile, `bench.py --kernel-table`); for the GEMMs and attention the "
                 "operands and results once each.\n\n"
                 "| kernel | dispatches | fetch MB/launch | write MB/launch | algorithmic MB/launch "
                 "| measured / algorithmic |\n|---|---|---|---|---|---|\n")
        for k, n, f, w in rows:
            a = _lookup(alg, k)
            extra = (f"| {a / 1e6:.2f} | {(f + w) / a:.2f} |" if a else "| | |")
            fh.write(f"| {k} | {n} | {f / 1e6:.2f} | {w / 1e6:.2f} {extra}\n")


def mfma_md(dst: str, csv_path: str, command: str, simds: int = 1024, xcds: int = 8) -> None:
    """Per kernel: MFMA busy and the MFMA work the counters saw.

    GRBM_GUI_ACTIVE is counted by the GRBM of each of the 8 XCDs and summed (on kernels over
    100 us it reads 8x the clock times the kernel's duration), so the kernel's GPU cycles are
    GRBM_GUI_ACTIVE / 8 and MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs).
    Executed MFMA work is SQ_INSTS_VALU_MFMA_MOPS_* x 512 flops; against the cycles and the
    per-SIMD MFMA rate (1024 flops per cycle for bf16/fp16, 64 for fp32) it gives the fraction
    of the MFMA peak at the clock the kernel ran at, a second reading of the same quantity."""
    acc: dict = {}
    for r in csv.DictReader(open(csv_path)):
        k = short_name(r["Kernel_Name"])
        d = acc.setdefault(k, {})
        c = r["Counter_Name"]
        d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
        if c == "GRBM_GUI_ACTIVE":
            d["n"] = d.get("n", 0) + 1
            d["ns"] = d.get("ns", 0) + int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    rate = {"BF16": 1024.0, "F16": 1024.0, "F32": 64.0}
    rows = []
    for k, d in acc.items():
        gui = d.get("GRBM_GUI_ACTIVE", 0.0)
        if not gui or not d.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            continue
        cyc = gui / xcds
        util = 100.0 * d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)
        mops = {f: d.get(f"SQ_INSTS_VALU_MFMA_MOPS_{f}", 0.0) * 512 for f in rate}
        frac = 100.0 * sum(mops[f] / rate[f] for f in rate) / (cyc * simds)
        rows.append((k, d["n"], util, frac, {f: mops[f] / d["n"] / 1e9 for f in rate},
                     cyc / d["n"], cyc / d["ns"]))
    rows.sort(key=lambda r: -r[5] * r[1])
    with open(dst, "w") as fh:
        fh.write("# MFMA busy per kernel (rocprofv3 counters)\n\n"
                 f"Command (from the repository root, on one MI355X):\n\n```\n{command}\n```\n\n"
                 "GPU cycles = GRBM_GUI_ACTIVE / 8: the counter is summed over the GRBMs of the 8 "
                 "XCDs (it reads 8x clock x duration). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                 "(GPU cycles x 1024 SIMDs). Executed work = SQ_INSTS_VALU_MFMA_MOPS_* x 512 "
                 "flops per dispatch; `work / peak` divides it by GPU cycles x 1024 SIMDs x the "
                 "per-SIMD MFMA rate (1024 flops/cycle bf16 and fp16, 64 fp32), the same "
                 "fraction from the instruction counts. All dispatches of the run (warmup and "
                 "timed steps) are summed; the clock column is GPU cycles over the dispatches' "
                 "time stamps (under counter collection).\n\n"
                 "| kernel | dispatches | MFMA busy % | work / peak % | bf16 GFLOP/launch | "
                 "f16 GFLOP/launch | f32 GFLOP/launch | GPU cycles/launch | clock GHz |\n"
                 "|---|---|---|---|---|---|---|---|---|\n")
        for k, n, util, frac, mops, cyc, ghz in rows:
            fh.write(f"| {k} | {n} | {util:.1f} | {frac:.1f} | {mops['BF16']:.1f} | "
                     f"{mops['F16']:.1f} | {mops['F32']:.1f} | {cyc:.0f} | {ghz:.2f} |\n")


def main(argv: list[str]) -> int:
    if argv[:1] == ["stats"] and len(argv) == 5:
        stats_md(*argv[1:])
        return 0
    if argv[:1] == ["traffic"] and len(argv) == 9:
        rec = traffic_json(argv[1], argv[2], argv[3], argv[4], argv[5], argv[6],
                           float(argv[7]), argv[8])
        print(json.dumps(rec, indent=1))
        return 0
    if argv[:1] == ["traffic-table"] and len(argv) in (8, 9):
        traffic_md(argv[1], argv[2], argv[3], argv[4], argv[5], float(argv[6]), argv[7],
                   argv[8] if len(argv) == 9 else None)
        return 0
    if argv[:1] == ["mfma"] and len(argv) == 4:
        mfma_md(argv[1], argv[2], argv[3])
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
