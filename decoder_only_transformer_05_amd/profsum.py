"""Short text summaries of rocprofv3 output, for the measurement records kept with the code.

    python -m decoder_only_transformer_05_amd.profsum stats KERNEL_STATS_CSV OUT_MD "COMMAND" "TITLE"
    python -m decoder_only_transformer_05_amd.profsum traffic OUT_JSON KERNEL \\
        FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES "COMMANDS"
    python -m decoder_only_transformer_05_amd.profsum traffic-table OUT_MD \\
        FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES "COMMANDS"

``stats`` turns a ``--kernel-trace --stats`` kernel_stats.csv into a markdown table.

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


def short_name(n: str) -> str:
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
           "bytes_per_launch": round(fetch_b + write_b),
           "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": cf_kib,
                                "write_kib": cw_kib, "fetch_scale": scale_f,
                                "write_scale": scale_w},
           "source_sha256": source_hash(kernel), "command": command}
    with open(dst, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


def traffic_md(dst: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
               copy_write_csv: str, copy_bytes: float, command: str) -> None:
    """Calibrated HBM bytes per launch of every kernel of the run, largest total first."""
    fe = counter_per_kernel(fetch_csv, "FETCH_SIZE")
    wr = counter_per_kernel(write_csv, "WRITE_SIZE")
    sf = copy_bytes / (copy_kib(copy_fetch_csv, "FETCH_SIZE") * 1024.0)
    sw = copy_bytes / (copy_kib(copy_write_csv, "WRITE_SIZE") * 1024.0)
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
                 f"write x{sw:.3f} (the counters' KiB times these give bytes).\n\n"
                 "| kernel | dispatches | fetch MB/launch | write MB/launch |\n|---|---|---|---|\n")
        for k, n, f, w in rows:
            fh.write(f"| {k} | {n} | {f / 1e6:.2f} | {w / 1e6:.2f} |\n")


def main(argv: list[str]) -> int:
    if argv[:1] == ["stats"] and len(argv) == 5:
        stats_md(*argv[1:])
        return 0
    if argv[:1] == ["traffic"] and len(argv) == 9:
        rec = traffic_json(argv[1], argv[2], argv[3], argv[4], argv[5], argv[6],
                           float(argv[7]), argv[8])
        print(json.dumps(rec, indent=1))
        return 0
    if argv[:1] == ["traffic-table"] and len(argv) == 8:
        traffic_md(argv[1], argv[2], argv[3], argv[4], argv[5], float(argv[6]), argv[7])
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
