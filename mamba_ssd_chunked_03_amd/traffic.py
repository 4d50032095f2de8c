"""HBM traffic per kernel launch from rocprofv3 counters, and its record under profiles/.

The HBM bytes a launch really moves come from two counter runs of the same bench command
(`rocprofv3 --pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`; KiB per dispatch).  Each counter
is scaled by what it reads for a plain copy of known size (`bench.py --copy-calibration
MIB` under the same counter): bytes the copy must move / bytes the counter reports.

The record is a markdown table in profiles/ with one row per kernel, holding the scaled
traffic and a sha256 of the sources the kernel is built from.  bench.py reports a
kernel's traffic only while those sources still hash to the recorded value (otherwise
the kernel has changed since the counters were taken and the figure is null).

    python -m mamba_ssd_chunked_03_amd.traffic DIR COPY_MIB OUT.md   # DIR: the four .db files
"""
import collections
import hashlib
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# stage -> (pattern in the kernel's symbol, sources it is built from)
KERNELS = {
    "chunk_cumsum": ("chunk_cumsum_kernel", ["chunk_cumsum.hip", "ssd_internal.h"]),
    "chunk_state": ("chunk_state_(pipe|mfma)_kernel", ["chunk_mfma.hip", "mfma_common.h",
                                                        "ssd_internal.h"]),
    "state_passing": ("state_passing_kernel", ["state_passing.hip", "ssd_internal.h"]),
    "chunk_scan": ("chunk_scan_mfma_kernel", ["chunk_scan_mfma.hip", "mfma_common.h",
                                              "ssd_internal.h"]),
}


def source_hash(stage):
    h = hashlib.sha256()
    for f in KERNELS[stage][1] + ["../build.py"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _per_dispatch_kib(db, counter, pattern):
    c = sqlite3.connect(db)
    rows = c.execute("select dispatch_id, kernel_name, sum(value) from counters_collection "
                     "where counter_name = ? group by dispatch_id", (counter,)).fetchall()
    vals = [v for _, k, v in rows if re.search(pattern, k)]
    return sum(vals) / len(vals) if vals else None


def summarize(dir_, copy_mib):
    """Rows per stage: fetch/write KiB per dispatch, scale factors, HBM bytes per launch."""
    copy_bytes = copy_mib * (1 << 20)
    cf = _per_dispatch_kib(os.path.join(dir_, "cfetch_results.db"), "FETCH_SIZE", "copy")
    cw = _per_dispatch_kib(os.path.join(dir_, "cwrite_results.db"), "WRITE_SIZE", "copy")
    sf, sw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    rows = collections.OrderedDict()
    for stage, (pat, _) in KERNELS.items():
        f = _per_dispatch_kib(os.path.join(dir_, "fetch_results.db"), "FETCH_SIZE", pat)
        w = _per_dispatch_kib(os.path.join(dir_, "write_results.db"), "WRITE_SIZE", pat)
        if f is None or w is None:
            continue
        rows[stage] = dict(fetch_kib=f, write_kib=w, fetch_scale=sf, write_scale=sw,
                           bytes=int(round(f * 1024 * sf + w * 1024 * sw)),
                           sources=source_hash(stage))
    return rows


def write_md(rows, path, title, commands):
    with open(path, "w") as fh:
        fh.write(f"# {title}\n\n")
        fh.write("Commands (from the repository root on one MI355X; `cd /tmp && export "
                 "TMPDIR=/tmp` first), one counter per run:\n\n```\n")
        fh.write("\n".join(commands) + "\n```\n\n")
        fh.write("Scale factors: what a plain copy of known size should move divided by what "
                 "the same counter reports for it.\n\n")
        fh.write("| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | fetch scale | "
                 "write scale | HBM bytes/launch | sources sha256 |\n")
        fh.write("|---|---|---|---|---|---|---|\n")
        for stage, r in rows.items():
            fh.write(f"| {stage} | {r['fetch_kib']:.1f} | {r['write_kib']:.1f} | "
                     f"{r['fetch_scale']:.3f} | {r['write_scale']:.3f} | {r['bytes']} | "
                     f"{r['sources']} |\n")


def load(path):
    """stage -> (HBM bytes per launch, sources hash) from a record written by write_md."""
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        m = re.match(r"\|\s*(\w+)\s*\|\s*[\d.]+\s*\|\s*[\d.]+\s*\|\s*[\d.]+\s*\|\s*[\d.]+\s*\|"
                     r"\s*(\d+)\s*\|\s*([0-9a-f]+)\s*\|", line)
        if m:
            out[m.group(1)] = (int(m.group(2)), m.group(3))
    return out


def current_mfma_busy(path, stage):
    """The matrix-core busy fraction of `stage` in the forward run of the SQ-counter record
    (profiles/sq_counters_*.md) if taken on the current sources, else None."""
    if not os.path.exists(path):
        return None
    for line in open(path):
        m = re.match(r"\|\s*fwd\s*\|\s*(\w+)\s*\|[^|]*\|\s*([\d.]+)%\s*\|.*\|\s*([0-9a-f]+)\s*\|\s*$",
                     line)
        if m and m.group(1) == stage:
            return round(float(m.group(2)) / 100, 4) if m.group(3) == source_hash(stage) else None
    return None


def current_traffic(path, stage):
    """HBM bytes per launch of `stage` if recorded for the current sources, else None."""
    rec = load(path).get(stage)
    if rec is None or rec[1] != source_hash(stage):
        return None
    return rec[0]


if __name__ == "__main__":
    d, mib, out = sys.argv[1], int(sys.argv[2]), sys.argv[3]
    title = sys.argv[4] if len(sys.argv) > 4 else "HBM traffic per launch"
    cmds = sys.argv[5:] if len(sys.argv) > 5 else []
    write_md(summarize(d, mib), out, title, cmds)
    print(open(out).read())
