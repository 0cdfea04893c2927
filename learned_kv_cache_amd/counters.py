"""HBM traffic per kernel launch from rocprofv3 counter runs.

Two `rocprofv3 --pmc` passes over the same program give FETCH_SIZE (first
pass) and WRITE_SIZE (second pass), in KiB per dispatch.  On MI355X these
counters do not read the full device traffic at face value, so each is scaled
by what it reads for a plain elementwise copy of known size that the same
program runs at its end (`bench.py --copy-calib MiB`: torch.neg over a bf16
tensor, which reads and writes that many bytes once).

    python -m learned_kv_cache_amd.counters FETCH.csv WRITE.csv --kind decode_step \
        --copy-mib 1024 --out profiles/decode_step_counters.json

The record carries a hash of the kernel's sources; bench.py reports the
traffic only while the hash matches the current sources.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "learned_kv_cache_amd", "csrc")

# Per kind of record: the kernel (a substring of its name) and the sources
# that decide what it does.
KINDS = {
    "decode_attn": ("decode_attn_fast_kernel", ("decode_attn.hip", "dms_internal.h")),
    "decode_step": ("decode_step_kernel", ("decode_attn.hip", "decode_prep.h", "dms_internal.h")),
    "decode_layers": ("decode_layers_kernel", ("decode_attn.hip", "decode_prep.h", "dms_internal.h")),
}
COPY_KERNEL = "neg_kernel"


def _code_lines(text: str):
    """The source without // comments and blank lines (edits to comments do
    not change what the kernel does)."""
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            yield code


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KINDS[kind][1]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            for line in _code_lines(fh.read()):
                h.update(line.encode())
                h.update(b"\n")
    return h.hexdigest()[:16]


def per_dispatch(path: str, counter: str, kernel: str):
    """Counter values (KiB) of every dispatch whose kernel name holds `kernel`."""
    vals = []
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    return vals


def calibrated(path: str, counter: str, kernel: str, copy_kib: float):
    k = per_dispatch(path, counter, kernel)
    c = per_dispatch(path, counter, COPY_KERNEL)
    # the calibration copies are the large ones; small neg launches elsewhere are ignored
    c = [x for x in c if x > 0.05 * copy_kib]
    if not k:
        raise SystemExit(f"{path}: no {counter} rows for a kernel named like {kernel!r}")
    if not c:
        raise SystemExit(f"{path}: no {counter} rows for the calibration copy ({COPY_KERNEL})")
    factor = copy_kib / statistics.mean(c)
    return {
        "dispatches": len(k),
        "kib_per_dispatch_raw": statistics.mean(k),
        "copy_kib_raw": statistics.mean(c),
        "copy_kib_expected": copy_kib,
        "factor": factor,
        "bytes_per_dispatch": statistics.mean(k) * factor * 1024.0,
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--kind", choices=sorted(KINDS), default="decode_step")
    ap.add_argument("--copy-mib", type=float, default=1024.0)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", action="append", default=[], help="command lines that made the CSVs")
    a = ap.parse_args(argv)
    kib = a.copy_mib * 1024.0
    kernel = KINDS[a.kind][0]
    f = calibrated(a.fetch_csv, "FETCH_SIZE", kernel, kib)
    w = calibrated(a.write_csv, "WRITE_SIZE", kernel, kib)
    rec = {
        "kind": a.kind,
        "kernel": kernel,
        "source_hash": source_hash(a.kind),
        "fetch": f,
        "write": w,
        "hbm_bytes_per_launch": f["bytes_per_dispatch"] + w["bytes_per_dispatch"],
        "commands": a.command,
    }
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
