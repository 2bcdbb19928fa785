"""HBM traffic record of one kernel from two rocprofv3 counter passes.

    python -m paged_kv_varlen_reshape_amd.traffic_record --kernel decode_mfma --config 2 \
        --fetch <pass dir>/run_counter_collection.csv --write <pass dir>/run_counter_collection.csv

Both passes profile the same bench command with `--pmc FETCH_SIZE` and
`--pmc WRITE_SIZE`; the command must also run the bench's ceiling copy
(pa_measure_copy, 4 GiB read + 4 GiB written), whose known size scales the
counters to bytes.  Prints the averages, the scale factors and the line that
bench.py reads from profiles/*.traffic.txt: it applies only while the hash of
the kernel's sources matches.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# sources whose hash guards a kernel's recorded traffic
KERNEL_SOURCES = {
    "decode_mfma": ("decode_mfma.hip", "decode.hip", "plan.hip", "internal.h"),
    "decode_streamk": ("decode.hip", "plan.hip", "internal.h"),
    "chunk_mfma": ("chunk.hip", "plan.hip", "internal.h"),
}
# kernel-name patterns in the traces
KERNEL_PATTERNS = {
    "decode_mfma": r"decode_mfma_kernel",
    "decode_streamk": r"decode_streamk_kernel",
    "chunk_mfma": r"chunk_mfma_kernel",
}
COPY_PATTERN = r"copy_kernel"
COPY_BYTES = 1 << 32  # read and written by the ceiling copy


def sources_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def average(path: str, counter: str, pattern: str) -> tuple[float, int]:
    """Mean counter value (KiB) per dispatch of the kernels matching pattern."""
    vals = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter and re.search(pattern, r["Kernel_Name"]):
                # one row per dispatch (values are already summed over the device)
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for /{pattern}/ in {path}")
    return sum(vals.values()) / len(vals), len(vals)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    ap.add_argument("--config", type=int, required=True)
    ap.add_argument("--fetch", required=True, help="counter CSV of the FETCH_SIZE pass")
    ap.add_argument("--write", required=True, help="counter CSV of the WRITE_SIZE pass")
    args = ap.parse_args()
    pat = KERNEL_PATTERNS[args.kernel]
    f_k, nf = average(args.fetch, "FETCH_SIZE", pat)
    w_k, nw = average(args.write, "WRITE_SIZE", pat)
    f_c, _ = average(args.fetch, "FETCH_SIZE", COPY_PATTERN)
    w_c, _ = average(args.write, "WRITE_SIZE", COPY_PATTERN)
    sf = COPY_BYTES / (f_c * 1024.0)
    sw = COPY_BYTES / (w_c * 1024.0)
    fetch = int(round(f_k * 1024.0 * sf))
    write = int(round(w_k * 1024.0 * sw))
    print(f"{args.kernel}: FETCH_SIZE {f_k:.1f} KiB over {nf} dispatches, WRITE_SIZE {w_k:.1f} KiB over {nw}")
    print(f"copy kernel: FETCH_SIZE {f_c:.1f} KiB, WRITE_SIZE {w_c:.1f} KiB -> scale FETCH x{sf:.4f}, WRITE x{sw:.4f}")
    print(f"traffic: kernel={args.kernel} config={args.config} src_sha={sources_sha(args.kernel)} "
          f"fetch_bytes={fetch} write_bytes={write}")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
