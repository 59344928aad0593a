#!/usr/bin/env python3
"""The state-passing kernels of one named workload, launched alone (the step's own
launch re-issued through SSD_FLAG_FWD_KERNEL / SSD_FLAG_BWD_KERNEL on a complete
call's buffers) as the associative scan with segments sized to the chains, as the
plain sequential loop it replaces, and as the tuned table's choice, `--reps`
launches each: the program a kernel trace of the comparison runs.

    python -m mamba_ssd_chunked_03_amd.tuning.scan_ab --config 2 [--reps 20]

(workload ids as in mamba_ssd_chunked_03_amd/inputs.py: 2 the layer with its
backward, 3 long context, 4 packed).  Prints the median of HIP-event timings."""
import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args()
    import torch
    import bench
    w = bench.Workload(args.config, torch.device("cuda:0"))
    tm = bench.Timer(torch.device("cuda:0"))
    res = w.scan_ab(tm, args.reps)
    for name, e in res.items():
        print("%s: %s" % (name, ", ".join("%s (variant %d) %.1f us" % (k, v["variant"], v["ms"] * 1e3)
                                           for k, v in e.items() if k != "alg_bytes")), flush=True)


if __name__ == "__main__":
    main()
