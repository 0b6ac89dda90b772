"""Child process of the forced-kernel GPU tests: runs the contiguous workloads 4
and 5 through libsmla.so with SMLA_KERNEL set in the environment (the library
reads it once, when it loads), in the row format given as the second argument
(0, fp32 group scales, by default; 1, UE8M0), and saves the outputs to the
.npz named on the command line.  Run from the repository root."""

import sys

import numpy as np

from tests._gpu import log, run_decode
from workloads import config_workload

CASES = ((4, 0), (5, 1))


def main(path, row_format=0):
    res = {}
    for cfg, ns in CASES:
        w = config_workload(cfg, row_format=row_format)
        log(f"forced-kernel case: config {cfg} num_splits {ns}")
        out, lse = run_decode(w, num_splits=ns)
        res[f"cfg{cfg}.out"] = out
        res[f"cfg{cfg}.lse"] = lse
    np.savez(path, **res)


if __name__ == "__main__":
    main(sys.argv[1], int(sys.argv[2]) if len(sys.argv) > 2 else 0)
