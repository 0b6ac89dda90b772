"""Write tests/golden/oracle_cfg1.json and oracle_cfg1_ue8m0.json from the
oracle (the only code it calls).

Regression fixtures of the tiny workload (1 token, 16 heads, 64 of 256 rows),
with fp32 group scales and with UE8M0 scale bytes: all 16 lse values and 256
sampled output values each.  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import config_workload  # noqa: E402

for row_format, name, label in ((0, "oracle_cfg1.json", ""),
                                 (1, "oracle_cfg1_ue8m0.json", ", UE8M0 scale bytes")):
    w = config_workload(1, row_format=row_format)
    out, lse = oracle.decode(w)
    rng = np.random.default_rng(2024)
    index = np.sort(rng.choice(out.size, 256, replace=False))
    doc = {
        "workload": f"workloads config 1 (seed 1): B=1, H=16, seqlen 256, top-k 64{label}",
        "lse": [float(v) for v in lse.ravel()],
        "out_index": [int(i) for i in index],
        "out_value": [float(v) for v in out.reshape(-1)[index]],
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), name), "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", name)
