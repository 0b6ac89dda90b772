"""Child process of the SMLA_DEBUG_VALIDATE GPU test: runs every case of
tests/_debug_cases.py through libsmla.so with the scan switched on, and saves
the outputs and the flags each call reported to the .npz named on the command
line.  Run from the repository root with SMLA_DEBUG_VALIDATE=1 in the
environment."""

import sys

import numpy as np
import torch

import sparse_mla_decode_02_amd as smla
from tests._debug_cases import cases
from tests._gpu import device_inputs, log, run_decode
from tests.test_gpu_paged import run_paged


def main(path):
    assert smla.debug_validate_enabled(), "SMLA_DEBUG_VALIDATE is not set"
    assert smla.debug_flags(clear=True) == 0
    res = {}
    for name, kind, w, lay in cases():
        log(f"debug-validate case {name} ({kind})")
        if kind == "decode":
            out, lse = run_decode(w, num_splits=0)
        elif kind == "paged":
            out, lse = run_paged(w, lay, num_splits=0)
        else:
            q, cache, idx, seqlens = device_inputs(w)
            o = torch.full((w.batch, w.heads, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
            l = torch.full((w.batch, w.heads), float("nan"), dtype=torch.float32, device="cuda:0")
            smla.sparse_mla_decode_per_head(q, cache, idx, seqlens, w.scale, o, l,
                                            kv_seq_stride=w.kv_seq_stride)
            torch.cuda.synchronize()
            out = o.float().cpu().numpy().astype(np.float64)
            lse = l.cpu().numpy().astype(np.float64)
        res[f"{name}.flags"] = np.array(smla.debug_flags(clear=True), dtype=np.int64)
        res[f"{name}.out"] = out
        res[f"{name}.lse"] = lse
    np.savez(path, **res)
    log("debug-validate child done")


if __name__ == "__main__":
    main(sys.argv[1])
