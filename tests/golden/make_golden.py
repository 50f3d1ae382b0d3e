"""Writes tests/golden/tiny_block.json: digests and sampled values of the
oracle's outputs for the 64-row bf16 block (C=256, H=768) and its FP8 form.

The pages print no worked example, so this file is a regression record of the
oracle, not an outside pin: it calls only ``oracle/`` and the seeded input
generator.  Re-run it only with a commit that names the passage, or the
reading of one, that justifies a change in the oracle's arithmetic.
"""

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
from transformer_ffn_block_residual_amd import workloads as W  # noqa: E402

KEYS = ("residual", "y", "rstd", "gu", "h", "down", "next_residual")


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def record():
    w = W.WORKLOADS["tiny"]
    d = W.block_inputs(w.N, w.C, w.H, w.seed, w.w_std, w.outliers)
    out = {"workload": "tiny (N=64, C=256, H=768, eps=1e-5)", "seed": w.seed}
    for fp8 in (False, True):
        b = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], w.eps, fp8=fp8)
        rec = {k: digest(b[k]) for k in KEYS}
        rec["absmax_y"] = float(b["absmax_y"])
        rec["absmax_h"] = float(b["absmax_h"])
        rec["down_row0_first8"] = [int(v) for v in b["down"][0, :8]]
        if fp8:
            rec.update(qy=digest(b["qy"]), qh=digest(b["qh"]), s_y=float(b["s_y"]), s_h=float(b["s_h"]),
                       s_gu=float(b["s_gu"]), s_d=float(b["s_d"]))
        out["fp8" if fp8 else "bf16"] = rec
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_block.json"), "w") as f:
        json.dump(record(), f, indent=1, sort_keys=True)
        f.write("\n")
