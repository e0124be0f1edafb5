"""Writes tests/golden/tiny_f32_oracle_digest.json from the CPU oracle alone.

The digest is a regression guard: it records what the oracle (and the seeded
input generator) give for the tiny fp32 workload, so that an accidental change
to either shows up.  Run ``python -m tests.golden.make_golden`` from the
repository root after an intended change, and say in the commit which passage
of the pages justifies it.
"""
import hashlib
import json
import os

import numpy as np

from oracle import moe_oracle
from mixture_experts_transformer_moe_amd import configs
from mixture_experts_transformer_moe_amd.inputs import LayerInputs


def _sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


def tiny_digest():
    shape = configs.TINY_F32
    inp = LayerInputs(shape)
    out, r = moe_oracle.forward(inp, shape.alpha, shape.k)
    return {
        "workload": shape.name,
        "topk_idx_sha256": _sha(r.topk_idx),
        "sorted_token_sha256": _sha(r.sorted_token),
        "out_samples": [float(v) for v in out[::7, ::31].ravel()],
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle_digest.json")
    with open(path, "w") as f:
        json.dump(tiny_digest(), f, indent=1)
    print("wrote", path)
