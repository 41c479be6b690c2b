"""Write tests/golden/bf16_yardstick.json: the errors of the plain bf16 PyTorch evaluation
(oracle.bf16_reference) against the fp64 oracle on the seeded inputs of the backward
extreme-logit tests.  The Libra paper (section 6.7, "Numerical Fidelity") scales its tolerance by
these errors.  Calls only synth (inputs) and oracle (both evaluations).

Usage (repository root): python tests/golden/make_bf16_yardstick.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import attention as A, bf16_reference as R  # noqa: E402

LENS = (600, 1, 300, 199)       # the pack of the extreme-logit tests: 8 Q / 2 KV heads, d = 128
SEED = 7
KINDS = ("x4", "rising", "falling", "normal")


def inputs(kind):
    w = synth.Workload(f"logits-{kind}", sum(LENS), 8, 2, 128, 512, 4, fixed_lengths=LENS, fill=False)
    cu = synth.cu_seqlens(LENS)
    names = ("q", "k", "v", "dout")
    t = synth.make_tensors(w, SEED, names=names) if kind == "normal" else \
        synth.extreme_logit_inputs(w, cu, kind, SEED, names=names)
    return [A.widen_bf16(t[n]) for n in names], cu


def errors(kind):
    (q, k, v, do), cu = inputs(kind)
    scale = 1.0 / np.sqrt(128)
    o_ref, _ = A.forward(q, k, v, cu, scale)
    g_ref = A.backward(q, k, v, do, cu, scale)
    o, *g = R.attention(q, k, v, do, cu, scale)
    out = {"o_max_abs": float(np.abs(o - o_ref).max())}
    for name, a, r in zip(("dq", "dk", "dv"), g, g_ref):
        out[f"{name}_max_rel"] = float(np.abs(a - r).max() / np.abs(r).max())
    return out


def main():
    doc = {"source": "Libra paper, section 6.7 (Numerical Fidelity): tolerance = 2x the error of a bf16 "
                     "PyTorch reference against a high-precision one",
           "pack": {"lens": list(LENS), "h_q": 8, "h_kv": 2, "head_dim": 128, "seed": SEED},
           "errors": {kind: errors(kind) for kind in KINDS}}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bf16_yardstick.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(json.dumps(doc["errors"], indent=1))


if __name__ == "__main__":
    main()
