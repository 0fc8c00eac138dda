"""Write tests/golden/tiny_oracle.json from the oracle alone.

The pages print no worked example for the quantiser or the GEMM, so this
fixture is a regression record of the oracle itself on the tiny workload
(X [128, 256] with 1% x50 outliers, W [384, 256] ~ N(0, 0.02^2), seed 0):
any later change to the oracle's arithmetic shows up as a diff here and must
name, in its commit message, the passage or reading that justifies it.

Run from the repository root:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main():
    x, w = synth.linear_inputs("tiny", 0)
    out = {"workload": "tiny", "seed": 0,
           "input_sha256": {"x_bf16": sha(x.view(__import__("torch").int16).numpy()),
                            "w_bf16": sha(w.view(__import__("torch").int16).numpy())}}
    for pow2 in (False, True):
        qa, sa = oracle.quant_act_ref(x, pow2)
        qw, sw = oracle.quant_weight_ref(w, pow2)
        y = oracle.gemm_ref(qa, sa, qw, sw)
        key = "pow2" if pow2 else "amax_over_448"
        out[key] = {
            "qa_sha256": sha(qa), "sa_sha256": sha(sa),
            "qw_sha256": sha(qw), "sw_sha256": sha(sw),
            "sa_row0_hex": [float(v).hex() for v in sa[0]],
            "sw_hex": [[float(v).hex() for v in row] for row in sw],
            "y_samples": [[i, j, float(y[i, j]).hex()] for i, j in
                          ((0, 0), (1, 100), (63, 200), (127, 383), (77, 128))],
        }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
