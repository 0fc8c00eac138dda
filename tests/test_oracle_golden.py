"""The oracle reproduces its recorded results on the tiny workload (CPU).

``tests/golden/tiny_oracle.json`` is written by ``tests/golden/make_golden.py``
from ``oracle/`` and ``synth/`` alone; this guards the oracle (and the seeded
generators) against unintended change.
"""

import hashlib
import json
import os

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.json")


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_tiny_workload_matches_golden_record():
    with open(GOLDEN) as f:
        gold = json.load(f)
    x, w = synth.linear_inputs("tiny", 0)
    assert _sha(x.view(torch.int16).numpy()) == gold["input_sha256"]["x_bf16"]
    assert _sha(w.view(torch.int16).numpy()) == gold["input_sha256"]["w_bf16"]
    for pow2, key in ((False, "amax_over_448"), (True, "pow2")):
        rec = gold[key]
        qa, sa = oracle.quant_act_ref(x, pow2)
        qw, sw = oracle.quant_weight_ref(w, pow2)
        assert _sha(qa) == rec["qa_sha256"] and _sha(sa) == rec["sa_sha256"]
        assert _sha(qw) == rec["qw_sha256"] and _sha(sw) == rec["sw_sha256"]
        y = oracle.gemm_ref(qa, sa, qw, sw)
        for i, j, hx in rec["y_samples"]:
            assert y[i, j] == float.fromhex(hx)
