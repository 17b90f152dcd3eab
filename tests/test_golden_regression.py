"""The stored oracle outputs (tests/golden/oracle_small_cases.json, written by
tests/golden/make_golden.py from the oracle alone) still match the oracle, so
an unintended change to its arithmetic shows up as a diff here."""

import json
import os

import numpy as np

import oracle
from bit_gemm_bitlinear_amd import workloads as wls

PATH = os.path.join(os.path.dirname(__file__), "golden", "oracle_small_cases.json")


def load_cases():
    with open(PATH) as f:
        return json.load(f)["cases"]


def test_golden_cases_reproduce():
    for c in load_cases():
        x, w = wls.random_case(c["seed"], c["M"], c["N"], c["K"], scale=c["scale"])
        packed, ws = oracle.pack_weights(w)
        assert int(np.float32(ws).view(np.uint32)) == c["w_scale_bits"]
        assert packed.tobytes().hex() == c["packed_hex"]
        q, s = oracle.act_quant(x)
        assert s.view(np.uint32).tolist() == c["x_scale_bits"]
        assert q.tolist() == c["q"]
        acc = oracle.contract(q, oracle.unpack(packed))
        assert acc.tolist() == c["acc"]
        assert oracle.dequant(acc, s, ws).tolist() == c["y_bits"]
