"""Writes tests/golden/oracle_small_cases.json from the CPU oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
The inputs are seeded draws from the workload generator; every expected
value is computed by ``oracle`` (nothing here touches the HIP library).
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from bit_gemm_bitlinear_amd import workloads as wls  # noqa: E402

CASES = [  # (seed, M, N, K, activation scale)
    (1, 1, 16, 64, 1.0),
    (2, 3, 20, 36, 1.0),
    (3, 5, 33, 260, 0.001),
    (4, 17, 40, 516, 30.0),
]


def main():
    out = []
    for seed, m, n, k, sc in CASES:
        x, w = wls.random_case(seed, m, n, k, scale=sc)
        packed, ws = oracle.pack_weights(w)
        q, s = oracle.act_quant(x)
        acc = oracle.contract(q, oracle.unpack(packed))
        y = oracle.dequant(acc, s, ws)
        out.append({
            "seed": seed, "M": m, "N": n, "K": k, "scale": sc,
            "w_scale_bits": int(np.float32(ws).view(np.uint32)),
            "packed_hex": packed.tobytes().hex(),
            "x_scale_bits": s.view(np.uint32).tolist(),
            "q": q.tolist(),
            "acc": acc.tolist(),
            "y_bits": y.tolist(),
        })
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_cases.json")
    with open(path, "w") as f:
        json.dump({"source": "tests/golden/make_golden.py (oracle only)", "cases": out}, f)
        f.write("\n")


if __name__ == "__main__":
    main()
