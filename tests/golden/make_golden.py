"""Writes tests/golden/tiny_oracle.json: digests and sample values of the oracle's
outputs on the tiny configuration (M=64, K=256, N=128, R=16, seed 1001).

Calls only oracle/ and the seeded input generators; rerun after an intended,
justified change of the oracle's arithmetic:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import svdq as S  # noqa: E402


def compute():
    d = workloads.make_linear(**workloads.TINY)
    qw, ws = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    y64, y, qact, ascales = S.linear_w4a4(d["x"], d["smooth"], qw, ws, d["wcscales"],
                                          d["wtscale"], d["proj_down"], d["proj_up"], d["bias"])
    h = lambda a: hashlib.sha256(a.tobytes()).hexdigest()  # noqa: E731
    return {
        "config": "M=64 K=256 N=128 R=16 kind=tiny seed=1001",
        "qweight_sha256": h(qw), "wscales_sha256": h(ws),
        "qact_sha256": h(qact), "ascales_sha256": h(ascales), "y_bf16_sha256": h(y),
        "y64_samples": {f"{m},{n}": float(y64[m, n]) for m, n in [(0, 0), (7, 9), (63, 127), (32, 64)]},
        "ascales_first_row": [int(v) for v in ascales[0, :16]],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", out)
