"""Writes tests/golden/unit_oracle_digest.json: sha256 digests of the oracle's
outputs on the seeded 64x256x128 unit workload.  Calls only `oracle` and the
seeded input generators; the GPU library is never involved.  The digests pin the
oracle and the generators against unintended change; the truth of the values
themselves is pinned by the closed forms and brute force in the pin tests.

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
import synthetic  # noqa: E402


def main():
    shape = synthetic.CONFIGS["unit"][0]
    st = synthetic.streams(0, shape.config_id, shape.layer_id)
    x = synthetic.bf16_bits(synthetic.activations_bf16(st, shape.M, shape.K))
    w = synthetic.weights_f32(st, shape.N, shape.K)
    b = synthetic.bf16_bits(synthetic.bias_bf16(st, shape.N))
    wq, sw = oracle.quantize_rows_f32(w)
    out = oracle.linear(x, wq, sw, b)
    digest = {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
              for k, v in [("x", x), ("wq", wq), ("s_w", sw), ("q_x", out["q_x"]), ("s_x", out["s_x"]),
                           ("acc", out["acc"]), ("y", out["y"])]}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "unit_oracle_digest.json")
    with open(path, "w") as f:
        json.dump(digest, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
