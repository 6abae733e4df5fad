"""Write the oracle's outputs on the tiny fp32 workload to ``tiny_oracle.txt``.

The source pages print no worked example (no input -> output values), so the
only stored expected values are the oracle's own, written by this script: a
regression fixture that makes any later change of the oracle's arithmetic show
up in review.  It calls only ``oracle/`` for the values; the inputs come from
the seeded generators (their sha256 is stored so that a change of generator is
told apart from a change of oracle).

    python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from layer_rmsnorm_qkv_amd import workloads as wl  # noqa: E402  (input generator only)
import oracle.lrq_oracle as o  # noqa: E402


def tiny_problem():
    w = wl.get("tiny")
    inp = wl.make_inputs(w, with_dy=True)
    spec = o.Spec(d_model=w.d_model, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                  lora_rank=w.lora_rank, lora_alpha=w.lora_alpha, lora_targets=w.lora_targets,
                  eps=w.eps, rope_theta=w.rope_theta)
    return spec, inp


def input_digest(inp) -> str:
    h = hashlib.sha256()
    for key in ("x", "gamma", "w", "positions", "dy"):
        h.update(np.ascontiguousarray(inp[key]).tobytes())
    for t in sorted(inp["a"]):
        h.update(inp["a"][t].tobytes())
        h.update(inp["b"][t].tobytes())
    return h.hexdigest()


def main():
    spec, inp = tiny_problem()
    out = o.forward(spec, inp["x"], inp["gamma"], inp["w"], None, inp["a"], inp["b"], inp["positions"])
    dx, dA, dB = o.backward(spec, inp["x"], inp["gamma"], inp["w"], None, inp["a"], inp["b"],
                            inp["positions"], inp["dy"])
    path = os.path.join(HERE, "tiny_oracle.txt")
    with open(path, "w") as f:
        f.write("# oracle outputs on the tiny fp32 workload (T=8, d=64, 4q+2kv heads x 16, r=4 on q,v,\n")
        f.write("# alpha 8, theta 1e4, eps 1e-6, positions 0..7); written by make_golden.py from oracle/ only.\n")
        f.write(f"input_sha256 {input_digest(inp)}\n")
        for name, arr in [("out", out), ("dx", dx), ("dA_q", dA[1]), ("dB_q", dB[1]),
                          ("dA_v", dA[4]), ("dB_v", dB[4])]:
            f.write(f"{name} {' '.join(str(s) for s in arr.shape)}\n")
            f.write(" ".join(repr(float(v)) for v in arr.ravel()) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
