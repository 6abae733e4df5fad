"""The oracle reproduces its stored outputs on the tiny fp32 workload (regression fixture)."""
import os

import numpy as np

from golden.make_golden import HERE, input_digest, tiny_problem
import oracle.lrq_oracle as o


def _load():
    arrays, digest = {}, None
    with open(os.path.join(HERE, "tiny_oracle.txt")) as f:
        lines = [ln for ln in f.read().splitlines() if ln and not ln.startswith("#")]
    digest = lines[0].split()[1]
    for head, body in zip(lines[1::2], lines[2::2]):
        name, *shape = head.split()
        arrays[name] = np.array([float(v) for v in body.split()]).reshape([int(s) for s in shape])
    return digest, arrays


def test_tiny_golden():
    digest, ref = _load()
    spec, inp = tiny_problem()
    assert input_digest(inp) == digest, "seeded input generator changed"
    out = o.forward(spec, inp["x"], inp["gamma"], inp["w"], None, inp["a"], inp["b"], inp["positions"])
    dx, dA, dB = o.backward(spec, inp["x"], inp["gamma"], inp["w"], None, inp["a"], inp["b"],
                            inp["positions"], inp["dy"])
    got = {"out": out, "dx": dx, "dA_q": dA[1], "dB_q": dB[1], "dA_v": dA[4], "dB_v": dB[4]}
    for k, v in got.items():
        np.testing.assert_allclose(v, ref[k], rtol=1e-12, atol=1e-13, err_msg=k)
