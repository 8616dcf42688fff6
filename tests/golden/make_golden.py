"""Writes / reads ``oracle_small.txt``: fp64 oracle outputs of one small packed
problem (GQA 4/2, bottom-right causal, window 3, sinks, padded slots).

The pages print no worked example with values, so this fixture is not a pin:
it is a regression guard that catches an unintended change to the oracle's
arithmetic.  It is written only by this script, which calls only ``oracle``.

    python tests/golden/make_golden.py      # rewrite the fixture
"""
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import Problem  # noqa: E402

PATH = os.path.join(HERE, "oracle_small.txt")


def _rnd(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def compute():
    cap_q, cap_kv = [4, 8], [6, 7]
    cu_q, cu_kv = [0, 4, 12], [0, 6, 13]
    p = Problem.packed(4, 2, 4, cu_q, cu_kv, [3, 8], [6, 5], 12, 13, causal=True,
                       bottom_right=True, window_left=3, scale=0.5, has_sink=True)
    q, k, v, dO = _rnd((12, 4, 4), 1), _rnd((13, 2, 4), 2), _rnd((13, 2, 4), 3), _rnd((12, 4, 4), 4)
    sink = _rnd((4,), 5)
    r = oracle.backward(p, q, k, v, dO, sink)
    return {"o": r["o"], "lse": r["lse"], "dq": r["dq"], "dk": r["dk"], "dv": r["dv"], "dsink": r["dsink"]}


def write(path=PATH):
    out = compute()
    with open(path, "w") as f:
        f.write("# fp64 oracle outputs; see make_golden.py\n")
        for key, t in out.items():
            f.write(f"{key} {' '.join(str(s) for s in t.shape)}\n")
            f.write(" ".join(repr(float(x)) for x in t.reshape(-1)) + "\n")


def read(path=PATH):
    out = {}
    with open(path) as f:
        lines = [l for l in f.read().splitlines() if l and not l.startswith("#")]
    for head, body in zip(lines[0::2], lines[1::2]):
        key, *shape = head.split()
        vals = [float(x) for x in body.split()]
        out[key] = torch.tensor(vals, dtype=torch.float64).reshape([int(s) for s in shape])
    return out


if __name__ == "__main__":
    write()
    print("wrote", PATH)
