"""Write adam_worked_example.json: a 4-element, 2-step worked example of the
optimizer step, computed by the oracle alone (run from the repository root:
``python tests/golden/make_worked_example.py``).

Inputs: master [0.02, -0.0137, 0, 0.5]; unscaled gradients [1e-3, -2e-3, 0,
3e-9] then [-5e-4, 1e-3, 0, 1e-3], stored as fp16 after scaling by the loss
scale 2^16; Adam lr 1e-4, betas (0.9, 0.999), eps 1e-8, no weight decay.
The fourth element has |g| close to eps, so its first move is well below lr.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

S = 2.0 ** 16
HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)


def hexes(a):
    a = np.asarray(a)
    return [format(int(x), "04x" if a.dtype == np.uint16 else "08x")
            for x in (a if a.dtype == np.uint16 else a.view(np.uint32))]


def main():
    p0 = np.array([0.02, -0.0137, 0.0, 0.5], np.float32)
    grads = [np.array([1e-3, -2e-3, 0.0, 3e-9]), np.array([-5e-4, 1e-3, 0.0, 1e-3])]
    st = oracle.State(p0.copy(), np.zeros(4, np.float32), np.zeros(4, np.float32),
                      np.zeros(4, np.uint16), oracle.Scaler(S, 1.0, 1000, 1))
    out = {"inputs": {"master": hexes(p0), "loss_scale": S, **HP}, "steps": []}
    for g in grads:
        g16 = (g * S).astype(np.float16).view(np.uint16)
        oracle.step(st, g16, **HP)
        out["steps"].append({"grad16": hexes(g16), "master": hexes(st.master), "m": hexes(st.m),
                             "v": hexes(st.v), "p16": hexes(st.p16)})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "adam_worked_example.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
