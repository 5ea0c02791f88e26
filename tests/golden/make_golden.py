"""Write tests/golden/oracle_small.json: regression values of the oracle on
a small seeded case (per-step INT8 decode, a window with compensators and
its flush, the DAMP split, calibration).

The pages print no worked example, so no stored value here comes from them.
These values are written by this script, which calls only oracle/ and the
seeded generators; tests/test_golden.py recomputes them and fails if the
oracle's output moves.  Regenerate only with a reason tied to the pages:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth   # noqa: E402

OUT = os.path.join(HERE, "oracle_small.json")


def compute():
    cfg = dict(B=1, H=2, dk=8, dv=8, io="f32", decay="scalar", a_lo=0.9, seed=11)
    kcfg = dict(cfg, decay="channel", a_lo=0.8)
    nh = 2
    S = synth.random_states(11, nh, 8, 8)
    Q, s, c = oracle.quantize(S)
    inp = synth.steps_inputs(cfg, 0, 4)
    step = oracle.quant_step(Q, s, c, inp["q"][0], inp["k"][0], inp["v"][0], inp["a"][0], inp["b"][0])
    kin = synth.steps_inputs(kcfg, 0, 4)
    enc = oracle.compress(S.astype(np.float64), 2, 20)
    X0 = oracle.state_base(enc["Q"], enc["s"], enc["c"], enc["p"], enc["w"])
    o, u, SW = oracle.window(X0, kin["q"], kin["k"], kin["v"], kin["a"], kin["b"])
    fl = oracle.compress(SW, 2, 20)
    hp = np.array([[1, 5], [0, 7]], np.int32)
    Qd, cd, rows = oracle.quantize_damp(S, hp)
    idx, score = oracle.calibrate(np.zeros_like(S), kin["k"], kin["v"], kin["a"], kin["b"], 2)
    hx = lambda a: [float(x).hex() for x in np.asarray(a, np.float64).ravel()]
    return {
        "codec": {"Q": Q.ravel().tolist(), "s": hx(s), "c": hx(c)},
        "quant_step": {"Q": step["Q"].ravel().tolist(), "s": hx(step["s"]), "o": hx(step["o"])},
        "window": {"o": hx(o), "u": hx(u)},
        "flush": {"Q": fl["Q"].ravel().tolist(), "p": hx(fl["p"]), "w": hx(fl["w"])},
        "damp": {"Q": Qd.ravel().tolist(), "c": hx(cd), "rows": rows.ravel().tolist()},
        "calibrate": {"idx": idx.ravel().tolist(), "score": hx(score)},
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(compute(), f, indent=0)
    print("wrote", OUT)
