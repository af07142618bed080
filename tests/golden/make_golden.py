"""Writes the oracle regression fixtures in this folder.

The source pages print no worked numeric example for the layer, so these
fixtures are not the pages' numbers: they freeze the fp64 oracle's outputs
on two tiny seeded cases (after the oracle was pinned by finite differences,
closed forms and invariants), so that any later change to the oracle's
arithmetic shows up as a diff.  This script calls only ``oracle/``.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import oracle  # noqa: E402


def _case(kind, seed):
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 6, 2, 3, 2
    x = dict(q=rng.standard_normal((B, T, H, dk)), k=rng.standard_normal((B, T, H, dk)),
             v=rng.standard_normal((B, T, H, dv)), S_in=0.5 * rng.standard_normal((B, H, dk, dv)),
             dO=rng.standard_normal((B, T, H, dv)), dS_out=rng.standard_normal((B, H, dk, dv)))
    x["k"] /= np.linalg.norm(x["k"], axis=-1, keepdims=True)
    if kind == "gdn":
        x["g"] = -0.4 * np.abs(rng.standard_normal((B, T, H)))
        x["beta"] = rng.uniform(0.05, 0.95, (B, T, H))
        o, S = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
        r = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    else:
        x["g"] = -0.4 * np.abs(rng.standard_normal((B, T, H, dk)))
        o, S = oracle.gla_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
        r = oracle.gla_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"])
    out = dict(o=o, S_out=S, **r)
    return {"inputs": {k: v.tolist() for k, v in x.items()},
            "outputs": {k: v.tolist() for k, v in out.items()}}


def main():
    for kind, seed in (("gdn", 1234), ("gla", 4321)):
        with open(os.path.join(HERE, f"oracle_{kind}_tiny.json"), "w") as f:
            json.dump(_case(kind, seed), f, indent=0)


if __name__ == "__main__":
    main()
