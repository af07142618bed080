"""The oracle reproduces its frozen regression fixtures (tests/golden)."""
import json
import os

import numpy as np
import pytest

from oracle import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("kind", ["gdn", "gla"])
def test_oracle_matches_fixture(kind):
    d = json.load(open(os.path.join(HERE, f"oracle_{kind}_tiny.json")))
    x = {k: np.array(v) for k, v in d["inputs"].items()}
    if kind == "gdn":
        o, S = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
        r = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    else:
        o, S = oracle.gla_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
        r = oracle.gla_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"])
    got = dict(o=o, S_out=S, **r)
    for key, ref in d["outputs"].items():
        np.testing.assert_allclose(got[key], np.array(ref), rtol=1e-12, atol=1e-13, err_msg=key)
