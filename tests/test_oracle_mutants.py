"""The pins have teeth: plausible mistakes planted into a *copy* of the
oracle's C source (a dropped term, a wrong sign, a transposed operand, a wrong
index) must each be caught by the finite-difference or closed-form pins.
The copy is compiled to a temporary library on the CPU; the real oracle
source is never modified."""
import os
import tempfile

import numpy as np
import pytest

from oracle import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "clr_oracle.c")

# (description, text to find, replacement) -- each must occur exactly once.
MUTANTS = [
    ("gdn: drop alpha in delta", "Si[j] = alpha * Si[j] + bki * (vt[j] - alpha * a_out[j]);",
     "Si[j] = alpha * Si[j] + bki * (vt[j] - a_out[j]);"),
    ("gdn: dk sign of erase term", "dkt[i] = beta * x - alpha * y;", "dkt[i] = beta * x + alpha * y;"),
    ("gdn: dg drops a.ddelta", "*dg_out = alpha * (frob - adot);", "*dg_out = alpha * frob;"),
    ("gdn: dS_{t-1} missing erase", "dSi[j] = alpha * (dSi[j] - kt[i] * dd[j]);", "dSi[j] = alpha * dSi[j];"),
    ("gdn: ddelta without beta", "dd[j] *= beta;\n        dvt[j] = dd[j];", "dvt[j] = dd[j];"),
    ("gdn: dq uses S_{t-1}", "const double *Si = St + (size_t)i * dv;\n        double acc = 0.0;\n        for (int j = 0; j < dv; ++j) {\n            dSi[j] += qt[i] * dot[j];\n            acc += Si[j] * dot[j];\n        }\n        dqt[i] = acc;\n    }\n    /* a = S_{t-1}^T k",
     "const double *Si = Sp + (size_t)i * dv;\n        double acc = 0.0;\n        for (int j = 0; j < dv; ++j) {\n            dSi[j] += qt[i] * dot[j];\n            acc += Si[j] * dot[j];\n        }\n        dqt[i] = acc;\n    }\n    /* a = S_{t-1}^T k"),
    ("out: transposed state", "for (int j = 0; j < dv; ++j) ot[j] += Si[j] * qi;",
     "for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)j * dv + i] * qi;"),
    ("gla: dv wrong index", "dvt[j] += dSi[j] * kt[i];", "dvt[j] += dSi[j] * kt[j % dk];"),
    ("gla: dg missing alpha", "dgt[i] = al * frob;", "dgt[i] = frob;"),
    ("gla: decay on write", "Si[j] = al * Si[j] + kt[i] * vt[j];", "Si[j] = al * (Si[j] + kt[i] * vt[j]);"),
    ("m2: dg missing alpha", "*dgt = al * frob;", "*dgt = frob;"),
    ("m2: decay on write", "S[(size_t)i * dv + j] = al * S[(size_t)i * dv + j] + kt[i] * vt[j];",
     "S[(size_t)i * dv + j] = al * (S[(size_t)i * dv + j] + kt[i] * vt[j]);"),
    ("m2: dv transposed", "for (int i = 0; i < dk; ++i) y += dS[(size_t)i * dv + j] * kt[i];",
     "for (int i = 0; i < dk; ++i) y += dS[(size_t)i * dv + j] * kt[j % dk];"),
    ("m2: dS_{t-1} not decayed", "for (size_t e = 0; e < (size_t)dk * dv; ++e) dS[e] *= al;",
     "for (size_t e = 0; e < (size_t)dk * dv; ++e) dS[e] *= 1.0;"),
    ("m2: dk uses S_{t-1} adjoint before the q term", "dkt[i] = x;\n    }\n    /* dv_j", "dkt[i] = -x;\n    }\n    /* dv_j"),
    ("kda: no decay before the erase", "for (int j = 0; j < dv; ++j) Si[j] *= al;\n    }\n    for (int j = 0; j < dv; ++j) a_out[j] = 0.0;",
     "for (int j = 0; j < dv; ++j) Si[j] *= 1.0;\n    }\n    for (int j = 0; j < dv; ++j) a_out[j] = 0.0;"),
    ("kda: dk misses the erase term", "dkt[i] -= x;", "dkt[i] -= 0.0 * x;"),
    ("kda: dbeta sign", "*dbt = db;", "*dbt = -db;"),
    ("kda: dS' without the erase", "dS[(size_t)i * dv + j] -= kt[i] * dl[j];", "dS[(size_t)i * dv + j] -= 0.0 * kt[i] * dl[j];"),
    ("kda: dg from S_t", "frob += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];",
     "frob += dS[(size_t)i * dv + j] * St[(size_t)i * dv + j];"),
    ("bwd: checkpoint off by one token", "if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * ns, S, ns * sizeof(double));\n            gdn_token_fwd",
     "if (t % CKPT == 1 || t == 0) memcpy(ck + (size_t)(t / CKPT) * ns, S, ns * sizeof(double));\n            gdn_token_fwd"),
]


def _pins_pass(lib):
    """A compact version of the FD and closed-form pins; True if all pass."""
    from tests import test_oracle_fd as fd
    rng = np.random.default_rng(3)
    ok = True
    for kind in ("gdn", "gla", "m2", "kda"):
        for shape in [(1, 6, 1, 3, 2), (1, 70, 1, 2, 2)]:
            B, T, H, dk, dv = shape
            if kind in ("gdn", "kda"):
                x = fd._rand_gdn(rng, *shape)
                if kind == "kda":
                    x["g"] = np.repeat(x["g"][..., None], shape[3], -1) * (0.5 + rng.random(shape[:3] + (shape[3],)))
            elif kind == "gla":
                x = fd._rand_gla(rng, *shape)
            else:
                x = fd._rand_gla(rng, *shape)
                x["g"] = x["g"][..., 0].copy()
            dO = rng.standard_normal((B, T, H, dv))
            dS = rng.standard_normal((B, H, dk, dv))
            if kind in ("gdn", "kda"):
                fwd = oracle.gdn_fwd if kind == "gdn" else oracle.kda_fwd
                bwd = oracle.gdn_bwd if kind == "gdn" else oracle.kda_bwd

                def loss(xx, a, b, fwd=fwd):
                    o, S = fwd(xx["q"], xx["k"], xx["v"], xx["g"], xx["beta"], xx["S_in"], lib=lib)
                    return float(np.sum(o * a) + np.sum(S * b))
                r = bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], dO, dS, lib=lib)
                names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S_in="dS_in")
            else:
                fwd = oracle.gla_fwd if kind == "gla" else oracle.mamba2_fwd
                bwd = oracle.gla_bwd if kind == "gla" else oracle.mamba2_bwd

                def loss(xx, a, b, fwd=fwd):
                    o, S = fwd(xx["q"], xx["k"], xx["v"], xx["g"], xx["S_in"], lib=lib)
                    return float(np.sum(o * a) + np.sum(S * b))
                r = bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], dO, dS, lib=lib)
                names = dict(q="dq", k="dk", v="dv", g="dg", S_in="dS_in")
            for key, gname in names.items():
                f = fd._fd(loss, x, key, dO, dS)
                if np.max(np.abs(f - r[gname])) > 2e-7 * max(np.max(np.abs(f)), 1e-3):
                    ok = False
    # forward closed forms (one token; GLA zero gate)
    r2 = np.random.default_rng(1)
    dk, dv = 5, 3
    q = r2.standard_normal((1, 1, 1, dk)); k = r2.standard_normal((1, 1, 1, dk))
    v = r2.standard_normal((1, 1, 1, dv)); S0 = r2.standard_normal((1, 1, dk, dv))
    o, S1 = oracle.gdn_fwd(q, k, v, np.array([[[-0.3]]]), np.array([[[0.7]]]), S0, lib=lib)
    kk = k[0, 0, 0]
    Sref = np.exp(-0.3) * (np.eye(dk) - 0.7 * np.outer(kk, kk)) @ S0[0, 0] + 0.7 * np.outer(kk, v[0, 0, 0])
    ok &= np.allclose(S1[0, 0], Sref, atol=1e-12) and np.allclose(o[0, 0, 0], Sref.T @ q[0, 0, 0], atol=1e-12)
    Q = r2.standard_normal((1, 9, 1, dk)); K = r2.standard_normal((1, 9, 1, dk)); V = r2.standard_normal((1, 9, 1, dv))
    o, S1 = oracle.gla_fwd(Q, K, V, np.zeros((1, 9, 1, dk)), S0, lib=lib)
    ref = np.tril(Q[0, :, 0] @ K[0, :, 0].T) @ V[0, :, 0] + Q[0, :, 0] @ S0[0, 0]
    ok &= np.allclose(o[0, :, 0], ref, atol=1e-12)
    return bool(ok)


def test_unmutated_oracle_passes_compact_pins():
    assert _pins_pass(oracle.load())


@pytest.mark.parametrize("desc,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(desc, find, repl, tmp_path):
    src = open(SRC).read()
    assert src.count(find) == 1, desc
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(find, repl))
    so = str(tmp_path / "libmut.so")
    oracle.build(src=str(mut), out=so)
    lib = oracle.load(so)
    assert not _pins_pass(lib), "planted mistake not caught: " + desc
