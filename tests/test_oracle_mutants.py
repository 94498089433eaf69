"""Plants plausible mistakes in a temporary copy of the oracle source and
checks that at least one oracle pin fails for each.  The real oracle is never
modified; each mutant is compiled with gcc into a temporary directory and
swapped in for the duration of its check only (CPU only)."""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests.test_oracle import PINS

MUTANTS = [
    ("silu sign", "static double silu(double z) { return z * sigmoid(z); }",
     "static double silu(double z) { return z * sigmoid(-z); }"),
    ("silu derivative term", "return s * (1.0 + z * (1.0 - s));", "return s * (1.0 + z * s);"),
    ("gate/up swapped in SwiGLU", "return silu(g) * u; }", "return silu(u) * g; }"),
    ("tie to higher expert id", "(l[e] == l[best] && e < best)", "(l[e] == l[best] && e > best)"),
    ("renormalisation dropped",
     "for (int k = 0; k < K; ++k) wt[k] = exp((double)l[sel[k]] - lmax) / den;",
     "for (int k = 0; k < K; ++k) wt[k] = exp((double)l[sel[k]] - lmax);"),
    ("sigmoid sign", "wt[k] = sigmoid((double)l[sel[k]]);", "wt[k] = sigmoid(-(double)l[sel[k]]);"),
    ("router weight dropped in combine", "yt[j] += wk * ok[j];", "yt[j] += ok[j];"),
    ("router weight applied twice in dRW", "s += dyt[j] * ok[j];", "s += wk * dyt[j] * ok[j];"),
    ("dU path uses dG", "* dg[i] + wu[(size_t)i * D + j] * du[i];",
     "* dg[i] + wu[(size_t)i * D + j] * dg[i];"),
    ("sigmoid used for the silu derivative", "*dg = dh * u * silu_grad(g);",
     "*dg = dh * u * sigmoid(g);"),
    ("dU without the gate activation", "*du = dh * silu(g);", "*du = dh * g;"),
    ("router weight dropped in dW_down", "dwd[(size_t)j * I + i] += dov[j] * h[i];",
     "dwd[(size_t)j * I + i] += dy[t * D + j] * h[i];"),
    ("router weight dropped in dW_down entries", "acc += (w[f] * dy[t * D + j]) * swiglu(g, u);",
     "acc += dy[t * D + j] * swiglu(g, u);"),
    ("transposed down projection in dh", "s += wd[(size_t)j * I + i] * dov[j];",
     "s += wd[(size_t)(j % I) * D + (i % D)] * dov[j];"),
    ("dW entries pick the wrong gradient", "acc += (which[q] == 0 ? dg : du) * xt[c];",
     "acc += (which[q] == 0 ? du : dg) * xt[c];"),
    ("dW_gate uses the up gradient", "dwg[(size_t)i * D + c] += dg[i] * xt[c];",
     "dwg[(size_t)i * D + c] += du[i] * xt[c];"),
    ("router: renormalisation correction with the wrong sign",
     "dlt[idx[t * K + m]] = wt[m] * (gt[m] - s);", "dlt[idx[t * K + m]] = wt[m] * (gt[m] + s);"),
    ("router: sigmoid derivative factor dropped",
     "dlt[idx[t * K + k]] = gt[k] * wt[k] * (1.0 - wt[k]);", "dlt[idx[t * K + k]] = gt[k] * wt[k];"),
    ("router: projection reads W_r transposed",
     "s += x[t * D + j] * w_r[(size_t)j * E + e];",
     "s += x[t * D + j] * w_r[((size_t)e * D + j) % ((size_t)D * E)];"),
    ("router: dW_r pairs x with the wrong expert",
     "s += x[t * D + j] * dl[t * E + e];", "s += x[t * D + j] * dl[t * E + (E - 1 - e)];"),
    ("router: dX reads W_r transposed",
     "s += dl[t * E + e] * w_r[(size_t)j * E + e];",
     "s += dl[t * E + e] * w_r[((size_t)e * D + j) % ((size_t)D * E)];"),
    ("router: dW_r without the input",
     "s += x[t * D + j] * dl[t * E + e];", "s += dl[t * E + e];"),
    ("unstable placement inside an expert",
     "int32_t p = cursor[idx[f]]++;", "int32_t p = offsets[idx[f] + 1] - 1 - (cursor[idx[f]]++ - offsets[idx[f]]);"),
]


def _build_mutant(tmp_path, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                           str(path), "-lm"])
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    so = _build_mutant(tmp_path, old, new)
    real = oracle._load()
    oracle._lib = ctypes.CDLL(so)
    caught = []
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, RuntimeError):
                caught.append(pin.__name__)
    finally:
        oracle._lib = real
    assert caught, f"mutant '{name}' passed every oracle pin"
