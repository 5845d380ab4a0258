"""Mistakes planted in copies of the oracle (on the CPU) must each fail at
least one pin in test_oracle_pins.py.  This shows the pins constrain the
oracle rather than restate it."""
import inspect
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins
from conftest import load_golden

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "scale dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "causal excludes the diagonal": ("(j) <= causal_i))", "(j) < causal_i))"),
    "causal reversed": ("(j) <= causal_i))", "(j) >= causal_i))"),
    "no max shift": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "lse without max": ("if (lse) *lse = m + log(Z);", "if (lse) *lse = log(Z);"),
    "weights not normalised": ("double w = s[j] / Z;", "double w = s[j];"),
    "key padding ignored": ("if (c->seqlens_kv && c->seqlens_kv[b] < legal_end) legal_end = c->seqlens_kv[b];\n"
                            "    const double* q = c->q",
                            "const double* q = c->q"),
    "query padding ignored": ("if (c->seqlens_q && i >= c->seqlens_q[b]) {       /* padded query row */",
                              "if (0) {"),
    "heads interleaved in Q": ("const double* q = c->qp + r * wq + (int64_t)h * c->d_k;",
                               "const double* q = c->qp + r * wq + (int64_t)h;"),
    "concat order reversed": ("ocat + (int64_t)h * c->d_v, NULL);",
                              "ocat + (int64_t)(c->H - 1 - h) * c->d_v, NULL);"),
    "value row shifted": ("const double* vj = V + (int64_t)j * v_stride;",
                          "const double* vj = V + (int64_t)(j == 0 ? 0 : j - 1) * v_stride;"),
    "decode alignment off by one": ("int pos = legal_end - c->n_q + i;", "int pos = legal_end - c->n_q + i + 1;"),
    "decode aligned at the start": ("int pos = legal_end - c->n_q + i;", "int pos = i;"),
    "window one short on the left": ("lo = (long long)i - c->window,", "lo = (long long)i - c->window + 1,"),
    "window one long on the right": ("hi = (long long)i + c->window + 1;", "hi = (long long)i + c->window + 2;"),
    "bwd softmax Jacobian without D": ("double ds = P[j] * (dp - D);", "double ds = P[j] * dp;"),
    "bwd dK without scale": ("for (int x = 0; x < c->d_k; ++x) dkj[x] += c->scale * ds * qi[x];",
                             "for (int x = 0; x < c->d_k; ++x) dkj[x] += ds * qi[x];"),
    "bwd dV from the wrong weight": ("for (int x = 0; x < c->d_v; ++x) dvj[x] += P[j] * doi[x];",
                                     "for (int x = 0; x < c->d_v; ++x) dvj[x] += ds * doi[x];"),
    "PE sine and cosine swapped": ("(c & 1) ? cos(angle) : sin(angle);", "(c & 1) ? sin(angle) : cos(angle);"),
    "PE exponent i instead of 2i": ("int i2 = c - (c & 1);", "int i2 = (c - (c & 1)) / 2;"),
    "LayerNorm unbiased variance": ("var /= d;", "var /= (d - 1);"),
    "LayerNorm eps outside the root": ("double rstd = 1.0 / sqrt(var + eps);", "double rstd = 1.0 / (sqrt(var) + eps);"),
    "sublayer without the residual": ("for (int64_t t = 0; t < nz; ++t) z[t] += h[t];", "for (int64_t t = 0; t < 0; ++t) z[t] += h[t];"),
    "projection weight transposed": ("for (int n = 0; n < g->N; ++n) c[n] += ak * wk[n];",
                                     "for (int n = 0; n < g->N; ++n) c[n] += ak * g->w[(int64_t)n * g->K + kk];"),
}


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = inspect.signature(fn).parameters
        if "causal" in params:
            out += [(f"{name}[{c}]", fn, {"causal": c}) for c in (False, True)]
        elif "golden" in params:
            out.append((name, fn, {"golden": load_golden}))
        else:
            out.append((name, fn, {}))
    return out


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, tmp_path):
    old, new = MUTATIONS[mutation]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-pthread", "-o", str(so), str(mutated), "-lm"])
    saved_path, saved_lib = oracle._LIB_PATH, oracle._lib
    try:
        oracle._lib = None
        oracle._LIB_PATH = str(so)
        oracle._SRC = str(mutated)
        oracle._load()
        failed = []
        for name, fn, kw in _pin_functions():
            try:
                fn(**kw)
            except Exception:  # an assertion or a NaN-triggered error both count
                failed.append(name)
        assert failed, f"no pin caught the planted mistake: {mutation}"
    finally:
        oracle._lib, oracle._LIB_PATH, oracle._SRC = saved_lib, saved_path, SRC
