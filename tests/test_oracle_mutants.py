"""Plant plausible mistakes in a copy of the oracle and check the pins catch
each one.  The copies are built from text edits of ``oracle/lssar_ref.c`` in
a temporary directory (CPU only); the real oracle is never modified.  Every
mutant must fail at least one pin other than the brute-force restatement, so
the closed forms and invariants alone pin each step of the definition.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = open(oracle.SRC).read()

# (id, original text, mutated text): one plausible mistake per step
MUTANTS = [
    ("log2-base", "log((double)d) * log((double)i)", "log2((double)d) * log2((double)i)"),
    ("no-log-d", "log((double)d) * log((double)i)", "log((double)i)"),
    ("sqrt-d-temperature", "phi_fn(phi, scale * dot) * mask",
     "phi_fn(phi, scale * dot / sqrt((double)d)) * mask"),
    ("zero-based-i", "const int i = row + 1;", "const int i = row + 2;"),
    ("mask-before-softplus", "phi_fn(phi, scale * dot) * mask", "phi_fn(phi, scale * dot * mask)"),
    ("mask-excludes-diagonal", "(j <= i) ? 1.0 : 0.0", "(j < i) ? 1.0 : 0.0"),
    ("softplus-sign", "return x + log1p(exp(-x));", "return x + log1p(exp(x));"),
    ("softplus-neg-branch", "return log1p(exp(x));", "return log1p(exp(-x));"),
    ("no-stage1-l1", "a[j] /= l1;", "a[j] /= 1.0;"),
    ("O-two-rows", "(i <= 3) ? 0.0 : 1.0", "(i <= 2) ? 0.0 : 1.0"),
    ("O-four-rows", "(i <= 3) ? 0.0 : 1.0", "(i <= 4) ? 0.0 : 1.0"),
    ("O-none", "(i <= 3) ? 0.0 : 1.0", "1.0"),
    ("N-is-L", "a[j] * (double)i - o", "a[j] * (double)L - o"),
    ("N-is-i-minus-1", "a[j] * (double)i - o", "a[j] * (double)(i - 1) - o"),
    ("no-relu", "a[j] > 0.0 ? a[j] : 0.0", "a[j]"),
    ("p-minus-1", "a[j] = ipow(r, p);", "a[j] = ipow(r, p - 1);"),
    ("no-stage2-l1", "a[j] /= l1b;", "a[j] /= 1.0;"),
    ("no-degenerate-rule", "if (!(m > eps)) {", "if (m < -1.0) {"),
    ("v-off-by-one", "const double* vj = v + (size_t)j * d;",
     "const double* vj = v + (size_t)(j > 0 ? j - 1 : 0) * d;"),
    ("no-l2-normalise", "y[e] = x[e] / nrm;", "y[e] = x[e];"),
    ("dot-wrong-index", "dot += qh[e] * kj[e];", "dot += qh[e] * kj[0];"),
    ("norm-not-sqrt", "double nrm = sqrt(ss);", "double nrm = ss;"),
    # the ablation variants: Sigmoid as the stage-1 map, and stage 1 alone
    ("sigmoid-sign", "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    ("sigmoid-neg-branch", "return e / (1.0 + e);", "return 1.0 / (1.0 + e);"),
    ("sigmoid-ignored", "return phi == LSSAR_REF_PHI_SIGMOID ? sigmoid(x) : softplus(x);",
     "return softplus(x);"),
    ("sigmoid-everywhere", "return phi == LSSAR_REF_PHI_SIGMOID ? sigmoid(x) : softplus(x);",
     "return sigmoid(x);"),
    ("lssa-only-reweights", "    if (reweight) {", "    if (1) {"),
    ("never-reweights", "    if (reweight) {", "    if (0) {"),
    # the backward
    ("bwd-no-delta", "const double dr = (g[j] - delta) / R;", "const double dr = g[j] / R;"),
    ("bwd-no-eps", "const double da = (g[j] - eps1) / S;", "const double da = g[j] / S;"),
    ("bwd-no-sigmoid", "const double ds = da * sigmoid(s[j]);", "const double ds = da;"),
    ("bwd-power", "dr * (double)p * ipow(x[j], p - 1)", "dr * (double)p * ipow(x[j], p)"),
    ("bwd-no-N", "g[j] = (double)i * dx;", "g[j] = dx;"),
    ("bwd-no-lambda", "const double dc = lam * ds;", "const double dc = ds;"),
    ("bwd-no-projection", "out[e] = (g[e] - gx * x[e] / nrm) / nrm;", "out[e] = g[e] / nrm;"),
    ("bwd-dv-stage1-weights", "dv[(size_t)j * d + e] += w[j] * gi[e];",
     "dv[(size_t)j * d + e] += A[j] * gi[e];"),
    ("bwd-dk-wrong-operand", "dkh[(size_t)j * d + e] += dc * qi[e];",
     "dkh[(size_t)j * d + e] += dc * kh[(size_t)j * d + e];"),
    # the row statistics
    ("stats-mask-leak", "l1 += softplus(s) * mask;", "l1 += softplus(s);"),
    ("stats-max-over-masked", "if (mask == 1.0 && s > smax)", "if (s > smax)"),
    ("stats-max-of-softplus", "            smax = s;", "            smax = softplus(s);"),
    ("stats-unscaled", "const double s = scale * dot;", "const double s = dot;"),
    ("stats-normalised", "    st[0] = l1;", "    st[0] = l1 / (double)i;"),
    # the row-sampling entry and the stage-2 self-check
    ("rows-row-index", "reweight, rows[r], a, out", "reweight, r, a, out"),
    ("rows-query-row", "lssar_row(qh + (size_t)rows[r] * d", "lssar_row(qh + (size_t)r * d"),
    ("selfcheck-off", "if (!(fabs(a[j] / l1b - b[j] / l1c) <= 1e-12))", "if (0)"),
    ("selfcheck-power", "b[j] = ipow(fmax(a[j], 0.0) / m, p);",
     "b[j] = ipow(fmax(a[j], 0.0) / m, p - 1);"),
    ("bwd-degenerate-passes", "            continue;                            /* R16: no gradient */",
     "            ;"),
]

INDEPENDENT_PINS = [p for p in oracle_pins.PINS if p is not oracle_pins.brute_force_matrix_form]


def test_mutant_texts_apply():
    # a pattern may occur in the forward and in the backward (they share the
    # definition); every occurrence is mutated
    for name, old, new in MUTANTS:
        assert SRC.count(old) >= 1, f"mutant {name}: pattern not found"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "lssar_ref.c")
        with open(src, "w") as f:
            f.write(SRC.replace(old, new))
        hdr = os.path.join(os.path.dirname(oracle.SRC), "lssar_ref.h")
        with open(os.path.join(td, "lssar_ref.h"), "w") as f:
            f.write(open(hdr).read())
        lib = oracle.load(oracle.build(src, os.path.join(td, "libmut.so")))
        caught = []
        for pin in INDEPENDENT_PINS:
            try:
                pin(lib)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
        assert caught, f"mutant {name} passed every independent pin"
