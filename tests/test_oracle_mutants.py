"""Each planted mistake in a copy of the oracle must fail at least one pin (CPU only).

The copy is altered as text, compiled with gcc into a temporary directory and loaded in place of
the real oracle for the duration of one case; the real oracle source is never modified.  This
shows that the pins of oracle_pins.py are tight enough to catch a dropped term, a wrong sign or
index, or a transposed operand anywhere in the oracle."""
import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("replaced: r indexed by key, not distance", "t[j] = a[j] + r[i - j];", "t[j] = a[j] + r[j];"),
    ("replaced: a and r roles swapped", "t[j] = a[j] + r[i - j];", "t[j] = a[i - j] + r[j];"),
    ("replaced: r dropped", "t[j] = a[j] + r[i - j];", "t[j] = a[j];"),
    ("ordinary: scale dropped", "t[j] = scale * acc;", "t[j] = acc;"),
    ("ordinary: q and k transposed", "ordinary_logits(d, q, k, scale, i, t);",
     "ordinary_logits(d, k, q, scale, i, t);"),
    ("softmax: max not added back to lse", "return m + log(l);", "return log(l);"),
    ("softmax: not normalised", "for (int j = 0; j <= i; ++j) p[j] /= l;", ""),
    ("fwd: diagonal key dropped from O", "      for (int j = 0; j <= i; ++j) {\n        const double* vj = v + (size_t)j * d;\n        for (int c = 0; c < d; ++c) oi[c] += p[j] * vj[c];",
     "      for (int j = 0; j < i; ++j) {\n        const double* vj = v + (size_t)j * d;\n        for (int c = 0; c < d; ++c) oi[c] += p[j] * vj[c];"),
    ("bwd: delta term dropped in dq", "const double ds = p[j] * (dp[j] - delta);",
     "const double ds = p[j] * dp[j];"),
    ("bwd: scale dropped in dq", "dqi[c] += scale * ds * kj[c];", "dqi[c] += ds * kj[c];"),
    ("bwd: sign of dk", "dkj[c] += scale * ds * qi[c];", "dkj[c] -= scale * ds * qi[c];"),
    ("bwd: delta term dropped in dk", "const double ds = pij * (dpij - dl[i]);",
     "const double ds = pij * dpij;"),
    ("bwd: dv uses v instead of dO", "dvj[c] += pij * doi[c];", "dvj[c] += pij * vj[c];"),
    ("bwd: diagonal query dropped from dk/dv", "for (int i = j; i < T; ++i) {",
     "for (int i = j + 1; i < T; ++i) {"),
    ("bwd: replaced P transposed", "tij = a[j] + r[i - j];", "tij = a[i] + r[i - j];"),
    ("calibrate: mean divides by N-1", "mean[j] = s / N;", "mean[j] = s / (N - 1);"),
    ("calibrate: deviation from wrong entry", "const double e = A[(size_t)n * T + j] - mean[j];",
     "const double e = A[(size_t)n * T + j] - mean[i];"),
    ("Eq.(1) normaliser N instead of N-1",
     "*svar = acc / ((double)(N - 1) * (double)T * (double)T);",
     "*svar = acc / ((double)N * (double)T * (double)T);"),
    ("Eq.(1) normaliser T instead of T^2",
     "*svar = acc / ((double)(N - 1) * (double)T * (double)T);",
     "*svar = acc / ((double)(N - 1) * (double)T);"),
    ("KL score: entropy instead of divergence", "if (an > 0.0) acc += an * log(an / mean[j]);",
     "if (an > 0.0) acc += an * log(an);"),
    ("KL score: mean of the wrong entry", "if (an > 0.0) acc += an * log(an / mean[j]);",
     "if (an > 0.0) acc += an * log(an / mean[i]);"),
    ("KL maps: normaliser N T^2", "*skl = acc / ((double)N * (double)T);",
     "*skl = acc / ((double)N * (double)T * (double)T);"),
    ("pattern grad: r gradient by key", "pr[i - j] += dt;", "pr[j] += dt;"),
    ("pattern grad: a gradient by distance", "pa[j] += dt;", "pa[i - j] += dt;"),
    ("pattern grad: softmax row term dropped", "const double dt = p[j] * (g[j] - pg);",
     "const double dt = p[j] * g[j];"),
    ("pattern grad: row term unweighted", "pg += p[j] * acc;", "pg += acc;"),
    ("fit: row sums taken as 1", "rowsum += ai[j];", "rowsum = 1.0;"),
    ("fit: r gradient by key", "if (gr) gr[i - j] += g;", "if (gr) gr[j] += g;"),
    ("fit: Adam without bias correction", "*w -= lr * (m[x] / c1) / (sqrt(v[x] / c2) + eps);",
     "*w -= lr * m[x] / (sqrt(v[x]) + eps);"),
    ("fit: second-moment rate", "const double b1 = 0.9, b2 = 0.999, eps = 1e-8;",
     "const double b1 = 0.9, b2 = 0.99, eps = 1e-8;"),
    ("fit: KL without the entropy term", "*kl = L + ent / T;", "*kl = L;"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(desc, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) >= 1, "mutation anchor not found: " + desc
    lib = oracle.compile_source(src.replace(old, new, 1), str(tmp_path / "mutant.so"))
    oracle.use_library(lib)
    failed = []
    try:
        for check in oracle_pins.ALL_CHECKS:
            try:
                check()
            except AssertionError:
                failed.append(check.__name__)
    finally:
        oracle.use_library(None)
    assert failed, "no pin caught the planted mistake: " + desc
