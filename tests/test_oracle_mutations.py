"""Planted-mistake check for the oracle's pins.

Each mutant below is a plausible slip in oracle.c (a dropped term, a wrong
sign, an off-by-one index, a flipped tie-break, a transposed operand).  The
test builds the mutant on the CPU and runs the oracle pin suite against it in
a subprocess; every mutant must make at least one pin fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_score.py", "tests/test_oracle_refine.py",
        "tests/test_oracle_select.py", "tests/test_oracle_h2o.py",
        "tests/test_oracle_select_layer.py", "tests/test_oracle_nestedkv.py"]

MUTANTS = {
    "causal-off-by-one": ("const int64_t nvis = causal ? p + 1 : N;",
                          "const int64_t nvis = causal ? p : N;"),
    "no-max-subtraction": ("lsum += exp(x[i] - m);\n        for (int64_t i = 0; i < nvis; ++i) acc[i] += exp(x[i] - m) / lsum;",
                           "lsum += exp(x[i]);\n        for (int64_t i = 0; i < nvis; ++i) acc[i] += exp(x[i]) / lsum;"),
    "gqa-interleaved": ("const int h = g * G + hl;\n      for (int w = 0;",
                        "const int h = hl * Hkv + g;\n      for (int w = 0;"),
    "scale-dropped": ("x[i] = scale * dot;", "x[i] = dot;"),
    "key-query-transposed": ("dot += (double)qr[j] * (double)kr[j];",
                             "dot += (double)qr[j] * (double)kb[j * d + i];"),
    "entropy-sign": ("const double H = log(S) - A / S;", "const double H = log(S) + A / S;"),
    "beta-no-clip": ("if (bt > (double)beta_hi) bt = (double)beta_hi;", ""),
    "hub-window-narrow": ("const int half = pool / 2;", "const int half = pool / 2 - 1;"),
    "discount-hubs-instead": ("const float qi = hub ? si : gamma * si;",
                              "const float qi = hub ? gamma * si : si;"),
    "gate-sign": ("const float dlt = t - si;", "const float dlt = si - t;"),
    "gate-r-not-squared": ("const float r2 = r * r;", "const float r2 = r;"),
    "topk-ascending": ("if (x->z > y->z) return -1; /* descending", "if (x->z < y->z) return -1; /* descending"),
    "tie-to-newest": ("    if (x->z < y->z) return 1;\n  }\n  return (x->pos < y->pos) ? -1 : (x->pos > y->pos ? 1 : 0);",
                      "    if (x->z < y->z) return 1;\n  }\n  return (x->pos > y->pos) ? -1 : (x->pos < y->pos ? 1 : 0);"),
    "recent-window-short": ("const int prot = (i < n_sink) || (i >= N - n_recent);",
                            "const int prot = (i < n_sink) || (i > N - n_recent);"),
    "h2o-new-token-not-candidate": ("for (int j = -1; j < C; ++j) {", "for (int j = 0; j < C; ++j) {"),
    "h2o-evict-max": ("if (nbest == 0 || aj < best || (aj == best && pj < bpos)) {",
                      "if (nbest == 0 || aj > best || (aj == best && pj < bpos)) {"),
    "h2o-evict-newest-on-tie": ("(aj == best && pj < bpos)", "(aj == best && pj > bpos)"),
    "h2o-recent-off-by-one": ("if (pj < n_sink || pj > tt - n_recent) continue;",
                              "if (pj < n_sink || pj >= tt - n_recent) continue;"),
    "h2o-out-self-dropped": ("if (include_self) o += ps * (double)vn[e];", ""),
    "h2o-out-keys-for-values": ("o += exp(x[j] - m) / lsum * (double)V[(int64_t)j * d + e];",
                                "o += exp(x[j] - m) / lsum * (double)K[(int64_t)j * d + e];"),
    "h2o-out-unnormalised": ("o += exp(x[j] - m) / lsum * (double)V[(int64_t)j * d + e];",
                             "o += exp(x[j] - m) * (double)V[(int64_t)j * d + e];"),
    "h2o-out-empty-slots-included": ("if (P[j] >= 0) o += exp(x[j] - m)",
                                     "o += exp(x[j] - m)"),
    "layer-tie-to-higher-head": ("if (x->head != y->head) return x->head < y->head ? -1 : 1;",
                                 "if (x->head != y->head) return x->head > y->head ? -1 : 1;"),
    "layer-floor-off-by-one": ("if (j < f) {\n          kg[cand[j].pos] = 1; /* the head's floor */",
                               "if (j <= f) {\n          kg[cand[j].pos] = 1; /* the head's floor */"),
    "layer-pool-ascending": ("    if (x->z > y->z) return -1;\n    if (x->z < y->z) return 1;\n  }\n  if (x->head",
                             "    if (x->z < y->z) return -1;\n    if (x->z > y->z) return 1;\n  }\n  if (x->head"),
    "layer-no-floor": ("kg[cand[j].pos] = 1; /* the head's floor */", "(void)0;"),
    "layer-compact-wrong-head": ("const int64_t src = (int64_t)(l * Hkv + g) * T + cu + idx[o];",
                                 "const int64_t src = (int64_t)(l * Hkv + (g + 1) % Hkv) * T + cu + idx[o];"),
    "nkv-window-off-by-one": ("const int64_t c0 = i - window + 1 > 0 ? i - window + 1 : 0;",
                              "const int64_t c0 = i - window > 0 ? i - window : 0;"),
    "nkv-block-floor": ("const int64_t bs = (N + nblocks - 1) / nblocks;",
                        "const int64_t bs = N / nblocks > 0 ? N / nblocks : 1;"),
    "nkv-anomaly-sign": ("a[i * 3 + 0] = -cos_d(x, mu, d);", "a[i * 3 + 0] = cos_d(x, mu, d);"),
    "nkv-sample-std": ("(ai[2] - mean) * (ai[2] - mean)) / 3.0;", "(ai[2] - mean) * (ai[2] - mean)) / 2.0;"),
    "nkv-routing-inverted": ("if (sg > theta) {", "if (sg < theta) {"),
    "nkv-power-max-only": ("D[x] = hi - lo + (log_prior ? log_prior[x] : 0.0);",
                           "D[x] = hi + (log_prior ? log_prior[x] : 0.0);"),
    "h2o-no-acc-update": ("if (P[j] >= 0) A[j] = (float)((double)A[j] + add[j]);",
                          "if (P[j] >= 0) A[j] = A[j];"),
}


# the pin files that exercise each family of mutants (the rest run them all)
FAMILY = {"h2o-": ["tests/test_oracle_h2o.py"], "layer-": ["tests/test_oracle_select_layer.py"],
          "nkv-": ["tests/test_oracle_nestedkv.py"]}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c99", "-fPIC",
                           "-shared", str(mut), "-o", str(lib), "-lm"])
    env = dict(os.environ, HUBKV_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *next((v for k, v in FAMILY.items() if name.startswith(k)), PINS)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
