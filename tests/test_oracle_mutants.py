"""Plant plausible mistakes in a copy of the oracle and check the pins catch each one.

Each mutant is a textual edit of ``oracle/pisa_oracle.c`` (a dropped term, a wrong sign,
index or bound, a reversed order), compiled with gcc into a temporary library that the pin
suite then loads through ``PISA_ORACLE_LIB``.  The pin suite must fail on every mutant.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pisa_oracle.c")

MUTANTS = {
    "child-index-shift": ("int64_t c0 = x * q->g, c1 = c0 + q->g < q->n[l - 1]",
                          "int64_t c0 = x * q->g + 1, c1 = c0 + q->g < q->n[l - 1]"),
    "visibility-strict": ("return j * r->q->span[l] <= r->bq;", "return j * r->q->span[l] < r->bq;"),
    "tie-break-reversed": ("  return (x->j > y->j) - (x->j < y->j);\n}\n\nstatic int by_index",
                           "  return (x->j < y->j) - (x->j > y->j);\n}\n\nstatic int by_index"),
    "causal-excludes-self": ("  if (hi > r->i + 1) hi = r->i + 1;\n  double* vals",
                             "  if (hi > r->i) hi = r->i;\n  double* vals"),
    "causal-mask-dropped": ("  if (hi > r->i + 1) hi = r->i + 1;\n  double* vals", "  double* vals"),
    "leaf-scale-dropped": ("vals[m++] = q->s * dot(r->qrows + (int64_t)h * q->d, key, q->d);",
                           "vals[m++] = dot(r->qrows + (int64_t)h * q->d, key, q->d);"),
    "route-scale-dropped": ("vals[m++] = q->s * dot(r->qrows + (int64_t)h * q->d, r->pyr",
                            "vals[m++] = dot(r->qrows + (int64_t)h * q->d, r->pyr"),
    "gqa-first-head-only": ("    if (per_head) per_head[h] = v;\n    total += v;\n  }\n  return total;",
                            "    if (per_head) per_head[h] = v;\n    if (h == 0) total += v;\n  }\n  return total;"),
    "forced-prev-missing": ("  if (bq - 1 > 0) F[m++] = bq - 1;\n", ""),
    "leaf-mean-is-sum": ("      o[e] = acc / (double)(hi - lo);", "      o[e] = acc;"),
    "node-mean-weighted-wrong": ("        o[e] = acc / (double)(c1 - c0);", "        o[e] = acc / (double)q->g;"),
    "lse-missing-log": ("  return m + log(acc);", "  return m + acc;"),
    "route-keeps-K-minus-1": ("      int nk = nx < K ? nx : K;", "      int nk = nx < K - 1 ? nx : K - 1;"),
    "leaf-takes-one-less": ("  int Kp = K - nf;\n  int take = Kp < nr ? Kp : nr;\n  if (nr > Kp",
                            "  int Kp = K - nf - 1;\n  int take = Kp < nr ? Kp : nr;\n  if (nr > Kp"),
    "level-stop-early": ("while (n[L] > (int64_t)g * K && L < ORC_MAXL)", "while (n[L] > (int64_t)K && L < ORC_MAXL)"),
    "transposed-child-level": ("r->pyr + (q->off[l - 1] + c) * q->d, q->d);", "r->pyr + (q->off[l] + c % q->n[l]) * q->d, q->d);"),
    "pisa-scorer-ignored": ("  if (scorer == 0) return orc_lse(x, m);", "  return orc_lse(x, m);"),
    "pisa-drops-log-m": ("  double out = log((double)m) + mean;", "  double out = mean;"),
    "pisa1-keeps-variance": ("  if (scorer == 2) {\n    double var", "  if (scorer >= 1) {\n    double var"),
    "pisa2-variance-sign": ("    out += 0.5 * var / (double)m;", "    out -= 0.5 * var / (double)m;"),
    "pisa2-sample-variance": ("    out += 0.5 * var / (double)m;", "    out += 0.5 * var / (double)(m > 1 ? m - 1 : 1);"),
    "pisa2-no-half": ("    out += 0.5 * var / (double)m;", "    out += var / (double)m;"),
    "bsa-uses-level-2": ("r->pyr + (q->off[1] + j) * q->d, q->d);", "r->pyr + (q->off[2] + j) * q->d, q->d);"),
    "bsa-scale-dropped": ("    total += q->s * dot(r->qrows + (int64_t)h * q->d, r->pyr + (q->off[1] + j)",
                          "    total += dot(r->qrows + (int64_t)h * q->d, r->pyr + (q->off[1] + j)"),
    "bsa-first-head-only": ("  for (int h = 0; h < q->G; ++h)\n    total += q->s", "  for (int h = 0; h < 1; ++h)\n    total += q->s"),
    "bsa-sees-next-block": ("  for (int64_t j = 0; j <= r->bq; ++j) {\n    if (is_in(F, nf, j)) continue;\n    S[nr].j = j;",
                            "  for (int64_t j = 0; j <= r->bq + 1 && j < q->n[1]; ++j) {\n    if (is_in(F, nf, j)) continue;\n    S[nr].j = j;"),
    "bsa-keeps-one-more": ("  int Kp = K - nf;\n  int take = Kp < nr ? Kp : nr;\n  for (int t = 0; t < nf; ++t) {",
                           "  int Kp = K - nf + 1;\n  int take = Kp < nr ? Kp : nr;\n  for (int t = 0; t < nf; ++t) {"),
    "bsa-forced-scored": ("    S[take + t].s = INFINITY;", "    S[take + t].s = bsa_score(r, F[t]);"),
    "attn-causal-dropped": ('      if (hi > r.i + 1) hi = r.i + 1;\n      for (int64_t p = lo; p < hi; ++p) key[m++] = p;',
                           '      for (int64_t p = lo; p < hi; ++p) key[m++] = p;'),
    "attn-skips-block-0": ('      if (j < 0 || j > r.bq) continue;',
                           '      if (j <= 0 || j > r.bq) continue;'),
    "attn-scale-dropped": ('        x[c] = q.s * acc;',
                          '        x[c] = acc;'),
    "attn-values-are-keys": ('o[e] += w * ld(v, r.kbase',
                            'o[e] += w * ld(k, r.kbase'),
    "attn-unnormalised": ('        double w = exp(x[c] - z);',
                         '        double w = exp(x[c] - x[0]);'),
}


def _run(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor not unique ({src.count(old)})"
    path = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    open(path, "w").write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", path, "-o", lib, "-lm"])
    env = dict(os.environ, PISA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_mutant_is_caught():
    tmp = tempfile.mkdtemp(prefix="pisa_mut_")
    try:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda n: _run(n, tmp), sorted(MUTANTS)))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants not caught by the pins: %s" % [n for n, _ in survivors]
    # a mutant must fail a test, not crash the interpreter
    assert all(rc == 1 for _, rc, _ in results), [(n, rc, out) for n, rc, out in results if rc != 1]
