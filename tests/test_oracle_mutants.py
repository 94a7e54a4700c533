"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case below plants one mistake in a copy of the oracle's C source (a
dropped factor, a wrong sign, rounding or index, a transposed operand, a
swapped tie rule or layout entry), builds that copy, and runs the CPU pin
tests (test_oracle_*.py) against it. Every mutant must make at least one pin
fail; a mutant that passes them all marks a part of the oracle the pins do not
cover. Runs on the CPU only; the GPU library is not involved.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (exact text in oracle/owq_oracle.c, replacement); each must occur once
MUTANTS = {
    "lambda without the factor 2": ("lambda[j] *= 2.0;", "lambda[j] *= 1.0;"),
    "lambda sums |x| instead of x^2": ("lambda[j] += v * v;", "lambda[j] += fabs(v);"),
    "lambda reads X transposed": ("owq_oracle_f16_to_f64(X[t * K + j]);", "owq_oracle_f16_to_f64(X[j * T + t]);"),
    "range without zero": ("float lo = 0.0f, hi = 0.0f; /* R1 */", "float lo = INFINITY, hi = -INFINITY; /* R1 */"),
    "step over 8 levels": ("float s32 = (hi - lo) / 7.0f;", "float s32 = (hi - lo) / 8.0f;"),
    "zero point sign": ("rintf(-lo / sf);", "rintf(lo / sf);"),
    "code rounds down": ("float r = rintf(f16_to_f32(w) / sf);", "float r = floorf(f16_to_f32(w) / sf);"),
    "zero point added before rounding": ("float r = rintf(f16_to_f32(w) / sf);",
                                         "float r = rintf(f16_to_f32(w) / sf + (float)z) - (float)z;"),
    "error ignores the zero point": ("- s * (double)(q - (int)z);", "- s * (double)q;"),
    "error summed into the wrong column": ("e[j] += d * d;", "e[(j + 1) % K] += d * d;"),
    "score is lambda + e": ("score[j] = lambda[j] * e[j];", "score[j] = lambda[j] + e[j];"),
    "score is e alone": ("score[j] = lambda[j] * e[j];", "score[j] = e[j];"),
    "ties to the higher index": ("return ia < ib ? -1 : ia > ib ? 1 : 0; /* R6 */",
                                 "return ia < ib ? 1 : ia > ib ? -1 : 0; /* R6 */"),
    "smallest scores selected": ("return -1;\n    if (sa < sb)\n        return 1;",
                                 "return 1;\n    if (sa < sb)\n        return -1;"),
    "weak codes not zero-filled": ("int code = weak[j] ? (int)z : owq_oracle_code(row[j], s16, z);",
                                   "int code = owq_oracle_code(row[j], s16, z);"),
    "pack fits the weak columns too": ("owq_oracle_qparams(row, dense, K, &s16, &z);\n        pack_row(",
                                       "owq_oracle_qparams(row, NULL, K, &s16, &z);\n        pack_row("),
    "slot pair order swapped": ("static const int kSlot[32] = {1,  6,", "static const int kSlot[32] = {6,  1,"),
    "linear zero point sign": ("double t = s * (double)(q - z) *", "double t = s * (double)(q + z) *"),
    "linear drops the weak columns": ("double t = owq_oracle_f16_to_f64(w_weak[i * k + c]) *",
                                      "double t = 0.0 * owq_oracle_f16_to_f64(w_weak[i * k + c]) *"),
    "linear gathers x at c, not idx_c": ("owq_oracle_f16_to_f64(xm[weak_idx[c]]);", "owq_oracle_f16_to_f64(xm[c]);"),
    "bit formulas swapped": ("double extra = latency_favored ? 16.0 : 13.0;",
                             "double extra = latency_favored ? 13.0 : 16.0;"),
    "fp16 rounding truncates": ("double q = rint(ldexp(a, 10 - E));", "double q = floor(ldexp(a, 10 - E));"),
    "search ignores the weights": ("t = om[e] * t;", "t = 1.0 * t;"),
    "search error not squared": ("double t = d * d;", "double t = fabs(d);"),
    "search ties to the later grid point": ("if (E < best) { /* S3", "if (E <= best) { /* S3"),
    "search steps widen the range": ("(1.0f - (float)a / 40.0f)", "(1.0f + (float)a / 40.0f)"),
    "search keeps zero point 0": ("zc <= (zsearch ? 7 : zmm); zc++)", "zc <= (zsearch ? 0 : zmm); zc++)"),
    "search error ignores the zero point": ("- sd * (double)(q - zc);", "- sd * (double)q;"),
    "search fits the weak columns too": ("owq_oracle_search_qparams(row, dense, K, lambda,",
                                         "owq_oracle_search_qparams(row, NULL, K, lambda,"),
    "search rounds the quotient down": ("float r = rintf(wf[e] / sf);", "float r = floorf(wf[e] / sf);"),
    "groups fit the weak columns too": ("owq_oracle_qparams(row + g * G, dense + g * G, G, &s16, &z);",
                                        "owq_oracle_qparams(row + g * G, NULL, G, &s16, &z);"),
    "groups share the first group's step": ("scales[i * NG + g] = s16;", "scales[i * NG + g] = scales[i * NG];"),
    "grouped product reads the row's first step": ("double s = owq_oracle_f16_to_f64(scales[i * NG + g]);",
                                                   "double s = owq_oracle_f16_to_f64(scales[i * NG]);"),
    "grouped product ignores the zero point": ("int z = zeros[i * NG + g];", "int z = 0;"),
    "backward drops the weak columns": ("Wf[i * K + weak_idx[c]] += owq_oracle_f16_to_f64(w_weak[i * k + c]);",
                                        "Wf[i * K + weak_idx[c]] += 0.0 * owq_oracle_f16_to_f64(w_weak[i * k + c]);"),
    "backward zero point sign": ("Wf[i * K + j] = s * (double)(get_code(qcodes + (i * G + j / 32) * 3, (int)(j % 32)) - z);",
                                 "Wf[i * K + j] = s * (double)(get_code(qcodes + (i * G + j / 32) * 3, (int)(j % 32)) + z);"),
    "weak gradient gathers x at c": ("owq_oracle_f16_to_f64(x[m * K + weak_idx[c]]);",
                                     "owq_oracle_f16_to_f64(x[m * K + c]);"),
    "optq without compensation inside a batch": ("wr[b] -= e * U[a * K + b];", "wr[b] -= 0.0 * e * U[a * K + b];"),
    "optq without the later batches' update": ("wr[b] -= acc[b];", "wr[b] -= 0.0 * acc[b];"),
    "optq without damping": ("double damp = 0.01 * (dsum / (double)K);", "double damp = 0.0 * (dsum / (double)K);"),
    "optq error not scaled by the factor's diagonal": ("double e = (wr[a] - sd * (double)(q - (int)z)) / U[a * K + a];",
                                                      "double e = (wr[a] - sd * (double)(q - (int)z));"),
    "optq weak block not compensated": ("w_weak[i * k + c] = owq_oracle_f64_to_f16(wr[Kd + c]);",
                                        "w_weak[i * k + c] = row[weak_idx[c]];"),
    "storage fills the tail with code 0": ("put_code(qrow + (p / 32) * 3, (int)(p % 32), z);",
                                           "put_code(qrow + (p / 32) * 3, (int)(p % 32), 0);"),
    "storage product gathers x at the position": ("owq_oracle_f16_to_f64(xm[dcol[q]]);",
                                                  "owq_oracle_f16_to_f64(xm[q]);"),
    "storage codes fitted on the whole row": ("owq_oracle_qparams(row, dense, K, &s16, &z);\n        uint32_t* qrow",
                                              "owq_oracle_qparams(row, NULL, K, &s16, &z);\n        uint32_t* qrow"),
}


def _run_mutant(name, old, new, base):
    src = open(os.path.join(ROOT, "oracle", "owq_oracle.c")).read()
    assert src.count(old) == 1, f"{name}: the planted text must occur exactly once"
    work = tempfile.mkdtemp(prefix="owq_mutant_", dir=base)
    os.makedirs(os.path.join(work, "oracle"))
    for f in ("__init__.py", "oracle.py", "owq_oracle.h"):
        shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(work, "oracle", f))
    with open(os.path.join(work, "oracle", "owq_oracle.c"), "w") as fh:
        fh.write(src.replace(old, new))
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(work, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py", "test_gpu_*", "test_zz_*",
                                                  "test_binding_validation.py",
                                                  "test_abi.py", "test_build_resources.py",
                                                  "test_bench_accounting.py"))
    # the seeded input generator comes from the package; one OpenMP thread per copy,
    # since several copies run at once
    env = dict(os.environ, PYTHONPATH=ROOT, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", "tests"],
                       cwd=work, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin():
    base = tempfile.mkdtemp(prefix="owq_mutants_")
    try:
        with cf.ThreadPoolExecutor(max_workers=6) as ex:
            # the unchanged copy must pass, so that a failure below is the planted mistake's
            items = [("control (no change)", ("lambda[j] *= 2.0;", "lambda[j] *= 2.0;"))] + list(MUTANTS.items())
            res = list(ex.map(lambda kv: _run_mutant(kv[0], kv[1][0], kv[1][1], base), items))
    finally:
        shutil.rmtree(base, ignore_errors=True)
    control, res = res[0], res[1:]
    assert control[1] == 0, f"the unchanged oracle copy fails its pins: {control[2]}"
    survived = [(n, out) for n, rc, out in res if rc == 0]
    broken = [(n, out) for n, rc, out in res if rc not in (0, 1)]
    assert not broken, f"mutant runs that did not complete: {broken}"
    assert not survived, "mistakes no pin catches: " + "; ".join(n for n, _ in survived)
