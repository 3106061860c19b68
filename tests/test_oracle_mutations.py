"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant is oracle.c with one plausible mistake planted by a text substitution: a
flipped tie-break, a dropped bias, ascending selection, no renormalisation, W1 used for the
up half, a wrong silu sign, a transposed W2, an unstable sort, a wrong token id, an
unweighted combine, a truncating bf16 rounding, GLU in place of SwiGLU, the combine
ignoring dest_pos, and in the backward a wrong silu derivative, a transposed dW2, a
missing softmax-Jacobian term, a wrong dg and a wrong routing-weight gradient.  Each is
compiled on its own and the pin suite that covers it is run against it in a child process
(``ORACLE_LIB`` points the oracle loader at the mutant); the suite must fail.  The
unmutated source, compiled the same way, must pass, so a failure means the planted
mistake was seen.  The mutants live in a temporary directory; oracle.c itself is never
changed.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")
BWD = os.path.join(ROOT, "tests", "test_oracle_backward.py")

# name: (suite, text in oracle.c, replacement); every text occurs exactly once
MUTANTS = {
    "tie_break_flipped": (PINS, "order[j - 1] > e)", "order[j - 1] < e)"),
    "bias_dropped": (PINS, "if (bias) s += (double)bias[e];\n            l[e] = (float)s;",
                     "l[e] = (float)s;"),
    "ascending_selection": (PINS, "l[order[j - 1]] < l[e] ||", "l[order[j - 1]] > l[e] ||"),
    "no_renormalisation": (PINS, "(float)(p[order[j]] / zsel)", "(float)(p[order[j]])"),
    "w1_for_up_half": (PINS, "g += xv * load_elem(dt, w3, wbase1 + (size_t)f * H + c);",
                       "g += xv * load_elem(dt, w1, wbase1 + (size_t)f * H + c);"),
    "silu_sign": (PINS, "a / (1.0 + exp(-a)) * g", "a / (1.0 + exp(a)) * g"),
    "w2_transposed": (PINS, "load_elem(dt, w2, wbase2 + (size_t)c * F + f)",
                      "load_elem(dt, w2, wbase2 + (size_t)f * H + c)"),
    "unstable_sort": (PINS, "for (long i = 0; i < N; ++i) {          /* ascending i",
                      "for (long i = N - 1; i >= 0; --i) {          /* ascending i"),
    "wrong_token_id": (PINS, "token_ids[p] = (int32_t)(i / k);", "token_ids[p] = (int32_t)(i % k);"),
    "unweighted_combine": (PINS,
                           "s += (double)top_weights[(size_t)t * k + j] * load_elem(dt, y, p * H + c);",
                           "s += load_elem(dt, y, p * H + c);"),
    "truncating_bf16": (PINS, "nearbyint(ldexp(a, -lsb_exp))", "floor(ldexp(a, -lsb_exp))"),
    "glu_not_swiglu": (PINS, "store_elem(dt, hrow, hoff + f, a / (1.0 + exp(-a)) * g);",
                       "store_elem(dt, hrow, hoff + f, 1.0 / (1.0 + exp(-a)) * g);"),
    "combine_ignores_dest_pos": (PINS, "size_t p = (size_t)dest_pos[(size_t)t * k + j];",
                                 "size_t p = (size_t)t * k + j;"),
    "silu_derivative": (BWD, "sg * (1.0 + a * (1.0 - sg))", "sg * (1.0 - sg)"),
    "dw2_transposed": (BWD, "dw2[wb2 + (size_t)c * F + f] +=", "dw2[wb2 + (size_t)f * H + c] +="),
    "softmax_jacobian_term": (BWD, "double r = dw[(size_t)t * k + j] - wdw;",
                              "double r = dw[(size_t)t * k + j];"),
    "dg_missing_a": (BWD, "dg[(size_t)p * F + f] = dh * a * sg;", "dg[(size_t)p * F + f] = dh * sg;"),
    "routing_weight_grad": (BWD, "d += g * load_elem(dt, y, p * H + c);", "d += g;"),
}


def _compile(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"],
                   check=True, capture_output=True)
    return so


def _run_suite(suite, so):
    env = dict(os.environ, ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", suite, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_every_mutant_applies_once(source):
    for name, (_, old, _new) in MUTANTS.items():
        assert source.count(old) == 1, name


def test_unmutated_copy_passes_and_every_mutant_fails(source, tmp_path):
    jobs = {"unmutated": (PINS, source), "unmutated_bwd": (BWD, source)}
    for name, (suite, old, new) in MUTANTS.items():
        jobs[name] = (suite, source.replace(old, new))

    def run(item):
        name, (suite, text) = item
        return name, _run_suite(suite, _compile(text, str(tmp_path), name))

    with ThreadPoolExecutor(max_workers=4) as pool:
        results = dict(pool.map(run, jobs.items()))
    for name in ("unmutated", "unmutated_bwd"):
        rc, out = results[name]
        assert rc == 0, f"{name}: the pins fail on the unmutated source:\n{out}"
    survivors = [n for n in MUTANTS if results[n][0] != 1]
    assert not survivors, "mutants not caught by a failing pin: " + ", ".join(
        f"{n} (rc {results[n][0]}):\n{results[n][1]}" for n in survivors)
