"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one slip in a copy of ``oracle/attn_oracle.c`` -- the kind
of error the pins are meant to catch: a dropped scale, a wrong sign, a
missing normalisation, a transposed operand, the wrong V row, a misread head
or sequence partition, a wrong bf16 widening, a gather from the wrong rank
-- compiles it, and runs the oracle pin and layout tests against that build
in a separate process.  Every mutant must fail at least one pin; the
unmodified source must pass them all.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_oracle_layout.py")]

# name -> (text in attn_oracle.c, replacement)
MUTANTS = {
    "dropped_scale": ("w[j] = acc * scale;", "w[j] = acc;"),
    "exp_sign": ("w[j] = exp(w[j] - m);", "w[j] = exp(m - w[j]);"),
    "no_normalisation": ("for (int64_t j = 0; j < S; ++j) w[j] /= l;", ""),
    "scores_transposed": ("acc += widen(Q[bshd(b, s, h, k, S, Hl, d)]) *\n                   widen(K[bshd(b, j, h, k, S, Hl, d)]);",
                          "acc += widen(Q[bshd(b, j, h, k, S, Hl, d)]) *\n                   widen(K[bshd(b, s, h, k, S, Hl, d)]);"),
    "v_row_of_query": ("acc += w[j] * widen(V[bshd(b, j, h, k, S, Hl, d)]);",
                       "acc += w[j] * widen(V[bshd(b, s, h, k, S, Hl, d)]);"),
    "heads_interleaved": ("int64_t g = rank * Hl + h_l;", "int64_t g = h_l * P + rank;"),
    "sequence_strided": ("int64_t p = s / chunk;\n    int64_t i = s % chunk;",
                         "int64_t p = s % P;\n    int64_t i = s / P;"),
    "widen_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "gather_rank0": ("int64_t off = oracle_dest_offset(b, s, h, B, S, H, d, P, rank);\n                memcpy(X_local",
                     "int64_t off = oracle_dest_offset(b, s, h, B, S, H, d, P, 0);\n                memcpy(X_local"),
}


def _run_pins(lib):
    env = dict(os.environ, UA_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + PINS,
                          cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True, timeout=600)


def _build(text, tmp_path, name):
    src = tmp_path / (name + ".c")
    src.write_text(text)
    lib = str(tmp_path / ("lib" + name + ".so"))
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", str(src), "-o", lib, "-lm"])
    return lib


def test_unmodified_oracle_passes_the_pins(tmp_path):
    r = _run_pins(_build(open(SRC).read(), tmp_path, "unmodified"))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    text = open(SRC).read()
    old, new = MUTANTS[name]
    assert text.count(old) == 1, "mutation site not found: %s" % name
    r = _run_pins(_build(text.replace(old, new), tmp_path, name))
    assert r.returncode != 0, "no pin caught the mutant %s:\n%s" % (name, r.stdout[-2000:])
    assert "failed" in r.stdout, r.stdout[-2000:]   # a failing pin, not a crash
