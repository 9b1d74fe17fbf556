"""The oracle's pins must bite: each plausible mistake below, planted in a private copy
of ``oracle/oracle.c`` and compiled on the CPU, has to make at least one pin in
``test_oracle.py`` fail.  (The real oracle is never modified.)"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
import tests.test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, planted mistake); every mistake keeps the oracle's reads in
# bounds, so a mutant fails pins instead of crashing the test process
MUTANTS = [
    ("rope sign flipped", "y[j] = a * c - b * s;", "y[j] = a * c + b * s;"),
    ("rope turns clockwise", "y[j + half] = a * s + b * c;", "y[j + half] = -a * s + b * c;"),
    ("eps outside the root", "1.0 / sqrt(ms + eps)", "1.0 / (sqrt(ms) + eps)"),
    ("sum instead of mean", "double ms = ss / (double)d;", "double ms = ss;"),
    ("scale weight dropped", "y[c] = x[c] * r * w[c];", "y[c] = x[c] * r;"),
    ("exponent over head_dim", "-2.0 * (double)j / (double)n", "-2.0 * (double)j / (double)d"),
    ("positions never restart", "int64_t pos = t - c->offsets[s];", "int64_t pos = t;"),
    ("gqa map modulo", "int kv = h / g;", "int kv = h % c->Hkv;"),
    ("diagonal hidden", "c->causal ? last :", "c->causal ? last - 1 + (last == lo) :"),
    ("softmax scale dropped", "double sj = c->scale * dot;", "double sj = dot;"),
    ("k and v swapped", "const double* vj = c->v +", "const double* vj = c->k +"),
    ("sequence boundary ignored", "int64_t lo = c->kv_offsets[s];", "int64_t lo = 0;"),
    ("cached prefix ignored", "int64_t last = lo + base + (i - c->offsets[s]);",
     "int64_t last = lo + (i - c->offsets[s]);"),
    ("prefix one short", "int64_t last = lo + base + (i - c->offsets[s]);",
     "int64_t last = lo + base - (base > 0) + (i - c->offsets[s]);"),
    ("start positions ignored", "if (c->pos0) pos += c->pos0[s];", "(void)c->pos0;"),
    ("window one key wider", "last - c->window + 1 > lo) lo = last - c->window + 1;",
     "last - c->window > lo) lo = last - c->window;"),
    ("gate sign flipped", "o[x] *= 1.0 / (1.0 + exp(-g));", "o[x] *= 1.0 / (1.0 + exp(g));"),
    ("gate head index off", "c->gate[i * c->H + h]", "c->gate[i * c->H + (h + 1) % c->H]"),
    ("quant divisor 128", "const float scale = amax / 127.0f;",
     "const float scale = amax / 128.0f;"),
    ("quant truncates", "rintf(xr[i] / scale)", "truncf(xr[i] / scale)"),
    ("quant ties away from zero", "rintf(xr[i] / scale)", "roundf(xr[i] / scale)"),
    ("fake-quant value unscaled", "deq[r * len + i] = c * scale;", "deq[r * len + i] = c;"),
]

PIN_TESTS = [getattr(pins, n) for n in dir(pins)
             if n.startswith("test_") and callable(getattr(pins, n))
             and n not in ("test_workload_generator_is_seeded_and_shaped",
                           "test_oracle_thread_count_does_not_change_results",
                           "test_oracle_rejects_bad_arguments")]


def _run_pins():
    """Names of the pins that fail (parametrised pins run over their own cases)."""
    failed = []
    for fn in PIN_TESTS:
        marks = getattr(fn, "pytestmark", [])
        cases = [{}]
        for m in marks:
            if m.name == "parametrize":
                names = [s.strip() for s in m.args[0].split(",")]
                new = []
                for c in cases:
                    for vals in m.args[1]:
                        vals = vals if isinstance(vals, tuple) else (vals,)
                        new.append({**c, **dict(zip(names, vals))})
                cases = new
        for c in cases:
            try:
                fn(**c)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(fn.__name__)
                break
    return failed


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, before, after, monkeypatch):
    text = open(SRC).read()
    assert text.count(before) == 1, f"mutation site for '{name}' not unique in oracle.c"
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "mutant.c")
        so = os.path.join(td, "libmutant.so")
        open(src, "w").write(text.replace(before, after))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", so, src, "-lm",
                        "-lpthread"], check=True)
        real = oracle._load()
        mut = ctypes.CDLL(so)
        for fn in ("oracle_qknorm_rope", "oracle_gqa_attn", "oracle_qknorm_rope_from",
                   "oracle_chunk_attn", "oracle_quant_rows"):
            getattr(mut, fn).argtypes = getattr(real, fn).argtypes
            getattr(mut, fn).restype = getattr(real, fn).restype
        monkeypatch.setattr(oracle, "_lib", mut)
        failed = _run_pins()
    assert failed, f"no pin catches the planted mistake '{name}'"
