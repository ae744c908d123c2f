"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each mutation is a textual edit of ``oracle/wa_oracle.c`` (a dropped term, a
wrong sign, a wrong index, a wrong operand).  The mutated copy is compiled
on the CPU into a temporary library, swapped in for the real one, and every
pin of ``test_oracle_pins`` is run against it: at least one must fail.
All mutations keep memory accesses in bounds.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "wa_oracle.c")

MUTATIONS = {
    "mean divides by rows-1": ("out[col] = out[col] / (double)rows;",
                               "out[col] = out[col] / (double)(rows - 1);"),
    "mean reads the neighbouring column": ("out[col] += elem(x, dtype, t * hd + col);",
                                           "out[col] += elem(x, dtype, t * hd + (col + 1) % hd);"),
    "score drops 1/sqrt(d)": ("alpha[j] = s / sqrt((double)head_dim);", "alpha[j] = s;"),
    "score pairs the wrong columns": ("s += qbar[col] * kbar[col];",
                                      "s += qbar[col] * kbar[hd - 1 - col];"),
    "top-k keeps the lowest score": ("return sa > sb ||", "return sa < sb ||"),
    "top-k tie goes to the higher id": ("(sa == sb && ia < ib)", "(sa == sb && ia > ib)"),
    "cosine forgets a square root": ("dot / (sqrt(pp) * sqrt(nn)) : -INFINITY;",
                                     "dot / (sqrt(pp) * nn) : -INFINITY;"),
    "candidates take pages of the rank, not the chunk":
        ("chunk_pages[(int64_t)chunks_out[r] * pages_per_chunk + p];",
         "chunk_pages[(int64_t)r * pages_per_chunk + p];"),
    "gather copies rank r, not page idx[r]": ("(const char *)pool + (int64_t)idx[r] * page_bytes",
                                              "(const char *)pool + (int64_t)r * page_bytes"),
    "attention drops the scale": ("s[n] = dot * scale;", "s[n] = dot;"),
    "attention forgets to normalise": ("= acc[c] / l;", "= acc[c];"),
    "attention reads the query of the list position": (
        "qi[c] = elem(q, dtype, i * hd + (int64_t)h * head_dim + c);",
        "qi[c] = elem(q, dtype, r * hd + (int64_t)h * head_dim + c);"),
    "attention values ignore the head": (
        "acc[c] += s[n] * elem(vb, dtype, row * hd + (int64_t)h * head_dim + c);",
        "acc[c] += s[n] * elem(vb, dtype, row * hd + c);"),
    "attention lse drops the max": ("= m + log(l);", "= log(l);"),
    "attention ignores the own segment": ("const int64_t n_keys = n_ctx + n_own;",
                                          "const int64_t n_keys = n_ctx > 0 ? n_ctx : n_own;"),
}


def _pin_calls():
    calls = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        argnames, values = params[0].args
        argnames = [a.strip() for a in argnames.split(",")]
        for v in values:
            v = v if isinstance(v, tuple) else (v,)
            calls.append((name, fn, dict(zip(argnames, v))))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(mutation, tmp_path, monkeypatch):
    old, new = MUTATIONS[mutation]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not found once: %r" % old
    mutated = tmp_path / "wa_oracle_mut.c"
    mutated.write_text(text.replace(old, new))
    lib_path = tmp_path / "libwa_oracle_mut.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", str(lib_path), str(mutated), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.configure(ctypes.CDLL(str(lib_path))))
    caught = []
    for name, fn, kwargs in _pin_calls():
        try:
            fn(oracle_lib=oracle, **kwargs)
        except Exception:          # an assertion, or a shape/index error
            caught.append(name)
    assert caught, "no pin failed for the planted mistake: %s" % mutation
