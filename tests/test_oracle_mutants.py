"""Plants plausible mistakes in copies of the oracle and checks that the pins catch them.

Each mutant is a textual edit of oracle/pa_oracle.c compiled with gcc into a
temporary library (CPU only).  The pin tests of test_oracle_pins.py are then
run against it (with those of test_oracle_fp8.py and test_oracle_prefill.py);
at least one must fail.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from oracle import build as oracle_build
import tests.test_oracle_fp8 as fp8_pins
import tests.test_oracle_pins as pins
import tests.test_oracle_prefill as prefill_pins

SRC = os.path.join(os.path.dirname(oracle_build.LIB), "pa_oracle.c")

MUTANTS = {
    "scale dropped": ("z[t] = scale * dot;", "z[t] = dot;"),
    "kv head = h mod Hkv": ("const int32_t g = h / group;", "const int32_t g = h % num_kv_heads;"),
    "no max shift": ("z[t] = exp(z[t] - m);", "z[t] = exp(z[t]);"),
    "slot forgets block size": ("return (int64_t)table_row[pos / block_size] * block_size + pos % block_size;",
                                "return (int64_t)table_row[pos / block_size] + pos % block_size;"),
    "values read from K": ("const uint16_t *vr = v_slots +", "const uint16_t *vr = k_slots +"),
    "no normalisation": ("o[i] /= l;", "o[i] /= 1.0;"),
    "f16 exponent bias": ("ldexp((double)(1024 + frac), e - 25)", "ldexp((double)(1024 + frac), e - 24)"),
    "one token too many": ("for (int64_t t = 0; t < ctx; ++t) {\n            z[t] = exp",
                           "for (int64_t t = 0; t < ctx; ++t) {\n            z[t] = (t == ctx - 1 && ctx > 1) ? 0.0 : exp"),
    "q head as kv index in V": ("(slot * num_kv_heads + g) * head_dim;\n            for (int32_t i = 0; i < head_dim; ++i)\n                o[i]",
                                "(slot * num_kv_heads + (h % num_kv_heads)) * head_dim;\n            for (int32_t i = 0; i < head_dim; ++i)\n                o[i]"),
    "e4m3 exponent bias": ("ldexp((double)(8 + frac), e - 10)", "ldexp((double)(8 + frac), e - 11)"),
    "e4m3 ties round up": ("best = (lo & 1) ? (uint8_t)(lo + 1) : lo; /* tie: even code */",
                           "best = (uint8_t)(lo + 1);"),
    "e4m3 overflow to NaN": ("        best = 0x7e;\n    } else {", "        best = 0x7f;\n    } else {"),
    "fp8 k_scale dropped": ("(pa_oracle_e4m3_to_f64(kr[i]) * k_scale)", "(pa_oracle_e4m3_to_f64(kr[i]))"),
    "prefill causal limit off by one": ("const int64_t n = (int64_t)seq_lens[s] - q_len + j + 1;",
                                        "const int64_t n = (int64_t)seq_lens[s] - q_len + j;"),
    "prefill ignores the history": ("const int64_t n = (int64_t)seq_lens[s] - q_len + j + 1;",
                                    "const int64_t n = j + 1;"),
    "prefill row owner": ("while (query_start[s + 1] <= qi)", "while (query_start[s + 1] < qi)"),
    "prefill kv head = h mod Hkv": ("const int32_t g = h / group;\n        int32_t s = 0;",
                                    "const int32_t g = h % num_kv_heads;\n        int32_t s = 0;"),
}


def _pin_calls():
    calls = []
    members = inspect.getmembers(pins, inspect.isfunction) + \
        inspect.getmembers(fp8_pins, inspect.isfunction) + \
        inspect.getmembers(prefill_pins, inspect.isfunction)
    for name, fn in members:
        if not name.startswith("test_"):
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


def _compile(tmp_path, old, new):
    text = open(SRC).read()
    assert old in text, f"mutation anchor not found: {old!r}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(text.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib),
                    str(mutated), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, tmp_path, monkeypatch):
    old, new = MUTANTS[mutant]
    path = _compile(tmp_path, old, new)
    saved = oracle._lib
    monkeypatch.setattr(oracle._build, "LIB", path)
    oracle._lib = None
    try:
        oracle._load()
        caught = []
        for name, fn, kwargs in _pin_calls():
            try:
                fn(**kwargs)
            except (Exception, pytest.fail.Exception):
                caught.append(name)
        assert caught, f"no pin caught mutant {mutant!r}"
    finally:
        oracle._lib = saved


def test_unmutated_oracle_passes_every_pin():
    for name, fn, kwargs in _pin_calls():
        fn(**kwargs)
