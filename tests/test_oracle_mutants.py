"""Mutation check of the oracle's pins: each plausible mistake, planted in a
copy of the oracle's C source and built on the CPU, must fail at least one
pin. The oracle itself is never modified."""
import os

import pytest

import oracle
import oracle_pins
from oracle.build import SOURCE, compile_source

MUTANTS = {
    "scale dropped": ("return p->scale * acc;", "return acc;"),
    "q and k rows swapped": (
        "double qc = load(p->q, at(p->layout, p->H, p->Sq, p->d, b, h, i, c), p->dtype);\n"
        "        double kc = load(p->k, at(p->layout, p->H, p->Sk, p->d, b, h, j, c), p->dtype);",
        "double qc = load(p->q, at(p->layout, p->H, p->Sq, p->d, b, h, j % p->Sq, c), p->dtype);\n"
        "        double kc = load(p->k, at(p->layout, p->H, p->Sk, p->d, b, h, i % p->Sk, c), p->dtype);"),
    "causal diagonal masked": ("if (p->causal && j > i) return 0;", "if (p->causal && j >= i) return 0;"),
    "causal direction flipped": ("if (p->causal && j > i) return 0;", "if (p->causal && j < i) return 0;"),
    "padding off by one": ("if (j >= nb) return 0;", "if (j > nb && j < p->Sk) return 0;"),
    "no max shift": ("a[j] = exp(s[j] - m); l += a[j];", "a[j] = exp(s[j]); l += a[j]; m = 0.0;"),
    "exponent sign": ("a[j] = exp(s[j] - m); l += a[j];", "a[j] = exp(m - s[j]); l += a[j];"),
    "no normalisation": ("a[j] = a[j] / l;", "a[j] = a[j];"),
    "lse without max": ("*lse = m + log(l);", "*lse = log(l);"),
    "bshd read as bhsd": ("return ((b * S + s) * H + h) * d + c;", "return ((b * H + h) * S + s) * d + c;"),
    "empty row lse zero": ("*lse = -INFINITY;\n        return;", "*lse = 0.0;\n        return;"),
    "fp16 subnormal exponent": ("mag = ldexp((double)f, -24);", "mag = ldexp((double)f, -25);"),
    "fp16 exponent bias": ("mag = ldexp((double)(f + 1024), e - 25);", "mag = ldexp((double)(f + 1024), e - 24);"),
    "bf16 shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)(h & 0x7fff) << 16;"),
    "online carry not rescaled": ("0.0 : d_prev * exp(m_prev - m);", "0.0 : d_prev;"),
    "merge weight sign": ("double w = exp(m[s] - mx);", "double w = exp(mx - m[s]);"),
    "weighted sum skips last key": (
        "for (int64_t j = 0; j < p->Sk; ++j)\n            if (key_valid(p, nb, i, j))\n"
        "                acc += a[j] *",
        "for (int64_t j = 0; j + 1 < p->Sk; ++j)\n            if (key_valid(p, nb, i, j))\n"
        "                acc += a[j] *"),
    "qkv weight read in-major": ("load(w, n * D + i, dtype)", "load(w, i * 3 * HD + n, dtype)"),
    "qkv outputs rotated": ("double* outs[3] = {q, k, v};", "double* outs[3] = {k, v, q};"),
    "qkv heads interleaved": ("const int64_t n = t * HD + h * d + c;", "const int64_t n = t * HD + c * H + h;"),
    "qkv drops last input": ("for (int64_t i = 0; i < D; ++i)\n                        acc +=",
                             "for (int64_t i = 0; i + 1 < D; ++i)\n                        acc +="),
    "softmax rows without max shift": ("yr[j] = v == -INFINITY ? 0.0 : exp(scale * v - m);",
                                       "yr[j] = v == -INFINITY ? 0.0 : exp(scale * v);"),
    "softmax rows scale dropped": ("yr[j] = v == -INFINITY ? 0.0 : exp(scale * v - m);",
                                   "yr[j] = v == -INFINITY ? 0.0 : exp(v - m);"),
    "softmax rows not normalised": ("for (int64_t j = 0; j < n; ++j) yr[j] = yr[j] / l;",
                                    "for (int64_t j = 0; j < n; ++j) yr[j] = yr[j];"),
    "softmax rows lse without max": ("lse[r] = m + log(l);", "lse[r] = log(l);"),
    "softmax rows masked kept": ("yr[j] = v == -INFINITY ? 0.0 : exp(scale * v - m);",
                                 "yr[j] = v == -INFINITY ? 1e-30 : exp(scale * v - m);"),
    "split groups transposed": ("return (((b * (H / g) + h / g) * S + s) * g + h % g) * d + c;",
                                "return (((b * (H / g) + h % (H / g)) * S + s) * g + h / (H / g)) * d + c;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutation site not unique/found: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = compile_source(str(path), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            caught.append(f"{pin.__name__}: {e}")
    assert caught, f"mutant {name!r} passed every pin"
