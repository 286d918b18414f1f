"""Plausible mistakes planted in a copy of the oracle must each trip a pin.

Each mutant is one textual edit of ``oracle/tt_oracle.c`` (a dropped term, a wrong
sign, index or operator), compiled with gcc into a temporary library. The pin
suite of ``pins.py`` runs against it and at least one pin must fail. An edit
whose target text is missing from the oracle fails the test, so the list stays
in step with the source. Everything runs on the CPU.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "tt_oracle.c")

MUTANTS = [
    ("drop in-block keys", "const int n = L + (Kd ? S : 0);", "const int n = L;"),
    ("wrong GQA head map", "const int g = h / G;", "const int g = h % Hkv;"),
    ("scale dropped", "sc[j] = scale * dot;", "sc[j] = dot;"),
    ("page table ignored", "int page = page_table[(size_t)b * max_pages + j / page_size];",
     "int page = b * max_pages + j / page_size;"),
    ("upper length clamp dropped", "if (L > len_cap) L = len_cap;", ""),
    ("page id above the pool clamped to page 0", "if (page >= num_pages) page = num_pages - 1;",
     "if (page >= num_pages) page = 0;"),
    ("negative page id clamped to the last page", "if (page < 0) page = 0;", "if (page < 0) page = num_pages - 1;"),
    ("slot off by one", "* page_size + j % page_size) * D;", "* page_size + (j + 1) % page_size) * D;"),
    ("Q layout transposed", "const size_t qoff = (((size_t)b * S + s) * Hq + h) * D;",
     "const size_t qoff = (((size_t)b * Hq + h) * S + s) * D;"),
    ("block K/V index transposed", "off[j] = (((size_t)b * S + (j - L)) * Hkv + g) * D;",
     "off[j] = (((size_t)(j - L) * Hkv + g) * S + b) * D;"),
    ("LSE without max", "LSE[r] = m + log(Z);", "LSE[r] = log(Z);"),
    ("softmax not normalised", "const double w = exp(sc[j] - m) / Z;", "const double w = exp(sc[j] - m);"),
    ("bf16 decode shift", "<< 16;", "<< 15;"),
    ("merge weight sign", "const double w = exp(l - M);", "const double w = exp(M - l);"),
    ("merge LSE without max", "lse[i] = M + log(W);", "lse[i] = log(W);"),
    ("merge not normalised", "for (int k = 0; k < D; ++k) o[k] /= W;", ""),
    ("argmax takes last tie", "if (x > m) { m = x; a = v; }", "if (x >= m) { m = x; a = v; }"),
    ("temperature ignored", "Z += exp((ld(logits, base + v, dtype) - m) / temperature);",
     "Z += exp(ld(logits, base + v, dtype) - m);"),
    ("threshold not strict", "if (mk[l]) { ++M; if (cf[l] > gamma) ++n_pass; }",
     "if (mk[l]) { ++M; if (cf[l] >= gamma) ++n_pass; }"),
    ("commit not strict", "if (mk[l] && cf[l] > gamma) {", "if (mk[l] && cf[l] >= gamma) {"),
    ("k_min floor", "const int k_min = (M + steps_left - 1) / steps_left;",
     "const int k_min = M / steps_left;"),
    ("fallback tie to higher position", "(cf[ord[j]] == cf[cur] && ord[j] > cur)",
     "(cf[ord[j]] == cf[cur] && ord[j] < cur)"),
    ("fallback ascending", "while (j >= 0 && (cf[ord[j]] < cf[cur]", "while (j >= 0 && (cf[ord[j]] > cf[cur]"),
    ("num_masked not updated", "num_masked_out[b] = M - committed;", "num_masked_out[b] = M;"),
    ("fallback commits one", "for (int i = 0; i < k_min; ++i) {", "for (int i = 0; i < 1 && i < k_min; ++i) {"),
    ("append slot off by one", "const int slot = j % page_size;", "const int slot = (j + 1) % page_size;"),
    ("append pool from the bottom", "if (*e < 0) *e = pool[count - 1 - k++];", "if (*e < 0) *e = pool[k++];"),
    ("append ctx_len not grown", "ctx_len[b] = L + S;", "ctx_len[b] = L;"),
    ("append capacity off by one", "if ((long long)L + S > cap) return 1;", "if ((long long)L + S >= cap) return 1;"),
    ("append V from K", "memcpy(Vc + dst, Vn + src, row);", "memcpy(Vc + dst, Kn + src, row);"),
    ("append pool count kept", "if (needed > 0) *pool_count = count - needed;", ""),
    ("append new-row index transposed", "const size_t src = (((size_t)b * S + s) * Hkv + g) * row;",
     "const size_t src = (((size_t)s * B + b) * Hkv + g) * row;"),
    ("nll without the max", "? m + log(Z) - ld(logits, base + y, dtype) : NAN;", "? log(Z) - ld(logits, base + y, dtype) : NAN;"),
    ("nll target sign", "? m + log(Z) - ld(logits, base + y, dtype) : NAN;", "? m + log(Z) + ld(logits, base + y, dtype) : NAN;"),
    ("nll mean over every row", "*loss_out = count > 0 ? sum / count : 0.0;",
     "*loss_out = count > 0 ? sum / ((double)B * S) : 0.0;"),
    ("sample cumulative not strict", "if (a < 0 && Cn > t) {", "if (a < 0 && Cn >= t) {"),
    ("sample without temperature", "e[v] = exp((ld(logits, base + v, dtype) - m) / temperature);",
     "e[v] = exp(ld(logits, base + v, dtype) - m);"),
    ("sample conf of the max", "*conf = e_a / Z;", "*conf = 1.0 / Z;"),
    ("sample fallback to the last index", "if (a < 0) { a = last;", "if (a < 0) { a = V - 1;"),
    ("sample u not scaled by Z", "const double t = u * Z;", "const double t = u;"),
    ("sample reversed order", "const double Cn = C + e[v];", "const double Cn = C + e[V - 1 - v];"),
    ("nll at temperature 2", "Z += exp(ld(logits, base + v, dtype) - m);", "Z += exp((ld(logits, base + v, dtype) - m) / 2);"),
    ("nll counts unmasked rows", "if (!mask[row]) continue;", "if (!mask[row] && row > 0) continue;"),
]


def _build(tmp, name, text):
    src = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", src, "-o", lib, "-lm"],
                   check=True, capture_output=True)
    return lib


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation target for '{name}' not found exactly once in the oracle"
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build(tmp, "mutant", text.replace(old, new))
        caught = []
        with oracle.use_library(lib):
            for pin in pins.ALL_PINS:
                try:
                    pin()
                except (AssertionError, ValueError):
                    caught.append(pin.__name__)
        assert caught, f"no pin detects the mutant '{name}'"


def test_unmutated_copy_passes():
    """Control: the same build path with no edit passes every pin."""
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build(tmp, "clean", open(SRC).read())
        with oracle.use_library(lib):
            for pin in pins.ALL_PINS:
                pin()
