"""Planted mistakes in the oracle turn its pins red (CPU only).

Each case copies hti_oracle.c, changes one expression the way a plausible
misreading or slip would, compiles the copy with the oracle's own flags, and
runs the pins through it.  The case passes when at least one pin fails on
the altered copy -- the evidence that the pins, and not only agreement
between the oracle and the kernels, fix that part of the method.  The
original source is untouched.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "hti_oracle.c")

# (name, text in hti_oracle.c, replacement, pins expected to catch it)
MUTANTS = [
    ("pooler temperature dropped",
     "    float scale = 1.0f / sqrtf((float)d);\n    float *a",
     "    float scale = 1.0f;\n    float *a", "pooler"),
    ("pooler temperature halved",
     "    float scale = 1.0f / sqrtf((float)d);\n    float *a",
     "    float scale = 0.5f / sqrtf((float)d);\n    float *a", "pooler"),
    ("pooler temperature doubled",
     "    float scale = 1.0f / sqrtf((float)d);\n    float *a",
     "    float scale = 2.0f / sqrtf((float)d);\n    float *a", "pooler"),
    ("pooler temperature 1/d",
     "    float scale = 1.0f / sqrtf((float)d);\n    float *a",
     "    float scale = 1.0f / (float)d;\n    float *a", "pooler"),
    ("every chain pooled with the first reference",
     "const float *r = refs + (size_t)j * d;",
     "const float *r = refs;", "pooler"),
    ("levels above the first pool the first reference's chain",
     "child0 = lvl_k[l - 2] + ((size_t)(i * fb) * R + j) * d;",
     "child0 = lvl_k[l - 2] + ((size_t)(i * fb) * R + 0) * d;", "pooler"),
    ("node ties go to the higher index",
     "return (a->pos < b->pos) ? -1 : (a->pos > b->pos);",
     "return (a->pos > b->pos) ? -1 : (a->pos < b->pos);", "ties"),
    ("reference ties go to the later reference",
     "if (gmean > best) { best = gmean; jbest = j; }",
     "if (gmean >= best) { best = gmean; jbest = j; }", "ties"),
    ("attention logits without the 1/sqrt(d) scale",
     "zt[j * G + h] = dot_seq(qr + (size_t)h * d, kr, d) * scale;",
     "zt[j * G + h] = dot_seq(qr + (size_t)h * d, kr, d);", "query"),
    ("summary values dropped from the shared softmax",
     "for (long i = 0; i < m && !A->leaf_only; ++i) {",
     "for (long i = 0; i < m && 0; ++i) {", "query"),
    # (fan mutants stay inside the arrays the pins allocate: the value mean of
    # the build, and traversal mutants checked only on trees where the wrong
    # fan-in reads fewer nodes than exist)
    ("values above the first level averaged over the chunk size",
     "acc = acc / (float)fb;",
     "acc = acc / (float)b;", "fan_build"),
    ("traversal descends with the chunk size at every level",
     "const int fb = (l == 1) ? A->b : A->fan;",
     "const int fb = A->b;", "fan_up"),
    ("traversal descends with the fan at level 1 too",
     "const int fb = (l == 1) ? A->b : A->fan;",
     "const int fb = A->fan;", "fan_down"),
]

PINS = {
    "pooler": [
        lambda: [P.test_pooler_temperature_closed_form(d) for d in (16, 36, 128)],
        lambda: P.test_pooler_per_reference_chains(4096 + 300, 4, 5, 3, 32),
        lambda: P.test_pooler_per_reference_chains(1000, 3, 6, 2, 16),
    ],
    "ties": [
        lambda: [P.test_exact_ties_topk(R) for R in (1, 2, 3)],
        lambda: [P.test_exact_ties_topp(p, c) for p, c in ((0.3, 16), (0.5, 2), (0.9, 16))],
    ],
    "query": [
        lambda: P.test_dense_equivalence_tiny_workload("topk"),
        lambda: P.test_prefill_matches_f64_entry_softmax(),
    ],
    "fan_build": [
        lambda: P.test_pooler_fanout_chains(3000, 8, 3, 4, 2, 32),
        lambda: P.test_pooler_fanout_chains(5000, 3, 16, 2, 2, 16),
    ],
    "fan_up": [lambda: P.check_fanout_cases(lambda b, fan: b < fan)],
    "fan_down": [lambda: P.check_fanout_cases(lambda b, fan: fan < b)],
}


def _build_mutant(tmp_path, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique / missing: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-shared", "-fPIC", "-o", lib, str(path), "-lm"])
    return lib


@pytest.mark.parametrize("name,old,new,kind", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, kind):
    lib = _build_mutant(tmp_path, old, new)
    caught = []
    with oracle.library(lib):
        for pin in PINS[kind]:
            try:
                pin()
            except AssertionError:
                caught.append(pin)
    assert caught, f"no pin fails on the oracle with '{name}'"


def test_unaltered_copy_passes(tmp_path):
    """The same harness on an unaltered copy: every pin passes."""
    lib = _build_mutant(tmp_path, "#include <math.h>", "#include <math.h>")
    with oracle.library(lib):
        for pins in PINS.values():
            for pin in pins:
                pin()
