"""The pins are strong enough: each plausible mistake, planted in a copy of the
oracle's C source and compiled on the CPU, fails at least one of them.

The planted mistakes: the interleaved nibble order instead of split-half, a
dropped or reversed offset of 8, a big-endian scale, a wrong scale index, a
dropped last term, transposed activation or output indexing, a wrong
binary16 exponent bias or subnormal scale, a signed magnitude sum.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
import synth
from test_oracle_pins import (GOLDEN_CASES, _golden_blocks, brute_force)

SRC = open(obuild.SRC).read()

MUTANTS = {
    "interleaved_nibbles": (
        "return (j < 16) ? (qs[j] & 0x0f) : (qs[j - 16] >> 4);",
        "return (j & 1) ? (qs[j >> 1] >> 4) : (qs[j >> 1] & 0x0f);"),
    "no_offset": ("(float)(q4o_code(qs, j) - 8)", "(float)(q4o_code(qs, j))"),
    "reversed_offset": ("(float)(q4o_code(qs, j) - 8)", "(float)(8 - q4o_code(qs, j))"),
    "big_endian_scale": ("(uint16_t)(blk[0] | (blk[1] << 8))",
                         "(uint16_t)(blk[1] | (blk[0] << 8))"),
    "scale_of_first_block": (
        "float d = q4o_half_to_float((uint16_t)(blk[0] | (blk[1] << 8)));",
        "const uint8_t *b0 = blocks + o * nb * Q4O_BLOCK_BYTES;"
        " float d = q4o_half_to_float((uint16_t)(b0[0] | (b0[1] << 8)));"),
    "dropped_last_term": ("for (int64_t k = 0; k < j->in; ++k) {",
                          "for (int64_t k = 0; k < j->in - 1; ++k) {"),
    "transposed_x": ("double p = (double)w[k] * (double)xt[k];",
                     "double p = (double)w[k] * (double)j->x[k * j->n + t];"),
    "transposed_y": ("j->y[t * j->nrows + i] = acc;", "j->y[i * j->n + t] = acc;"),
    "half_bias": ("v = ldexpf((float)(1024 + f), e - 25);",
                  "v = ldexpf((float)(1024 + f), e - 24);"),
    "half_subnormal": ("v = ldexpf((float)f, -24);", "v = ldexpf((float)f, -25);"),
    "signed_den": ("mag += fabs(p);", "mag += p;"),
}


def battery(o):
    """Run the pins against oracle build ``o``; return the names that fail."""
    failed = []
    # binary16 decoder against numpy on every pattern
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ref = ref.astype(np.float32)
    got = np.array([o.half_to_float(b) for b in range(65536)], np.float32)
    fin = ~np.isnan(ref)
    if not (np.array_equal(np.isnan(got), ~fin) and
            np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))):
        failed.append("half")
    # all codes 8 -> zero
    blk = synth.make_blocks(5, 64, seed=3)
    blk[..., 2:] = 0x88
    y, den = o.matmul(blk, synth.make_x(2, 64, seed=4), 5, 64)
    if not (np.all(y == 0) and np.all(den == 0)):
        failed.append("zero")
    # golden one-hot examples
    for case in GOLDEN_CASES:
        b = _golden_blocks(case)
        for k, expect in case["onehot"]:
            x = np.zeros((1, case["in"]), np.float32)
            x[0, k] = 1.0
            y, _ = o.matmul(b, x, case["out"], case["in"])
            if y[0].tolist() != expect:
                failed.append("golden")
                break
    # exact brute force, n > 1 and out > 1
    from fractions import Fraction
    for seed in range(2):
        blk = synth.make_blocks(3, 64, seed=seed)
        x = synth.make_x(2, 64, seed=seed)
        y, den = o.matmul(blk, x, 3, 64)
        ye, de = brute_force(blk, x)
        ok = all(abs(Fraction(y[t, r]) - ye[t][r]) <= Fraction(1e-12) * de[t][r]
                 and abs(den[t, r] - float(de[t][r])) <= 1e-12 * float(de[t][r])
                 for t in range(2) for r in range(3))
        if not ok:
            failed.append("brute")
            break
    return failed


def test_unmutated_oracle_passes_battery():
    assert battery(oracle.default()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "mut.c")
        with open(src, "w") as f:
            f.write(SRC.replace(old, new))
        lib = obuild.build(src=src, lib=os.path.join(tmp, "libmut.so"))
        failed = battery(oracle.Oracle(lib))
    assert failed, f"mutant {name} passed every pin"
