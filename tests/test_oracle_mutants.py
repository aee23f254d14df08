"""The pins are strong enough: each plausible mistake, planted in a copy of the
oracle's C source and compiled on the CPU, fails at least one of them.

The planted mistakes: the interleaved nibble order instead of split-half, a
dropped or reversed offset of 8, a big-endian scale, a wrong scale index, a
dropped last term, transposed activation or output indexing, a wrong
binary16 exponent bias or subnormal scale, a signed magnitude sum; in the
W4A8 part, ties rounded away from zero, a 255 instead of a 127 scale, a
signed maximum, a dropped offset, the first block's activation scale.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
import synth
from test_oracle_pins import (GOLDEN_CASES, _brute_w4a8, _golden_blocks, brute_force)

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
    "x8_ties_away": ("(int8_t)rintf(xb[j] / s)", "(int8_t)roundf(xb[j] / s)"),
    "x8_scale_255": ("float s = amax / 127.0f;", "float s = amax / 255.0f;"),
    "x8_signed_max": ("float a = fabsf(xb[j]);", "float a = xb[j];"),
    "w4a8_no_offset": ("(int64_t)(q4o_code(blk + 2, k) - 8) * (int64_t)qx[k]",
                       "(int64_t)(q4o_code(blk + 2, k)) * (int64_t)qx[k]"),
    "w4a8_first_dx": ("double dx = (double)j->d[t * nb + b];",
                      "double dx = (double)j->d[t * nb];"),
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
    # W4A8: hand-worked quantizer block, reconstruction bound, brute force
    xq = np.array([[127.0, 0.5, 1.5, 2.5, -1.5, -127.0, 63.5, -0.49] + [0.0] * 24 +
                   [-3.0, 1.0] + [0.0] * 30], np.float32)
    q, d = o.quantize_x8(xq)
    if q[0, :8].tolist() != [127, 0, 2, 2, -2, -127, 64, 0] or d[0, 1] != np.float32(3) / 127:
        failed.append("x8_hand")
    xr = synth.make_x(2, 128, seed=5)
    q, d = o.quantize_x8(xr)
    dd = np.repeat(d.astype(np.float64), 32, axis=1)
    if not (np.all(np.abs(xr - q * dd) <= dd * (0.5 + 1e-5)) and np.abs(q).max() == 127):
        failed.append("x8_bound")
    blk = synth.make_blocks(3, 64, seed=8)
    q, d = o.quantize_x8(synth.make_x(2, 64, seed=8))
    y, den = o.matmul_w4a8(blk, q, d, 3, 64)
    ye, de = _brute_w4a8(blk.reshape(3, 2, 18), q, d)
    if not all(abs(Fraction(y[t, r]) - ye[t][r]) <= Fraction(1e-12) * de[t][r]
               for t in range(2) for r in range(3)):
        failed.append("w4a8_brute")
    return failed


def test_unmutated_oracle_passes_battery():
    assert battery(oracle.default()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "mut.c")
        with open(src, "w") as f:
            f.write(SRC.replace(old, new))
        lib = obuild.build(src=src, lib=os.path.join(tmp, "libmut.so"))
        failed = battery(oracle.Oracle(lib))
    assert failed, f"mutant {name} passed every pin"
