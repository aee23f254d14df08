"""The pins are strong enough: each plausible mistake, planted in a copy of the
oracle's C source and compiled on the CPU, fails at least one of them.

The planted mistakes: the interleaved nibble order instead of split-half, a
dropped or reversed offset of 8, a big-endian scale, a wrong scale index, a
dropped last term, transposed activation or output indexing, a wrong
binary16 exponent bias or subnormal scale, a signed magnitude sum; in the
W4A8 part, ties rounded away from zero, a 255 instead of a 127 scale, a
signed maximum, a dropped offset, the first block's activation scale.

The oracle's Python helpers get their own planted mistakes (PY_MUTANTS):
the acceptance ratio taken norm-wise, as a mean, against |y_ref|, without
the absolute value, without the den = 0 or the non-finite rule; the greedy
pick keeping the last of equal values or letting NaN win; the pick's
tolerance test with a one-sided budget or none.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
import synth
from test_oracle_pins import (GOLDEN_CASES, _brute_w4a8, _golden_blocks, brute_force,
                              ratio_battery)

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


# ---- planted mistakes in the oracle's Python helpers ----------------------
def _ratio_norm_wise(y, y_ref, den):
    """max |err| / max den (a norm-wise ratio)"""
    return float(np.max(np.abs(y - y_ref)) / np.max(den))


def _ratio_mean(y, y_ref, den):
    nz = den != 0
    if np.any(~nz & (y != 0)) or not np.all(np.isfinite(y[nz])):
        return float("inf")
    return float(np.mean(np.abs(y - y_ref)[nz] / den[nz])) if nz.any() else 0.0


def _ratio_vs_ref(y, y_ref, den):
    nz = den != 0
    if np.any(~nz & (y != 0)) or not np.all(np.isfinite(y[nz])):
        return float("inf")
    return float(np.max(np.abs(y - y_ref)[nz] / np.abs(y_ref[nz]))) if nz.any() else 0.0


def _ratio_signed(y, y_ref, den):
    nz = den != 0
    if np.any(~nz & (y != 0)) or not np.all(np.isfinite(y[nz])):
        return float("inf")
    return float(np.max((y - y_ref)[nz] / den[nz])) if nz.any() else 0.0


def _ratio_no_zero_rule(y, y_ref, den):
    nz = den != 0
    if not np.all(np.isfinite(y[nz])):
        return float("inf")
    return float(np.max(np.abs(y - y_ref)[nz] / den[nz])) if nz.any() else 0.0


def _ratio_nan_ignored(y, y_ref, den):
    nz = den != 0
    if np.any(~nz & (y != 0)):
        return float("inf")
    return float(np.nanmax(np.abs(y - y_ref)[nz] / den[nz])) if nz.any() else 0.0


def _pick_last_of_ties(y_ref):
    vals, idxs = [], []
    for row in np.asarray(y_ref, np.float64):
        best, bi = -np.inf, -1
        for i, v in enumerate(row.tolist()):
            if v >= best and not np.isnan(v):
                best, bi = v, i
        vals.append(best if bi >= 0 else np.nan)
        idxs.append(bi)
    return np.array(vals), np.array(idxs)


def _pick_nan_wins(y_ref):
    vals, idxs = [], []
    for row in np.asarray(y_ref, np.float64):
        i = int(np.argmax(row))           # numpy's argmax returns the first NaN
        vals.append(row[i])
        idxs.append(i)
    return np.array(vals), np.array(idxs)


def _pick_battery(pick):
    y = np.array([[1.0, 3.0, 3.0, -2.0],
                  [np.nan, -1.0, -1.0, -5.0],
                  [np.nan, np.nan, np.nan, np.nan],
                  [-np.inf, -np.inf, -7.0, -np.inf]])
    v, i = pick(y)
    ok = (list(i) == [1, 1, -1, 2] and v[0] == 3.0 and v[1] == -1.0 and np.isnan(v[2])
          and v[3] == -7.0)
    return [] if ok else ["pick"]


def _within_one_sided(y_ref, den, idx, tol):
    best, bi = oracle.greedy_pick(y_ref)
    for t, i in enumerate(np.asarray(idx).tolist()):
        if i < 0 or i >= y_ref.shape[1]:
            return False
        if y_ref[t, i] < best[t] - tol * den[t, bi[t]]:
            return False
    return True


def _within_exact(y_ref, den, idx, tol):
    _, bi = oracle.greedy_pick(y_ref)
    return bool(np.all(np.asarray(idx) == bi))


def _within_battery(within):
    failed = []
    y = np.array([[1.0, 1.0 - 1e-9, 0.5]])
    den = np.full_like(y, 10.0)
    if not (within(y, den, np.array([0]), 1e-3) and within(y, den, np.array([1]), 1e-3)):
        failed.append("near_tie")
    if within(y, den, np.array([2]), 1e-3) or within(y, den, np.array([-1]), 1e-3):
        failed.append("far")
    # the budget is both outputs' errors: 1.5e-3 below the maximum, dens 1 and 1
    # (1e-3 each): inside 2e-3, outside a one-sided 1e-3
    y2 = np.array([[1.0, 1.0 - 1.5e-3]])
    if not within(y2, np.ones_like(y2), np.array([1]), 1e-3):
        failed.append("two_sided")
    return failed


PY_MUTANTS = {
    "ratio_norm_wise": ("max_ratio", _ratio_norm_wise),
    "ratio_mean": ("max_ratio", _ratio_mean),
    "ratio_vs_ref": ("max_ratio", _ratio_vs_ref),
    "ratio_signed": ("max_ratio", _ratio_signed),
    "ratio_no_zero_rule": ("max_ratio", _ratio_no_zero_rule),
    "ratio_nan_ignored": ("max_ratio", _ratio_nan_ignored),
    "pick_last_of_ties": ("greedy_pick", _pick_last_of_ties),
    "pick_nan_wins": ("greedy_pick", _pick_nan_wins),
    "within_one_sided": ("pick_within_tolerance", _within_one_sided),
    "within_exact": ("pick_within_tolerance", _within_exact),
}
PY_BATTERY = {"max_ratio": ratio_battery, "greedy_pick": _pick_battery,
              "pick_within_tolerance": _within_battery}


@pytest.mark.parametrize("fn", sorted(PY_BATTERY))
def test_unmutated_helpers_pass_battery(fn):
    assert PY_BATTERY[fn](getattr(oracle, fn)) == []


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_planted_helper_mistake_is_caught(name):
    fn, mutant = PY_MUTANTS[name]
    assert PY_BATTERY[fn](mutant), f"mutant {name} of {fn} passed every pin"
