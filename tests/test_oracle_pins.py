"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against something the pages or the mathematics fix:
  - the binary16 decoder against numpy's conversion on all 65536 patterns;
  - all codes 8 give y = 0 exactly (every weight is d * 0);
  - d = 1 and all codes 9 give the row sum of x; constant codes c and constant
    d give d * (c - 8) * sum(x), against an independently rounded sum;
  - exact rational brute force on tiny shapes, with a decoder written here
    from the split-half rule of goinfer primer ch. 10 "Layout, concretely";
  - a vectorised numpy decode and a float64 library matmul at full sizes;
  - the hand-worked one-hot examples in tests/golden/;
  - invariants: linearity in x, exact power-of-two scaling of d, x = 0,
    independence of a token's result from the other tokens, row subsets,
    binary16 activations, IEEE propagation of Inf/NaN scales.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "q4_0_split_half_onehot.txt")


# ---------------------------------------------------------------- decoders
def _f16_bits_to_fraction(lo: int, hi: int) -> Fraction:
    """binary16 scale -> exact Fraction via the struct module's decoder."""
    return Fraction(struct.unpack("<e", bytes([lo, hi]))[0])


def brute_force(blocks: np.ndarray, x: np.ndarray):
    """Exact y and den as Fractions, decoded here independently of the oracle.

    blocks: uint8 [out, nb, 18]; x: [n, in] float32/float16.
    Split-half rule: code byte i of a block carries weight i in its low four
    bits and weight i + 16 in its high four bits; weight = d * (q - 8).
    """
    out, nb, _ = blocks.shape
    in_ = nb * 32
    n = x.shape[0]
    xs = [[Fraction(float(v)) for v in row] for row in x.astype(np.float64)]
    y = [[Fraction(0)] * out for _ in range(n)]
    den = [[Fraction(0)] * out for _ in range(n)]
    for o in range(out):
        w = [Fraction(0)] * in_
        for b in range(nb):
            blk = [int(v) for v in blocks[o, b]]
            d = _f16_bits_to_fraction(blk[0], blk[1])
            for i in range(16):
                byte = blk[2 + i]
                w[32 * b + i] = d * ((byte & 0x0F) - 8)
                w[32 * b + 16 + i] = d * ((byte >> 4) - 8)
        for t in range(n):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(in_):
                p = w[k] * xs[t][k]
                acc += p
                mag += abs(p)
            y[t][o] = acc
            den[t][o] = mag
    return y, den


def numpy_dequant(blocks: np.ndarray) -> np.ndarray:
    """Vectorised decode to float64 [out, in] (a third, independent decoder)."""
    out, nb, _ = blocks.shape
    d = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    qs = blocks[..., 2:].astype(np.int16)
    lo = (qs & 0x0F) - 8                      # weights 0..15 of each block
    hi = (qs >> 4) - 8                        # weights 16..31
    q = np.concatenate([lo, hi], axis=-1)     # [out, nb, 32]
    return (d[..., None] * q).reshape(out, nb * 32)


# ---------------------------------------------------------------- binary16
def test_half_decoder_matches_numpy_on_all_patterns():
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ref = ref.astype(np.float32)
    o = oracle.default()
    got = np.array([o.half_to_float(b) for b in range(65536)], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("n,out,in_", [(1, 7, 32), (3, 33, 320), (2, 16, 2560)])
def test_all_codes_eight_give_exact_zero(n, out, in_):
    blk = synth.make_blocks(out, in_, seed=3)
    blk[..., 2:] = 0x88                       # q = 8 in both nibbles
    x = synth.make_x(n, in_, seed=4)
    y, den = oracle.matmul(blk, x, out, in_)
    assert np.all(y == 0.0) and np.all(den == 0.0)


@pytest.mark.parametrize("n,out,in_", [(1, 4, 32), (4, 9, 1024), (2, 3, 9728)])
def test_unit_scale_code_nine_gives_row_sum(n, out, in_):
    blk = synth.constant_blocks(out, in_, d_bits=0x3C00, code_byte=0x99)
    x = synth.make_x(n, in_, seed=5)
    y, den = oracle.matmul(blk, x, out, in_)
    for t in range(n):
        s = math.fsum(float(v) for v in x[t])           # correctly rounded
        a = math.fsum(abs(float(v)) for v in x[t])
        bound = in_ * 2.0 ** -52 * a
        assert np.all(np.abs(y[t] - s) <= bound)
        assert np.allclose(den[t], a, rtol=1e-12, atol=0)


@pytest.mark.parametrize("code", range(16))
def test_constant_code_constant_scale(code):
    out, in_, n = 5, 96, 2
    d = 0.375                                          # exact in binary16
    d_bits = int(np.array(d, dtype=np.float16).view(np.uint16))
    blk = synth.constant_blocks(out, in_, d_bits, code | (code << 4))
    x = synth.make_x(n, in_, seed=6)
    y, den = oracle.matmul(blk, x, out, in_)
    for t in range(n):
        exact = Fraction(d) * (code - 8) * sum(Fraction(float(v)) for v in x[t])
        mag = Fraction(d) * abs(code - 8) * sum(abs(Fraction(float(v))) for v in x[t])
        assert np.all(np.abs(y[t] - float(exact)) <= 1e-13 * float(mag) + 0.0)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("in_", [32, 64, 96])
def test_exact_rational_brute_force(seed, in_):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 4))
    out = int(rng.integers(1, 6))
    blk = synth.make_blocks(out, in_, seed=seed)
    # widen the scale range so signs, large and tiny scales all appear
    d = rng.uniform(-4, 4, size=(out, in_ // 32)).astype(np.float16)
    blk[..., 0:2] = d.view(np.uint8).reshape(out, in_ // 32, 2)
    x = synth.make_x(n, in_, seed=seed).astype(
        np.float16 if seed % 2 else np.float32)
    y, den = oracle.matmul(blk, x, out, in_)
    ye, dene = brute_force(blk, x)
    for t in range(n):
        for o in range(out):
            mag = float(dene[t][o])
            assert den[t, o] == pytest.approx(mag, rel=1e-13, abs=0)
            assert abs(Fraction(y[t, o]) - ye[t][o]) <= Fraction(1e-12) * dene[t][o]


def test_dequantize_matches_brute_force_decoder():
    blk = synth.make_blocks(6, 128, seed=11)
    w = oracle.dequantize(blk, 6, 128).astype(np.float64)
    assert np.array_equal(w, numpy_dequant(blk))


# ---------------------------------------------------------------- library
@pytest.mark.parametrize("out,in_,n", [(1024, 1024, 1), (9728, 2560, 1)])
def test_numpy_float64_matmul_at_full_size(out, in_, n):
    blk = synth.make_blocks(out, in_, seed=0)
    x = synth.make_x(n, in_, seed=0)
    y, den = oracle.matmul(blk, x, out, in_)
    w = numpy_dequant(blk)
    y_np = x.astype(np.float64) @ w.T
    den_np = np.abs(x.astype(np.float64)) @ np.abs(w).T
    assert np.all(np.abs(y - y_np) <= 1e-12 * den_np)
    assert np.allclose(den, den_np, rtol=1e-12, atol=0)


# ---------------------------------------------------------------- golden
def _parse_golden(path):
    cases, cur = [], None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "blocks": [], "onehot": []}
        elif tok[0] == "shape":
            cur["out"], cur["in"] = int(tok[1]), int(tok[2])
        elif tok[0] == "block":
            cur["blocks"].append((int(tok[1]), int(tok[2]), int(tok[3], 16),
                                  bytes.fromhex(tok[4])))
        elif tok[0] == "onehot":
            cur["onehot"].append((int(tok[1]), [float(v) for v in tok[2:]]))
        elif tok[0] == "end":
            cases.append(cur)
    return cases


def _golden_blocks(case):
    out, in_ = case["out"], case["in"]
    blk = synth.constant_blocks(out, in_, 0x3C00, 0x88)
    for row, b, d_bits, qs in case["blocks"]:
        blk[row, b, 0] = d_bits & 0xFF
        blk[row, b, 1] = d_bits >> 8
        blk[row, b, 2:] = np.frombuffer(qs, dtype=np.uint8)
    return blk


GOLDEN_CASES = _parse_golden(GOLDEN)


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=[c["name"] for c in GOLDEN_CASES])
def test_golden_split_half_onehot(case):
    out, in_ = case["out"], case["in"]
    blk = _golden_blocks(case)
    for k, expect in case["onehot"]:
        x = np.zeros((1, in_), dtype=np.float32)
        x[0, k] = 1.0
        y, _ = oracle.matmul(blk, x, out, in_)
        assert y[0].tolist() == expect, (case["name"], k)


def test_golden_file_is_not_trivial():
    assert len(GOLDEN_CASES) >= 3
    assert sum(len(c["onehot"]) for c in GOLDEN_CASES) >= 20


# ---------------------------------------------------------------- invariants
def test_linearity_in_x():
    out, in_ = 37, 640
    blk = synth.make_blocks(out, in_, seed=21)
    x1 = synth.make_x(2, in_, seed=22)
    x2 = synth.make_x(2, in_, seed=23)
    a, b = 0.75, -2.5
    xc = (a * x1.astype(np.float64) + b * x2.astype(np.float64))
    y1, d1 = oracle.matmul(blk, x1, out, in_)
    y2, d2 = oracle.matmul(blk, x2, out, in_)
    yc, _ = oracle.matmul(blk, xc.astype(np.float32), out, in_)
    # xc rounded to float32: allow that rounding plus fp64 accumulation
    tol = 2.0 ** -23 * (abs(a) * d1 + abs(b) * d2) * 2
    assert np.all(np.abs(yc - (a * y1 + b * y2)) <= tol)


@pytest.mark.parametrize("shift", [-3, 1, 4])
def test_power_of_two_scale_of_d_scales_y_exactly(shift):
    out, in_ = 19, 256
    blk = synth.make_blocks(out, in_, seed=31)
    x = synth.make_x(3, in_, seed=32)
    d = blk[..., 0:2].copy().view(np.float16)
    d2 = (d.astype(np.float32) * 2.0 ** shift).astype(np.float16)
    assert np.array_equal(d2.astype(np.float32), d.astype(np.float32) * 2.0 ** shift)
    blk2 = blk.copy()
    blk2[..., 0:2] = d2.view(np.uint8)
    y, _ = oracle.matmul(blk, x, out, in_)
    y2, _ = oracle.matmul(blk2, x, out, in_)
    assert np.array_equal(y2, y * 2.0 ** shift)


def test_zero_x_gives_zero():
    blk = synth.make_blocks(10, 64, seed=41)
    y, den = oracle.matmul(blk, np.zeros((2, 64), np.float32), 10, 64)
    assert np.all(y == 0) and np.all(den == 0)


def test_token_results_independent_of_batch():
    out, in_ = 50, 512
    blk = synth.make_blocks(out, in_, seed=51)
    x = synth.make_x(8, in_, seed=52)
    y8, d8 = oracle.matmul(blk, x, out, in_)
    for t in (0, 5, 7):
        y1, d1 = oracle.matmul(blk, x[t:t + 1], out, in_)
        assert np.array_equal(y1[0], y8[t]) and np.array_equal(d1[0], d8[t])


def test_row_subset_and_thread_count_agree_bitwise():
    out, in_ = 300, 320
    blk = synth.make_blocks(out, in_, seed=61)
    x = synth.make_x(3, in_, seed=62)
    y, den = oracle.matmul(blk, x, out, in_, nthreads=1)
    y4, den4 = oracle.matmul(blk, x, out, in_, nthreads=4)
    assert np.array_equal(y, y4) and np.array_equal(den, den4)
    rows = np.array([299, 0, 17, 17, 150], dtype=np.int64)
    ys, ds = oracle.matmul(blk, x, out, in_, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(ds, den[:, rows])


def test_f16_activations_equal_their_f32_upcast():
    out, in_ = 40, 384
    blk = synth.make_blocks(out, in_, seed=71)
    xh = synth.make_x(5, in_, seed=72, dtype=np.float16)
    ya, da = oracle.matmul(blk, xh, out, in_)
    yb, db = oracle.matmul(blk, xh.astype(np.float32), out, in_)
    assert np.array_equal(ya, yb) and np.array_equal(da, db)


def test_inf_and_nan_scales_propagate():
    out, in_ = 3, 64
    blk = synth.constant_blocks(out, in_, 0x3C00, 0x99)
    blk[0, 1, 0:2] = [0x00, 0x7C]             # +Inf scale, codes 9 -> +Inf
    blk[1, 0, 0:2] = [0x00, 0x7E]             # NaN scale
    blk[2, 0, 0:2] = [0x00, 0x7C]
    blk[2, 0, 2:] = 0x88                      # Inf * 0 -> NaN
    x = np.ones((1, in_), np.float32)
    y, _ = oracle.matmul(blk, x, out, in_)
    assert y[0, 0] == np.inf
    assert np.isnan(y[0, 1]) and np.isnan(y[0, 2])


def test_rejects_shapes_that_are_not_whole_blocks():
    o = oracle.default()
    blk = np.zeros(18, np.uint8)
    with pytest.raises(ValueError):
        o.matmul(blk, np.zeros((1, 33), np.float32), 1, 33)
    assert o.lib.q4o_dequantize(None, 1, 48, None) == -1


def test_brute_force_detects_nibble_order_swap():
    """The independent decoder used above is itself sensitive to the order:
    swapping the nibbles of every byte changes the exact result."""
    blk = synth.make_blocks(2, 32, seed=81)
    x = synth.make_x(1, 32, seed=82)
    ya, _ = brute_force(blk, x)
    sw = blk.copy()
    sw[..., 2:] = ((blk[..., 2:] & 0x0F) << 4) | (blk[..., 2:] >> 4)
    yb, _ = brute_force(sw, x)
    assert ya != yb


def test_greedy_pick_brute_force_ties_and_nan():
    """The pick: largest value, smallest index among ties, NaN never wins."""
    y = np.array([[1.0, 3.0, 3.0, -2.0],
                  [np.nan, -1.0, -1.0, -5.0],
                  [np.nan, np.nan, np.nan, np.nan],
                  [-np.inf, -np.inf, -7.0, -np.inf]])
    v, i = oracle.greedy_pick(y)
    assert i.tolist() == [1, 1, -1, 2]
    assert v[0] == 3.0 and v[1] == -1.0 and np.isnan(v[2]) and v[3] == -7.0
    rng = np.random.default_rng(5)
    z = rng.integers(-3, 4, size=(20, 9)).astype(np.float64)
    v, i = oracle.greedy_pick(z)
    for t in range(z.shape[0]):
        m = max(z[t])
        assert v[t] == m and i[t] == min(k for k in range(9) if z[t, k] == m)


def test_pick_within_tolerance_accepts_near_ties_only():
    y = np.array([[1.0, 1.0 - 1e-9, 0.5]])
    den = np.full_like(y, 10.0)
    assert oracle.pick_within_tolerance(y, den, np.array([0]), 1e-3)
    assert oracle.pick_within_tolerance(y, den, np.array([1]), 1e-3)   # within budget
    assert not oracle.pick_within_tolerance(y, den, np.array([2]), 1e-3)
    assert not oracle.pick_within_tolerance(y, den, np.array([-1]), 1e-3)


# ------------------------------------------------- the acceptance ratio
# The tolerance of the product's contract is per output: |y - y_ref| divided
# by that output's own sum of |w x|, maximised over every (row, output) pair;
# an output whose every product is zero must come out exactly zero.  Each
# case below is worked by hand and names what a plausible mistake in
# max_ratio would change.
RATIO_CASES = [
    # (name, y, y_ref, den, expected)
    # per-output, not norm-wise: 0.5 / 1 = 0.5; max|err| / max(den) = 0.005
    ("per_output", [[1.5, 100.0]], [[1.0, 100.0]], [[1.0, 100.0]], 0.5),
    # the ratio of a small error on a small den beats a large error on a
    # large den: max(1/100, 0.1/0.1) = 1; max|err| / den(argmax err) = 0.01
    ("small_den_wins", [[101.0, 0.2]], [[100.0, 0.1]], [[100.0, 0.1]], 1.0),
    # absolute value: y below y_ref counts the same
    ("below_ref", [[1.5]], [[2.0]], [[1.0]], 0.5),
    # den = 0 with y = 0 is ignored; the other output decides: 0.5 / 2
    ("zero_den_zero_y", [[0.0, 1.5]], [[0.0, 1.0]], [[0.0, 2.0]], 0.25),
    # den = 0 with y != 0, however small: infinite
    ("zero_den_nonzero_y", [[1e-30, 1.0]], [[0.0, 1.0]], [[0.0, 1.0]], float("inf")),
    # a NaN or an infinity where den > 0: infinite
    ("nan_y", [[float("nan"), 1.0]], [[0.0, 1.0]], [[1.0, 1.0]], float("inf")),
    ("inf_y", [[1.0, float("inf")]], [[1.0, 1.0]], [[1.0, 1.0]], float("inf")),
    # every den 0 and every y 0: nothing to compare, 0
    ("all_zero", [[0.0, 0.0], [0.0, 0.0]], [[0.0, 0.0], [0.0, 0.0]],
     [[0.0, 0.0], [0.0, 0.0]], 0.0),
    # maximum over rows and outputs, each error against its own den:
    # errors [[0.1, 0.2], [0.3, 0.0]], dens [[1, 4], [2, 1]] -> 0.15
    ("two_rows", [[1.1, 2.2], [3.3, 4.0]], [[1.0, 2.0], [3.0, 4.0]],
     [[1.0, 4.0], [2.0, 1.0]], 0.15),
]


def ratio_battery(fn):
    """Names of the hand-worked cases on which fn(y, y_ref, den) is wrong."""
    failed = []
    for name, y, y_ref, den, expect in RATIO_CASES:
        got = fn(np.array(y, np.float64), np.array(y_ref, np.float64),
                 np.array(den, np.float64))
        if expect == float("inf"):
            ok = got == float("inf")
        else:
            ok = abs(got - expect) <= 1e-12 * max(1.0, expect)
        if not ok:
            failed.append(name)
    return failed


def test_max_ratio_hand_worked_cases():
    assert ratio_battery(oracle.max_ratio) == []


def test_max_ratio_is_the_per_output_maximum_on_random_data():
    """On random data the ratio equals a plain loop over the outputs."""
    rng = np.random.default_rng(11)
    y_ref = rng.standard_normal((3, 40))
    den = np.abs(rng.standard_normal((3, 40))) + 0.01
    y = y_ref + rng.standard_normal((3, 40)) * 1e-4
    expect = 0.0
    for t in range(3):
        for o in range(40):
            expect = max(expect, abs(y[t, o] - y_ref[t, o]) / den[t, o])
    assert oracle.max_ratio(y, y_ref, den) == expect


# ------------------------------------------------------------------- W4A8
def test_quantize_x8_hand_worked_block():
    """amax 127 gives d = 1 exactly, so the codes are x rounded to nearest,
    ties to even; the largest magnitude maps to +-127."""
    blockv = [127.0, 0.5, 1.5, 2.5, -1.5, -127.0, 63.5, -0.49, 3.0, 126.5] + [0.0] * 22
    x = np.array([blockv], dtype=np.float32)
    q, d = oracle.quantize_x8(x)
    assert d[0, 0] == 1.0
    assert q[0, :10].tolist() == [127, 0, 2, 2, -2, -127, 64, 0, 3, 126]
    assert not q[0, 10:].any()


def test_quantize_x8_zero_and_nan_blocks():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 40] = np.nan
    x[1, 41] = 5.0
    x[1, 3] = 2.0
    q, d = oracle.quantize_x8(x)
    assert d[0].tolist() == [0.0, 0.0] and not q[0].any()
    assert np.isnan(d[1, 1]) and not q[1, 32:].any()      # NaN block: codes 0
    assert d[1, 0] == np.float32(2.0) / np.float32(127.0) and q[1, 3] == 127


@pytest.mark.parametrize("scale", [1e-30, 1e-3, 1.0, 1e4, 1e30])
def test_quantize_x8_reconstruction_bound_and_order(scale):
    """|x - q d| <= d/2 (plus float32 rounding of d), |q| <= 127 with the
    block's largest magnitude at +-127, and codes ordered as the values."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((5, 256)) * scale).astype(np.float32)
    q, d = oracle.quantize_x8(x)
    xb = x.reshape(5, 8, 32).astype(np.float64)
    qb = q.reshape(5, 8, 32).astype(np.float64)
    dd = d.astype(np.float64)[..., None]
    assert np.all(np.abs(qb) <= 127)
    assert np.all(np.abs(xb - qb * dd) <= dd * (0.5 + 1e-5))
    top = np.abs(xb).argmax(axis=-1)
    assert np.all(np.abs(np.take_along_axis(qb, top[..., None], -1)) == 127)
    order = np.argsort(xb, axis=-1, kind="stable")
    assert np.all(np.diff(np.take_along_axis(qb, order, -1), axis=-1) >= 0)


def _brute_w4a8(blocks, q, d):
    """Exact W4A8 y and den as Fractions, decoded here (split-half rule)."""
    out, nb, _ = blocks.shape
    n = q.shape[0]
    y = [[Fraction(0)] * out for _ in range(n)]
    den = [[Fraction(0)] * out for _ in range(n)]
    for o in range(out):
        for t in range(n):
            acc = mag = Fraction(0)
            for b in range(nb):
                blk = [int(v) for v in blocks[o, b]]
                dw = _f16_bits_to_fraction(blk[0], blk[1])
                dx = Fraction(float(d[t, b]))
                codes = [(blk[2 + i] & 0x0F) for i in range(16)] + \
                        [(blk[2 + i] >> 4) for i in range(16)]
                s = sum((c - 8) * int(q[t, 32 * b + i]) for i, c in enumerate(codes))
                a = sum(abs((c - 8) * int(q[t, 32 * b + i])) for i, c in enumerate(codes))
                acc += dw * dx * s
                mag += abs(dw * dx) * a
            y[t][o], den[t][o] = acc, mag
    return y, den


@pytest.mark.parametrize("n,out,in_", [(1, 3, 32), (2, 5, 64), (3, 4, 96)])
def test_w4a8_brute_force(n, out, in_):
    blk = synth.make_blocks(out, in_, seed=out + in_)
    x = synth.make_x(n, in_, seed=n)
    q, d = oracle.quantize_x8(x)
    y, den = oracle.matmul_w4a8(blk, q, d, out, in_)
    yb, denb = _brute_w4a8(blk.reshape(out, in_ // 32, 18), q, d)
    for t in range(n):
        for o in range(out):
            assert abs(Fraction(y[t, o]) - yb[t][o]) <= Fraction(1e-12) * denb[t][o]
            assert abs(Fraction(den[t, o]) - denb[t][o]) <= Fraction(1e-12) * denb[t][o]


def test_w4a8_equals_float_product_on_dequantized_activations():
    """The W4A8 result is the plain product of W with x-hat = q * d."""
    out, in_, n = 300, 1024, 3
    blk = synth.make_blocks(out, in_, seed=3)
    x = synth.make_x(n, in_, seed=4)
    q, d = oracle.quantize_x8(x)
    y, den = oracle.matmul_w4a8(blk, q, d, out, in_)
    xhat = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    w = numpy_dequant(blk.reshape(out, in_ // 32, 18))
    ref = xhat @ w.T
    assert np.all(np.abs(y - ref) <= 1e-12 * den + 1e-300)
    assert np.allclose(den, np.abs(xhat) @ np.abs(w).T, rtol=1e-12, atol=0)


def test_w4a8_zero_codes_and_quantization_error_bound():
    out, in_ = 64, 512
    x = synth.make_x(2, in_, seed=9)
    q, d = oracle.quantize_x8(x)
    z = synth.constant_blocks(out, in_, 0x3C00, 0x88)        # every weight 0
    y0, _ = oracle.matmul_w4a8(z, q, d, out, in_)
    assert not y0.any()
    blk = synth.make_blocks(out, in_, seed=10)
    y8, _ = oracle.matmul_w4a8(blk, q, d, out, in_)
    yf, _ = oracle.matmul(blk, x, out, in_)
    w = numpy_dequant(blk.reshape(out, in_ // 32, 18))
    # each activation moves by at most d/2: |y8 - y| <= sum_k |w_k| d_b(k) / 2
    half = np.repeat(d.astype(np.float64), 32, axis=1) * (0.5 + 1e-5)
    assert np.all(np.abs(y8 - yf) <= half @ np.abs(w).T + 1e-12)
