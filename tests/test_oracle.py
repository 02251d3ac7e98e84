"""Pins of the CPU oracle against what the pages and mathematics fix.

Page tag [P1] = "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and
MLX (fp16 Wins)", section "What changed in the computation" unless stated.
None of these checks retypes an oracle formula: they use a library routine
(scipy's Sylvester Hadamard, numpy's IEEE casts), an independent algorithm (a
textbook fast Walsh-Hadamard transform, exact rational arithmetic), closed
forms derived by hand (tests/golden/hand_cases.json) or invariants.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import convrot_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _f32_from_bits(h: str) -> np.float32:
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def _popcount(v):
    return bin(int(v)).count("1")


# --------------------------------------------------------------------------- H

def test_h4_is_sylvester():
    # [P1]: "4x4 Hadamard matrices"; reading: Sylvester's, as scipy builds it.
    assert np.array_equal(O.hadamard4(), scipy.linalg.hadamard(4))


def test_h256_matches_library_sylvester():
    assert np.array_equal(O.hadamard256_pm1(), scipy.linalg.hadamard(256))


def test_h256_closed_form_popcount():
    h = O.hadamard256()
    i = np.arange(256)
    closed = np.array([[(-1.0) ** _popcount(a & b) / 16.0 for b in i] for a in i])
    assert np.array_equal(h, closed)


def test_h_symmetric_orthonormal_exact():
    # [P1]: "H is symmetric with HH = I"; divided by sqrt(256) = 16.
    h = O.hadamard256()
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h, np.eye(256))
    assert set(np.unique(np.abs(h))) == {1.0 / 16.0}


def test_h_kron_h16():
    h16 = scipy.linalg.hadamard(16)
    assert np.array_equal(O.hadamard256_pm1(), np.kron(h16, h16))


# -------------------------------------------------------------------- rotation

def _fwht_textbook(v):
    """In-place iterative Walsh-Hadamard butterflies over the last axis (256)."""
    v = np.array(v, dtype=np.float64, copy=True)
    h = 1
    while h < v.shape[-1]:
        for i in range(0, v.shape[-1], 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v / 16.0


def test_rotation_equals_textbook_fwht_per_group():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3, (5, 1024)).astype(np.float16)
    got = O.rotate_activations_exact(x)
    want = np.concatenate([_fwht_textbook(x[:, g * 256:(g + 1) * 256].astype(np.float64))
                           for g in range(4)], axis=1)
    assert np.array_equal(got, want)          # both exact for fp16 inputs


def test_rotation_one_hot_gives_row_of_h_in_its_group():
    h = O.hadamard256()
    for g, i in ((0, 0), (0, 77), (2, 255), (3, 5)):
        x = np.zeros((1, 1024), np.float16)
        x[0, 256 * g + i] = 1.0
        r = O.rotate_activations_exact(x)[0]
        assert np.array_equal(r[256 * g:256 * (g + 1)], h[i])
        others = np.delete(r, np.s_[256 * g:256 * (g + 1)])
        assert not others.any()


def test_rotation_identity_e2():
    # [P1]: X_rot W_rot^T = (XH)(WH^T)^T = X H H W^T = X W^T.
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1, (16, 512))
    w = rng.normal(0, 0.02, (24, 512))
    lhs = O.rotate_f64(x) @ O.rotate_f64(w).T
    rhs = x @ w.T
    assert np.linalg.norm(lhs - rhs) <= 1e-13 * np.linalg.norm(rhs)
    # A wrong grouping (rotating across 512 with a mismatched layout) breaks it.
    xs = x.copy()
    xs[:, :256], xs[:, 256:] = x[:, 256:], x[:, :256]
    bad = O.rotate_f64(xs) @ O.rotate_f64(w).T
    assert np.linalg.norm(bad - rhs) > 0.1 * np.linalg.norm(rhs)


def test_activation_rotation_is_exact_for_extreme_fp16():
    # fp16 extremes: max, min subnormal, mixed signs; compare with Python ints.
    rng = np.random.default_rng(3)
    vals = np.array([65504, -65504, 2.0 ** -24, -(2.0 ** -24), 6.1e-5, 1.0, -0.333], np.float16)
    x = rng.choice(vals, size=(4, 256)).astype(np.float16)
    x[1] = rng.normal(0, 1000, 256).astype(np.float16)
    got = O.rotate_activations_exact(x)
    hp = scipy.linalg.hadamard(256)
    for r in range(4):
        ints = [int(Fraction(float(v)) * 2 ** 24) for v in x[r]]
        for c in range(256):
            exact = Fraction(sum(int(hp[k, c]) * ints[k] for k in range(256)), 2 ** 24 * 16)
            assert Fraction(float(got[r, c])) == exact


# ----------------------------------------------------------- exact rounding

def _exact_double(d):
    f = Fraction(float(d))
    den = f.denominator
    shift = den.bit_length() - 1
    assert den == 1 << shift
    return f.numerator, shift


def test_round_scaled_int_matches_ieee_casts():
    rng = np.random.default_rng(4)
    samples = list(rng.normal(0, 1, 300) * np.exp2(rng.integers(-160, 140, 300)))
    samples += list(rng.normal(0, 1, 200) * np.exp2(rng.integers(-30, 18, 200)))
    # near fp32/fp16 rounding boundaries and halfway cases
    samples += [1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 1 + 2.0 ** -24 + 2.0 ** -40,
                2.0 ** -150, 3 * 2.0 ** -151, 2.0 ** -149 * 1.5, 2.0 ** -149 * 2.5,
                3.4028235677973366e38, 3.4028235677973366e38 * (1 + 2.0 ** -25),
                float(np.finfo(np.float32).max) * (1 + 2.0 ** -24),
                65504.0, 65519.99, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, 1 + 2.0 ** -11,
                1 + 3 * 2.0 ** -11, 2049.0, 2051.0]
    for d in samples:
        for neg in (1.0, -1.0):
            t, sh = _exact_double(neg * d)
            with np.errstate(over="ignore"):
                want32 = float(np.float32(neg * d))
                want16 = float(np.float16(neg * d))
            assert O.round_scaled_int(t, sh, O.F32) == want32, (neg * d)
            assert O.round_scaled_int(t, sh, O.F16) == want16, (neg * d)


def _is_correct_rounding_f32(exact: Fraction, got: np.float32) -> bool:
    lo = np.nextafter(got, np.float32(-np.inf), dtype=np.float32)
    hi = np.nextafter(got, np.float32(np.inf), dtype=np.float32)
    d = abs(Fraction(float(got)) - exact)
    for nb in (lo, hi):
        dn = abs(Fraction(float(nb)) - exact)
        if dn < d:
            return False
        if dn == d:  # tie: the even significand wins
            if np.array([got], np.float32).view(np.uint32)[0] & 1:
                return False
    return True


# ------------------------------------------------------- weight rotation (R3)

def test_weight_rotation_exact_on_double_rounding_trap():
    # exact sum 1 + 2^-24 + 2^-80 lies just above an fp32 halfway point; a float64
    # sum drops 2^-80, lands on the halfway point and ties to even (downwards).
    w = np.zeros((1, 256), np.float32)
    w[0, 0], w[0, 1], w[0, 2] = 1.0, 2.0 ** -24, 2.0 ** -80
    got = O.rotate_weights_f32(w)[0, 0]
    exact = (Fraction(1) + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 80)) / 16
    assert _is_correct_rounding_f32(exact, got)
    assert got == np.float32((1 + 2.0 ** -23) / 16)
    naive = np.float32((w.astype(np.float64) @ O.hadamard256())[0, 0])
    assert naive != got                          # the plausible mistake fails


def test_weight_rotation_fast_path_equals_exact_path():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, (6, 512)).astype(np.float32)
    w[2, 7] = 1e-30                           # forces the exact path for that group
    w[4, 300] = 3e-12
    fast = O.rotate_weights_f32(w)
    exact = O.rotate_weights_f32(w, force_exact=True)
    assert np.array_equal(fast, exact)


def test_weight_rotation_correctly_rounded_sampled():
    rng = np.random.default_rng(6)
    w = (rng.normal(0, 1, (2, 256)) * np.exp2(rng.integers(-40, 10, (2, 256)))).astype(np.float32)
    got = O.rotate_weights_f32(w)
    hp = scipy.linalg.hadamard(256)
    for r in range(2):
        fr = [Fraction(float(v)) for v in w[r]]
        for c in rng.choice(256, 24, replace=False):
            exact = sum(int(hp[k, c]) * fr[k] for k in range(256)) / 16
            assert _is_correct_rounding_f32(exact, got[r, c])


# ---------------------------------------------------------------- quantisation

def test_tie_rows_round_half_even():
    g = _golden()["tie_rows"]
    rows = []
    for r in g["rows"]:
        x = np.empty(256, np.float64)
        x[0::2] = r["x_even_num"] / r["den"]
        x[1::2] = r["x_odd_num"] / r["den"]
        assert np.array_equal(x.astype(np.float16).astype(np.float64), x)  # fp16-exact
        rows.append(x)
    x16 = np.array(rows).astype(np.float16)
    q, s = O.quantize_activations(x16)
    assert np.all(s == np.float32(g["s_X"]))
    assert list(q[:, 0]) == [r["Q_X_0"] for r in g["rows"]]
    assert list(q[:, 1]) == [r["Q_X_1"] for r in g["rows"]]
    assert not q[:, 2:].any()
    assert list(q[:, 1]) != g["half_away_from_zero_would_give_Q_X_1"]
    assert list(q[:, 1]) != g["truncation_would_give_Q_X_1"]


def test_constant_row():
    g = _golden()["constant_row"]
    x16 = np.full((1, 256), g["c"], np.float16)
    q, s = O.quantize_activations(x16)
    assert s[0] == _f32_from_bits(g["s_X_bits"])
    assert q[0, 0] == 127 and not q[0, 1:].any()


def test_one_hot_end_to_end_identity():
    g = _golden()["one_hot"]
    x16 = np.eye(256, dtype=np.float16)
    w = np.eye(256, dtype=np.float32)
    qw, sw = O.quantize_weights(w)
    y, qx, sx, a = O.linear_w8a8(x16, qw, sw)
    s_bits = _f32_from_bits(g["s_X_bits"])
    assert np.all(sx == s_bits) and np.all(sw == s_bits)
    assert np.array_equal(qx.astype(np.int64), 127 * scipy.linalg.hadamard(256))
    assert np.array_equal(qw, qx)
    assert np.array_equal(a, g["A_diag"] * np.eye(256, dtype=np.int64))
    assert np.array_equal(y, np.eye(256, dtype=np.float16))


def test_quantisation_invariants():
    rng = np.random.default_rng(7)
    x = (rng.standard_t(3, (40, 1024)) * 3).astype(np.float16)
    x[5] = 0
    q, s = O.quantize_activations(x)
    assert q.min() >= -127 and q.max() <= 127            # -128 never occurs
    nz = s > 0
    assert not nz[5] and not q[5].any()                  # zero row: s = 0, Q = 0
    assert np.all(np.abs(q[nz]).max(axis=1) == 127)      # every nonzero row hits 127
    qn, sn = O.quantize_activations(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for p in (-3, 2):                                    # exact power-of-two scaling
        q2, s2 = O.quantize_activations((x.astype(np.float32) * 2.0 ** p).astype(np.float16))
        ok = np.isfinite(x.astype(np.float32) * 2.0 ** p).all()
        assert ok
        assert np.array_equal(q2, q) and np.array_equal(s2, (s * np.float32(2.0 ** p)))


def test_group_support_stays_in_group():
    x = np.zeros((1, 768), np.float16)
    x[0, 256:512] = np.linspace(-4, 4, 256).astype(np.float16)
    r = O.rotate_activations_exact(x)
    assert not r[0, :256].any() and not r[0, 512:].any()


def test_quantisation_close_to_exact_rational_rounding():
    # fp32 division + half-even rounding agrees with the exact-rational rounding
    # except where the exact quotient lies within one fp32 ulp of a half-integer.
    rng = np.random.default_rng(8)
    v = rng.normal(0, 1, (6, 256)).astype(np.float32)
    q, s = O.quantize_rows(v)
    for r in range(6):
        for k in range(0, 256, 7):
            ex = Fraction(float(v[r, k])) / Fraction(float(s[r]))
            fl = math.floor(ex)
            frac = ex - fl
            want = fl if frac < Fraction(1, 2) else fl + 1 if frac > Fraction(1, 2) else (fl if fl % 2 == 0 else fl + 1)
            if q[r, k] != want:
                assert abs(frac - Fraction(1, 2)) < Fraction(128, 2 ** 23)


# ------------------------------------------------------------- integer product

def test_int_gemm_bruteforce_pages_shape():
    # [P1] "Running int8xint8 in a Metal kernel": M=37, N=80, K=256, 0 mismatches.
    g = _golden()["int_parity_shape"]
    rng = np.random.default_rng(9)
    qx = rng.integers(-127, 128, (g["M"], g["K"]), dtype=np.int8)
    qw = rng.integers(-127, 128, (g["N"], g["K"]), dtype=np.int8)
    qx[0] = 127
    qw[0] = -127
    want = np.einsum("mk,nk->mn", qx.astype(np.int64), qw.astype(np.int64))
    got = O.int8_gemm(qx, qw)
    assert int((got != want).sum()) == g["mismatches"]


def test_int_gemm_extreme_k():
    k = O.K_MAX
    qx = np.full((1, k), 127, np.int8)
    qw = np.full((2, k), 127, np.int8)
    qw[1] = -127
    a = O.int8_gemm(qx, qw)
    assert a[0, 0] == 127 * 127 * k and a[0, 1] == -127 * 127 * k
    assert a[0, 0] < 2 ** 31


# ------------------------------------------------------------------- epilogue

def _rt32(fr: Fraction) -> float:
    t, sh = fr.numerator, 0
    d = fr.denominator
    sh = d.bit_length() - 1
    assert d == 1 << sh
    return O.round_scaled_int(t, sh, O.F32)


def _rt16(fr: Fraction) -> float:
    d = fr.denominator
    sh = d.bit_length() - 1
    return O.round_scaled_int(fr.numerator, sh, O.F16)


def test_epilogue_matches_exact_rational_emulation():
    rng = np.random.default_rng(10)
    a = rng.integers(-2 ** 30, 2 ** 30, (4, 5))
    a[0, 0] = 2 ** 24 + 1           # int -> fp32 rounding is exercised
    a[1, 1] = 0
    sx = (rng.random(4) * 1e-2).astype(np.float32)
    sw = (rng.random(5) * 1e-4).astype(np.float32)
    bias = rng.normal(0, 1, 5).astype(np.float32)
    for b in (None, bias):
        y = O.epilogue_w8a8(a, sx, sw, b)
        for m in range(4):
            for n in range(5):
                af = _rt32(Fraction(int(a[m, n])))
                sc = _rt32(Fraction(float(sx[m])) * Fraction(float(sw[n])))
                v = _rt32(Fraction(af) * Fraction(sc))
                if b is not None:
                    v = _rt32(Fraction(v) + Fraction(float(b[n])))
                want = _rt16(Fraction(v))
                assert float(y[m, n]) == want


# ------------------------------------------------- weight-only, fp16, quality

def test_f16_cast_of_exact_double_is_single_rounding():
    # fp16(exact X_rot) must round once; numpy's float64 -> float16 cast is
    # checked against the exact rounding routine on halfway-adjacent values.
    vals = [1 + 2.0 ** -11 + 2.0 ** -40, 1 + 2.0 ** -11 - 2.0 ** -40, 1 + 2.0 ** -11,
            2049.0 + 2.0 ** -30, 0.1, -7.123456789, 65519.0, 2.0 ** -25 + 2.0 ** -50]
    for d in vals:
        t, sh = _exact_double(d)
        assert float(np.float64(d).astype(np.float16)) == O.round_scaled_int(t, sh, O.F16)


def test_w8a16_one_hot():
    x16 = np.eye(256, dtype=np.float16)
    qw, sw = O.quantize_weights(np.eye(256, dtype=np.float32))
    y = O.linear_w8a16(x16, qw, sw)
    assert np.array_equal(y, np.eye(256, dtype=np.float16))


def test_w8a16_lora_rotated_form_identity():
    # [P4] "Design": the rotated down weight meets the rotated activation; since
    # H is symmetric and orthogonal, (XH)(DH)^T U^T = X D^T U^T.
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, (8, 512))
    d = rng.normal(0, 0.01, (4, 512))
    u = rng.normal(0, 0.01, (10, 4))
    a = (O.rotate_f64(x) @ O.rotate_f64(d).T) @ u.T
    b = (x @ d.T) @ u.T
    assert np.linalg.norm(a - b) <= 1e-13 * np.linalg.norm(b)


def test_w8a16_lora_and_bias_are_added():
    rng = np.random.default_rng(12)
    x16 = rng.normal(0, 1, (6, 256)).astype(np.float16)
    w = rng.normal(0, 0.02, (9, 256)).astype(np.float32)
    qw, sw = O.quantize_weights(w)
    d = rng.normal(0, 0.01, (3, 256)).astype(np.float32)
    u = rng.normal(0, 0.01, (9, 3)).astype(np.float32)
    bias = rng.normal(0, 1, 9).astype(np.float32)
    base = O.linear_w8a16(x16, qw, sw).astype(np.float64)
    full = O.linear_w8a16(x16, qw, sw, bias=bias, lora=(d, u, 2.0)).astype(np.float64)
    extra = 2.0 * (x16.astype(np.float64) @ d.T.astype(np.float64)) @ u.T.astype(np.float64) + bias
    assert np.abs(full - base - extra).max() < 4e-3 * (1 + np.abs(full).max())


def test_f16_baseline_integer_inputs_exact():
    rng = np.random.default_rng(13)
    x = rng.integers(-8, 9, (7, 256))
    w = rng.integers(-8, 9, (5, 256))
    y = O.linear_f16(x.astype(np.float16), w.astype(np.float16))
    assert np.array_equal(y.astype(np.int64), x @ w.T)      # |sums| < 2048: exact in fp16


def test_rotation_reduces_quantisation_error_on_outlier_channels():
    # [P1]: the rotation spreads outliers so that int8 rounding loses less.
    rng = np.random.default_rng(14)
    K = 2048
    x = rng.normal(0, 1, (64, K))
    x[:, rng.choice(K, K // 100, replace=False)] *= 50
    x16 = x.astype(np.float16)
    w = rng.normal(0, 0.02, (128, K)).astype(np.float32)
    truth = O.linear_true(x16.astype(np.float64), w)
    qw, sw = O.quantize_weights(w)
    y_rot = O.linear_w8a8(x16, qw, sw)[0].astype(np.float64)
    # same int8 scheme without rotation (reference only, computed here)
    qx_n, sx_n = O.quantize_rows(x16.astype(np.float32))
    qw_n, sw_n = O.quantize_rows(w)
    y_plain = (qx_n.astype(np.float64) @ qw_n.astype(np.float64).T) * np.outer(sx_n, sw_n)
    e_rot = np.linalg.norm(y_rot - truth) / np.linalg.norm(truth)
    e_plain = np.linalg.norm(y_plain - truth) / np.linalg.norm(truth)
    assert e_rot < 0.03
    assert e_plain > 2 * e_rot


def test_scale_spans_the_whole_row_not_one_group():
    # [P1]: s_X[m] = max over all k of the row, not per 256-group (reading R4).
    rng = np.random.default_rng(15)
    x = np.concatenate([rng.normal(0, 1, (3, 256)), 0.01 * rng.normal(0, 1, (3, 256))], axis=1)
    q, s = O.quantize_activations(x.astype(np.float16))
    assert np.all(np.abs(q[:, :256]).max(axis=1) == 127)
    assert np.all(np.abs(q[:, 256:]).max(axis=1) <= 3)


# ------------------------------------- W8A8 with bias, LoRA and residual (R8)

def _small_w8a8(seed, M=6, N=5, K=256):
    rng = np.random.default_rng(seed)
    x16 = rng.normal(0, 1, (M, K)).astype(np.float16)
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    qw, sw = O.quantize_weights(w)
    bias = rng.normal(0, 0.1, N).astype(np.float32)
    return rng, x16, qw, sw, bias


def test_w8a8_ex_plain_is_linear_w8a8():
    _, x16, qw, sw, bias = _small_w8a8(20)
    for b in (None, bias):
        a = O.linear_w8a8_ex(x16, qw, sw, bias=b)
        want = O.linear_w8a8(x16, qw, sw, b)[0]
        assert np.array_equal(a.view(np.uint16), want.view(np.uint16))


def test_epilogue_f32_is_the_value_before_the_cast():
    rng = np.random.default_rng(21)
    a = rng.integers(-2 ** 30, 2 ** 30, (3, 4))
    sx = (rng.random(3) * 1e-2).astype(np.float32)
    sw = (rng.random(4) * 1e-4).astype(np.float32)
    bias = rng.normal(0, 1, 4).astype(np.float32)
    y = O.epilogue_w8a8_f32(a, sx, sw, bias)
    assert y.dtype == np.float32
    for m in range(3):
        for n in range(4):
            af = _rt32(Fraction(int(a[m, n])))
            sc = _rt32(Fraction(float(sx[m])) * Fraction(float(sw[n])))
            v = _rt32(Fraction(af) * Fraction(sc))
            assert float(y[m, n]) == _rt32(Fraction(v) + Fraction(float(bias[n])))


def test_w8a8_ex_residual_is_one_fp16_addition():
    # [P4] "Design": the residual joins the layer output in eager's order, i.e.
    # one fp16 addition of the finished fp16 output and the residual; checked
    # against exact rational arithmetic with the exact rounding routine.
    rng, x16, qw, sw, bias = _small_w8a8(22)
    res = (rng.normal(0, 4, x16.shape[:1] + (qw.shape[0],))).astype(np.float16)
    res[0, 0] = np.float16(65504.0)               # overflow of the sum must give inf or stay finite exactly
    res[1, :] = np.float16(2.0 ** -24)            # smallest subnormal
    y = O.linear_w8a8(x16, qw, sw, bias)[0]
    got = O.linear_w8a8_ex(x16, qw, sw, bias=bias, residual=res)
    for (m, n), v in np.ndenumerate(got):
        want = _rt16(Fraction(float(y[m, n])) + Fraction(float(res[m, n])))
        assert float(v) == want


def test_w8a8_ex_exact_residual_cancellation():
    _, x16, qw, sw, bias = _small_w8a8(23)
    y = O.linear_w8a8(x16, qw, sw, bias)[0]
    got = O.linear_w8a8_ex(x16, qw, sw, bias=bias, residual=-y)
    assert np.all(got == 0) and not np.any(np.signbit(got[y != 0]))


def test_w8a8_ex_lora_closed_form_unit_down_rows():
    # With down rows e_k1, e_k2 the low-rank activation is two columns of X,
    # so the term is scale * (X[m,k1] U[n,0] + X[m,k2] U[n,1]); the result is
    # R5's fp32 value plus that term, rounded once to fp16 (exact rationals).
    rng, x16, qw, sw, bias = _small_w8a8(24, M=4, N=7, K=512)
    k1, k2 = 3, 300
    d = np.zeros((2, 512), np.float32)
    d[0, k1] = 1.0
    d[1, k2] = 1.0
    u = rng.normal(0, 0.5, (7, 2)).astype(np.float32)
    scale = 0.75
    qx, sx = O.quantize_activations(x16)
    y32 = O.epilogue_w8a8_f32(O.int8_gemm(qx, qw), sx, sw, bias)
    got = O.linear_w8a8_ex(x16, qw, sw, bias=bias, lora=(d, u, scale))
    for (m, n), v in np.ndenumerate(got):
        term = Fraction(scale) * (Fraction(float(x16[m, k1])) * Fraction(float(u[n, 0])) +
                                  Fraction(float(x16[m, k2])) * Fraction(float(u[n, 1])))
        assert float(v) == _rt16(Fraction(float(y32[m, n])) + term)
    # and a zero up weight leaves the plain layer
    z = O.linear_w8a8_ex(x16, qw, sw, bias=bias, lora=(d, np.zeros_like(u), scale))
    assert np.array_equal(z, O.linear_w8a8(x16, qw, sw, bias)[0])


# ------------------------------------- dequantise-every-call baseline (R10)

def test_dequantize_matches_exact_rationals():
    # fp16 of the exact un-rotated dequantised weight, element by element with
    # rational arithmetic and the explicit +-1 matrix
    rng = np.random.default_rng(30)
    q = rng.integers(-127, 128, (3, 512)).astype(np.int8)
    s = (rng.random(3) * 1e-3).astype(np.float32)
    s[2] = np.float32(2.0 ** -130)      # subnormal scale: results underflow in fp16
    w = O.dequantize_weights(q, s)
    hpm = O.hadamard256_pm1()
    for n in range(3):
        for k in (0, 1, 255, 256, 300, 511):
            g, c = divmod(k, 256)
            tot = sum(int(q[n, 256 * g + j]) * int(hpm[j, c]) for j in range(256))
            exact = Fraction(tot) * Fraction(float(s[n])) / 16
            assert float(w[n, k]) == _rt16(exact)


def test_dequantize_inverts_quantization_within_its_error():
    # H is orthogonal: per group the L2 distance to W is the rotated-domain
    # quantisation error, at most sqrt(256) * s_W / 2, plus fp16 rounding
    rng = np.random.default_rng(31)
    w = rng.normal(0, 0.02, (8, 768)).astype(np.float32)
    qw, sw = O.quantize_weights(w)
    wd = O.dequantize_weights(qw, sw).astype(np.float64)
    for n in range(8):
        for g in range(3):
            d = wd[n, 256 * g:256 * (g + 1)] - w[n, 256 * g:256 * (g + 1)]
            bound = 16 * float(sw[n]) / 2 + 16 * 2.0 ** -11 * np.abs(w[n]).max()
            assert np.linalg.norm(d) <= bound


def test_dequantize_of_scaled_hadamard_row_is_one_hot():
    # a weight row that is 127 * (row j of the +-1 matrix) with scale 1/127
    # un-rotates to 16 e_j (H = Hpm / 16 and Hpm Hpm = 256 I)
    hpm = O.hadamard256_pm1()
    q = (127 * hpm[[5, 200]]).astype(np.int8)
    s = np.full(2, 1 / 127, np.float32)
    w = O.dequantize_weights(q, s).astype(np.float64)
    exp = np.zeros((2, 256))
    exp[0, 5] = exp[1, 200] = 16 * 127 * float(np.float32(1 / 127))
    assert np.array_equal(w, exp.astype(np.float16).astype(np.float64))


def test_linear_dequant_is_fp16_matmul_of_the_dequantised_weight():
    rng = np.random.default_rng(32)
    x16 = rng.integers(-4, 5, (5, 256)).astype(np.float16)
    q = rng.integers(-127, 128, (6, 256)).astype(np.int8)
    s = np.full(6, 2.0 ** -10, np.float32)
    b = rng.integers(-3, 4, 6).astype(np.float32)
    wd = O.dequantize_weights(q, s)
    y = O.linear_dequant(x16, q, s, b)
    for m in range(5):
        for n in range(6):
            exact = sum(Fraction(float(x16[m, k])) * Fraction(float(wd[n, k])) for k in range(256)) + Fraction(float(b[n]))
            assert float(y[m, n]) == _rt16(exact)


# ---------------------------------------- range-safe weight-only path (R11)

def test_to_bf16_matches_torch_cast():
    import torch
    rng = np.random.default_rng(40)
    v = np.concatenate([rng.normal(0, 1, 2000) * 10.0 ** rng.integers(-40, 38, 2000),
                        [3.39e38, 3.4e38, -3.4e38, 1e-40, 2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134,
                         1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 0.0]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    got = O.to_bf16(v.astype(np.float64))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_rowscaled_near_max_fp16_row_stays_finite():
    # a constant row c rotates to 16 c in the first element of each group:
    # 16 * 65504 = 2^20 (1 - 2^-11) overflows fp16, the scaled value is the
    # largest fp16 below 1 with e = 20
    x = np.full((1, 512), 65504.0, np.float32)
    assert np.isinf(O.rotate_activations_f16(x.astype(np.float16))).any()
    x16, e = O.rotate_rowscaled_f16(x)
    assert e[0] == 20
    assert float(x16[0, 0]) == 1 - 2.0 ** -11 and float(x16[0, 256]) == 1 - 2.0 ** -11
    assert np.count_nonzero(x16) == 2


def test_rowscaled_power_of_two_max_and_zero_row():
    x = np.zeros((2, 256), np.float32)
    x[0, 0] = 16 * 2.0 ** 5            # rotates to 2^5 at every position of the group
    x16, e = O.rotate_rowscaled_f16(x)
    assert e.tolist() == [5, 0]
    assert np.all(x16[0] == 1.0) and np.all(x16[1] == 0)


def test_rowscaled_equals_unscaled_fp16_in_normal_range():
    rng = np.random.default_rng(41)
    x = rng.integers(-8, 9, (6, 768)).astype(np.float16)
    x16, e = O.rotate_rowscaled_f16(x.astype(np.float32))
    ref = O.rotate_activations_f16(x)
    restored = x16.astype(np.float64) * np.exp2(e.astype(np.float64))[:, None]
    assert np.array_equal(restored, ref.astype(np.float64))
    assert np.all(np.abs(x16).max(axis=1) <= 1) and np.all(np.abs(x16).max(axis=1) > 0.5)


def test_rowscaled_bf16_huge_and_integer_path():
    # bf16-sized values far beyond fp16 range; the Python-integer route for a
    # row whose groups span more than 45 binades agrees with exact rationals
    rng = np.random.default_rng(42)
    x = O.to_bf16(rng.normal(0, 1, (3, 256)) * 1e30)
    x[2, :4] = O.to_bf16([1e30, 1e-30, -3e20, 7e-25])     # wide span: integer route
    x16, e = O.rotate_rowscaled_f16(x)
    assert np.isfinite(x16.astype(np.float64)).all()
    for m in range(3):
        vals = O._row_rotation_exact(x[m])
        for k in (0, 1, 100, 255):
            sv = vals[k] / Fraction(2) ** int(e[m])
            assert float(x16[m, k]) == _rt16(sv)
        assert max(abs(v) for v in vals) <= Fraction(2) ** int(e[m]) < 2 * max(abs(v) for v in vals)


def test_linear_w8a16_rs_equals_w8a16_in_range():
    rng = np.random.default_rng(43)
    x = rng.integers(-8, 9, (5, 512)).astype(np.float16)
    w = rng.normal(0, 0.02, (7, 512)).astype(np.float32)
    qw, sw = O.quantize_weights(w)
    b = rng.normal(0, 0.1, 7).astype(np.float32)
    a = O.linear_w8a16_rs(x.astype(np.float32), qw, sw, bias=b, out="f16")
    ref = O.linear_w8a16(x, qw, sw, b)
    assert np.array_equal(a.view(np.uint16), ref.view(np.uint16))


def test_linear_w8a16_rs_near_max_inputs_finite_and_accurate():
    # rows of +-65504 overflow the plain weight-only path's fp16 rotation; the
    # range-safe path stays finite and close to the float64 product
    rng = np.random.default_rng(44)
    x = (np.sign(rng.normal(0, 1, (4, 256))) * 65504).astype(np.float32)
    w = rng.normal(0, 0.02, (6, 256)).astype(np.float32)
    qw, sw = O.quantize_weights(w)
    plain = O.linear_w8a16(x.astype(np.float16), qw, sw).astype(np.float64)
    assert not np.isfinite(plain).all()
    rs = O.linear_w8a16_rs(x, qw, sw, out="bf16").astype(np.float64)
    truth = x.astype(np.float64) @ O.dequantize_weights(qw, sw).astype(np.float64).T
    assert np.isfinite(rs).all()
    assert np.linalg.norm(rs - truth) <= 1e-2 * np.linalg.norm(truth)


# ------------------------------------------------- empty contraction (R12)

def test_empty_contraction_equals_zero_activation_rows():
    # With K = 0 every sum over k is empty, so each path must give exactly
    # what an all-zero activation row gives at any K (where the sums are sums
    # of zeros): pinned against the K = 256 computation through the general
    # formulas, bit for bit, and against the closed form fp16(+0 + bias).
    rng = np.random.default_rng(12)
    M, N, R = 3, 6, 4
    bias = np.array([0.5, -0.0, 1e-9, -3.25, 70000.0, 2.0 ** -20], np.float32)
    res16 = rng.normal(size=(M, N)).astype(np.float16)
    res32 = O.to_bf16(rng.normal(size=(M, N)))
    up = rng.normal(size=(N, R)).astype(np.float32)
    w = rng.normal(size=(N, 256)).astype(np.float32) * 0.02
    qw, sw = O.quantize_weights(w)
    qw0, sw0 = O.quantize_weights(np.zeros((N, 0), np.float32))
    assert qw0.shape == (N, 0) and np.array_equal(sw0, np.zeros(N, np.float32))
    x0 = np.zeros((M, 0), np.float16)
    xz = np.zeros((M, 256), np.float16)
    lora0 = (np.zeros((R, 0), np.float32), up, 0.5)
    loraz = (rng.normal(size=(R, 256)).astype(np.float32), up, 0.5)

    def same(a, b):
        a, b = np.asarray(a), np.asarray(b)
        assert a.dtype == b.dtype and a.shape == b.shape
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))

    same(O.linear_w8a8(x0, qw0, sw0, bias)[0], O.linear_w8a8(xz, qw, sw, bias)[0])
    same(O.linear_w8a8_ex(x0, qw0, sw0, bias, lora0, res16), O.linear_w8a8_ex(xz, qw, sw, bias, loraz, res16))
    same(O.linear_w8a16(x0, qw0, sw0, bias, lora0), O.linear_w8a16(xz, qw, sw, bias, loraz))
    same(O.linear_dequant(x0, qw0, sw0, bias), O.linear_dequant(xz, qw, sw, bias))
    for out, res in (("f16", res16), ("bf16", res32)):
        same(O.linear_w8a16_rs(x0, qw0, sw0, bias, res, out=out), O.linear_w8a16_rs(xz, qw, sw, bias, res, out=out))
    closed = np.broadcast_to((np.float32(0) + bias).astype(np.float16), (M, N))
    same(O.linear_w8a8(x0, qw0, sw0, bias)[0], np.ascontiguousarray(closed))
    assert not np.signbit(O.linear_w8a8(x0, qw0, sw0, bias)[0][:, 1]).any()   # -0 bias gives +0
    same(O.linear_f16(x0, np.zeros((N, 0), np.float16)), np.zeros((M, N), np.float16))
    q0, s0 = O.quantize_activations(x0)
    assert q0.shape == (M, 0) and np.array_equal(s0, np.zeros(M, np.float32))
    x16, e = O.rotate_rowscaled_f16(x0)
    assert x16.shape == (M, 0) and np.array_equal(e, np.zeros(M, np.int64))
    assert O.int8_gemm(np.zeros((M, 0), np.int8), qw0).shape == (M, N)
    with pytest.raises(ValueError):
        O.quantize_weights(np.zeros((N, 128), np.float32))
