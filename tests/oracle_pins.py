"""Pins for the CPU oracle: checks against facts fixed by the mathematics.

Each ``pin_*`` takes ``attn(q, k, v) -> float64 [H][N][d]`` and raises
``AssertionError`` when the implementation disagrees with a fact that does not
depend on the implementation: closed forms, textbook special cases, exact
brute force at 40 decimal digits, invariants and equivariances of
``out[h] = softmax(Q[h] K[h]^T) V[h]`` (row-wise softmax over every patch, no
scale inside; docs.rs page "rullama 0.1.0",
src/kernels/wgsl/vision_attention_flash_sub_hpd_f16.wgsl).

The same pins are run against the real oracle (they must all pass) and
against deliberately broken copies of it (some pin must fail), see
``test_oracle_pins.py``.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
from scipy.special import expit, softmax

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise AssertionError("%s: shape %s vs %s" % (what, a.shape, b.shape))
    if not np.all(np.isfinite(a)):
        raise AssertionError("%s: non-finite values" % what)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    if not err <= tol:
        raise AssertionError("%s: max |diff| %.3e > %.1e" % (what, err, tol))


# ---------------------------------------------------------------- closed forms

def pin_single_patch(attn):
    """N = 1: the only weight is exp(0)/exp(0) = 1, so out = V[:, 0] exactly."""
    r = _rng(1)
    q = _f32(r.standard_normal((3, 1, 5)) * 4)
    k = _f32(r.standard_normal((3, 1, 5)) * 4)
    v = _f32(r.standard_normal((3, 1, 5)))
    out = attn(q, k, v)
    if not np.array_equal(out, v.astype(np.float64)):
        raise AssertionError("N=1: out != V exactly")


def pin_zero_query_mean(attn):
    """Q = 0: all logits are 0, the softmax is uniform, out = mean of V rows."""
    r = _rng(2)
    h, n, d = 2, 37, 6
    q = np.zeros((h, n, d), np.float32)
    k = _f32(r.standard_normal((h, n, d)) * 5)
    v = _f32(r.standard_normal((h, n, d)))
    out = attn(q, k, v)
    for hh in range(h):
        mean = np.array([math.fsum(v[hh, :, c].astype(np.float64)) / n
                         for c in range(d)])
        _close(out[hh], np.broadcast_to(mean, (n, d)), 1e-13, "Q=0 mean")


def pin_constant_values(attn):
    """Every V row equal to c: any convex combination gives c."""
    r = _rng(3)
    h, n, d = 2, 29, 4
    q = _f32(r.standard_normal((h, n, d)) * 3)
    k = _f32(r.standard_normal((h, n, d)) * 3)
    c = _f32(r.standard_normal((h, 1, d)))
    v = _f32(np.broadcast_to(c, (h, n, d)))
    out = attn(q, k, v)
    _close(out, np.broadcast_to(c.astype(np.float64), (h, n, d)), 1e-14,
           "constant V")


def pin_one_hot_values_give_softmax(attn):
    """V = identity (N = d): out[h, i, :] is row i of softmax(Q K^T), a
    textbook routine (scipy.special.softmax over the key axis); rows are
    non-negative and sum to 1."""
    r = _rng(4)
    h, n = 3, 16
    q = _f32(r.standard_normal((h, n, n)))
    k = _f32(r.standard_normal((h, n, n)))
    v = _f32(np.broadcast_to(np.eye(n, dtype=np.float32), (h, n, n)))
    out = attn(q, k, v)
    logits = np.matmul(q.astype(np.float64), k.astype(np.float64).transpose(0, 2, 1))
    _close(out, softmax(logits, axis=-1), 1e-14, "one-hot V vs softmax")
    if np.any(out < 0):
        raise AssertionError("negative attention weight")
    _close(out.sum(axis=-1), np.ones((h, n)), 1e-14, "rows sum to 1")


def pin_two_patches_logistic(attn):
    """N = 2: weight of patch 0 is the logistic function of s0 - s1."""
    r = _rng(5)
    h, d = 4, 8
    q = _f32(r.standard_normal((h, 2, d)) * 2)
    k = _f32(r.standard_normal((h, 2, d)) * 2)
    v = _f32(r.standard_normal((h, 2, d)))
    out = attn(q, k, v)
    for hh in range(h):
        for i in range(2):
            s = [math.fsum(float(a) * float(b) for a, b in zip(q[hh, i], k[hh, j]))
                 for j in range(2)]
            w0 = expit(s[0] - s[1])
            w1 = expit(s[1] - s[0])
            exp_row = w0 * v[hh, 0].astype(np.float64) + w1 * v[hh, 1].astype(np.float64)
            _close(out[hh, i], exp_row, 1e-14, "N=2 logistic")


def pin_dominant_logit(attn):
    """q = a*e0, key j* = e0, other keys orthogonal to e0 (first component 0):
    logits are a for j* and 0 elsewhere, so out = V[j*] up to
    (N-1) e^-a * 2 max|v|."""
    r = _rng(6)
    n, d, a, jstar = 50, 8, 40.0, 17
    q = np.zeros((1, n, d), np.float32)
    q[0, :, 0] = a
    k = _f32(r.standard_normal((1, n, d)))
    k[0, :, 0] = 0.0
    k[0, jstar] = 0.0
    k[0, jstar, 0] = 1.0
    v = _f32(r.standard_normal((1, n, d)))
    out = attn(q, k, v)
    bound = (n - 1) * math.exp(-a) * 2 * float(np.max(np.abs(v)))
    _close(out[0], np.broadcast_to(v[0, jstar].astype(np.float64), (n, d)),
           max(bound, 1e-15), "dominant logit")


def pin_large_logits_stay_finite(attn):
    """Logits of magnitude ~1e4 (exp would overflow without subtracting the
    row maximum): result is finite and equals the exact result below."""
    r = _rng(7)
    q = _f32(r.standard_normal((2, 6, 4)) * 60)
    k = _f32(r.standard_normal((2, 6, 4)) * 60)
    v = _f32(r.standard_normal((2, 6, 4)))
    out = attn(q, k, v)
    _close(out, _decimal_attention(q, k, v), 1e-13, "large logits")


def pin_softmax_golden(attn):
    """Stored worked examples with hand-derived exact values (tests/golden)."""
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q = _f32(case["q"])
        k = _f32(case["k"])
        v = _f32(case["v"])
        out = attn(q, k, v)
        _close(out, np.asarray(case["out"], np.float64), case["tol"],
               "golden " + case["name"])


# ------------------------------------------------------------- brute force

def _decimal_attention(q, k, v, digits=40):
    """Exact-input evaluation at ``digits`` significant decimal digits."""
    getcontext().prec = digits
    h, n, d = q.shape
    out = np.zeros((h, n, d))
    for hh in range(h):
        for i in range(n):
            s = []
            for j in range(n):
                acc = Decimal(0)
                for c in range(d):
                    acc += Decimal(float(q[hh, i, c])) * Decimal(float(k[hh, j, c]))
                s.append(acc)
            m = max(s)
            e = [(x - m).exp() for x in s]
            l = sum(e, Decimal(0))
            for c in range(d):
                num = sum((e[j] * Decimal(float(v[hh, j, c])) for j in range(n)),
                          Decimal(0))
                out[hh, i, c] = float(num / l)
    return out


def pin_brute_force_small(attn):
    """N <= 8: agreement with a 40-digit Decimal evaluation from the same
    float32 inputs, for several shapes and value scales."""
    r = _rng(8)
    for (h, n, d, scale) in [(1, 1, 3, 1.0), (2, 3, 5, 1.0), (3, 5, 4, 2.0),
                             (2, 8, 8, 0.5), (1, 7, 16, 3.0), (2, 8, 2, 10.0)]:
        q = _f32(r.standard_normal((h, n, d)) * scale)
        k = _f32(r.standard_normal((h, n, d)) * scale)
        v = _f32(r.uniform(-2, 2, (h, n, d)))
        _close(attn(q, k, v), _decimal_attention(q, k, v), 1e-13,
               "brute force (%d,%d,%d)" % (h, n, d))


# ------------------------------------------------- invariants / equivariances

def pin_key_permutation_invariance(attn):
    """Permuting keys and values jointly leaves every output row unchanged."""
    r = _rng(9)
    h, n, d = 2, 23, 6
    q = _f32(r.standard_normal((h, n, d)))
    k = _f32(r.standard_normal((h, n, d)))
    v = _f32(r.standard_normal((h, n, d)))
    perm = r.permutation(n)
    _close(attn(q, k[:, perm], v[:, perm]), attn(q, k, v), 1e-13,
           "key permutation")


def pin_query_permutation_equivariance(attn):
    """Permuting query rows permutes output rows the same way."""
    r = _rng(10)
    h, n, d = 2, 19, 5
    q = _f32(r.standard_normal((h, n, d)))
    k = _f32(r.standard_normal((h, n, d)))
    v = _f32(r.standard_normal((h, n, d)))
    perm = r.permutation(n)
    _close(attn(q[:, perm], k, v), attn(q, k, v)[:, perm], 0.0,
           "query permutation")


def pin_heads_independent(attn):
    """One call over H heads equals H one-head calls (head-major offsets)."""
    r = _rng(11)
    h, n, d = 4, 13, 7
    q = _f32(r.standard_normal((h, n, d)))
    k = _f32(r.standard_normal((h, n, d)))
    v = _f32(r.standard_normal((h, n, d)))
    full = attn(q, k, v)
    for hh in range(h):
        _close(full[hh:hh + 1], attn(q[hh:hh + 1], k[hh:hh + 1], v[hh:hh + 1]),
               0.0, "head %d" % hh)


def pin_affine_values(attn):
    """V -> a V + b maps out -> a out + b (weights sum to one).  a and b are
    powers of two / small integers so the float32 inputs stay exact."""
    r = _rng(12)
    h, n, d = 2, 21, 4
    q = _f32(r.standard_normal((h, n, d)))
    k = _f32(r.standard_normal((h, n, d)))
    v = _f32(np.round(r.standard_normal((h, n, d)) * 64) / 64)
    a, b = 4.0, _f32([1.0, -2.0, 0.5, 3.0])
    out = attn(q, k, v)
    out2 = attn(q, k, _f32(a * v + b))
    _close(out2, a * out + b.astype(np.float64), 1e-12, "affine V")


def pin_key_shift_invariance(attn):
    """Adding one vector w to every key adds q.w to a whole row of logits,
    which the softmax ignores.  Inputs are small dyadic rationals so k + w is
    exact in float32."""
    r = _rng(13)
    h, n, d = 2, 17, 4
    q = _f32(np.round(r.standard_normal((h, n, d)) * 8) / 8)
    k = _f32(np.round(r.standard_normal((h, n, d)) * 8) / 8)
    v = _f32(r.standard_normal((h, n, d)))
    w = _f32(np.round(r.standard_normal((h, 1, d)) * 8) / 8)
    _close(attn(q, k + w, v), attn(q, k, v), 1e-13, "key shift")


def pin_output_in_value_hull(attn):
    """Each output coordinate lies between the min and max of that value
    coordinate (convex combination)."""
    r = _rng(14)
    h, n, d = 2, 40, 5
    q = _f32(r.standard_normal((h, n, d)) * 3)
    k = _f32(r.standard_normal((h, n, d)) * 3)
    v = _f32(r.standard_normal((h, n, d)))
    out = attn(q, k, v)
    lo = v.min(axis=1, keepdims=True).astype(np.float64) - 1e-12
    hi = v.max(axis=1, keepdims=True).astype(np.float64) + 1e-12
    if np.any(out < lo) or np.any(out > hi):
        raise AssertionError("output outside the hull of value rows")


ALL_PINS = [
    pin_single_patch,
    pin_zero_query_mean,
    pin_constant_values,
    pin_one_hot_values_give_softmax,
    pin_two_patches_logistic,
    pin_dominant_logit,
    pin_large_logits_stay_finite,
    pin_softmax_golden,
    pin_brute_force_small,
    pin_key_permutation_invariance,
    pin_query_permutation_equivariance,
    pin_heads_independent,
    pin_affine_values,
    pin_key_shift_invariance,
    pin_output_in_value_hull,
]


# ------------------------------------------------------------ rotary transform
# Pins of the NeoX rotary transform (docs.rs page "rullama 0.2.0",
# src/kernels/wgsl/rope_neox_backward.wgsl: forward rotation in its header
# comment, angle pos * base^(-2i/rope_dims) [/ factors[i]] in its main
# function).  Each ``rope_pin_*`` takes ``rope(x, rope_dims, base, factors,
# pos_offset) -> float64 [H][N][d]`` (patch n at position pos_offset + n) and
# ``attn`` as above.

def _decimal_angles(n_patches, pos_offset):
    """base 10000 and rope_dims 8 make the frequencies exact powers of ten:
    10000^(-2i/8) = 10^-i, so theta[n, i] = (pos_offset + n) * 10^-i."""
    pos = np.arange(n_patches, dtype=np.float64) + pos_offset
    return pos[:, None] * np.array([1.0, 0.1, 0.01, 0.001])[None, :]


def rope_pin_position_zero_is_identity(rope, attn):
    """Every angle is 0 at position 0: the first patch is unchanged."""
    x = _rng(40).standard_normal((2, 3, 12))
    y = rope(x, 12, 10000.0, None, 0)
    if not np.array_equal(y[:, 0], x[:, 0]):
        raise AssertionError("position 0 changed the row")


def rope_pin_decimal_frequencies(rope, attn):
    """Pairs (i, i+4) of rope_dims 8 with base 10000 turn by (pos)*10^-i,
    written as a complex product (x_i + j x_{i+4}) e^{j theta}; the two
    dimensions past rope_dims pass through."""
    x = _rng(41).standard_normal((2, 9, 10))
    y = rope(x, 8, 10000.0, None, 5)
    theta = _decimal_angles(9, 5)
    z = (x[:, :, 0:4] + 1j * x[:, :, 4:8]) * np.exp(1j * theta)[None]
    _close(y[:, :, 0:4], z.real, 1e-13, "rotated first halves")
    _close(y[:, :, 4:8], z.imag, 1e-13, "rotated second halves")
    if not np.array_equal(y[:, :, 8:], x[:, :, 8:]):
        raise AssertionError("dimensions past rope_dims changed")


def rope_pin_unit_vector_traces_the_angle(rope, attn):
    """x = e_0 at position p turns into (cos p, sin p) in dims (0, half):
    the lowest frequency is base^0 = 1 for every base."""
    x = np.zeros((1, 7, 6))
    x[:, :, 0] = 1.0
    y = rope(x, 6, 37.5, None, 0)
    for p in range(7):
        _close(y[0, p], [math.cos(p), 0, 0, math.sin(p), 0, 0], 1e-15, "e_0 at %d" % p)


def rope_pin_page_backward_inverts(rope, attn):
    """The page's backward step (rotation by -theta: dx_i c + dx_{i+h} s,
    -dx_i s + dx_{i+h} c) undoes the forward rotation exactly."""
    x = _rng(42).standard_normal((3, 6, 8))
    y = rope(x, 8, 10000.0, None, 11)
    theta = _decimal_angles(6, 11)[None]
    c, s = np.cos(theta), np.sin(theta)
    a, b = y[:, :, 0:4], y[:, :, 4:8]
    back = np.concatenate([a * c + b * s, -a * s + b * c], axis=2)
    _close(back, x, 1e-13, "backward(forward(x))")


def rope_pin_factors_divide_angles(rope, attn):
    """factors 10^-i cancel the decimal frequencies: every pair turns by pos."""
    x = _rng(43).standard_normal((2, 5, 8))
    y = rope(x, 8, 10000.0, np.array([1.0, 0.1, 0.01, 0.001]), 3)
    pos = (np.arange(5) + 3.0)[None, :, None]
    z = (x[:, :, 0:4] + 1j * x[:, :, 4:8]) * np.exp(1j * pos)
    _close(y[:, :, 0:4], z.real, 1e-13, "first halves")
    _close(y[:, :, 4:8], z.imag, 1e-13, "second halves")


def rope_pin_pair_norms_and_passthrough(rope, attn):
    """A rotation keeps |(x_i, x_{i+h})| for every pair and leaves the rest."""
    x = _rng(44).standard_normal((2, 40, 24))
    y = rope(x, 16, 523.0, np.linspace(0.5, 4.0, 8), 2)
    nx = x[:, :, 0:8] ** 2 + x[:, :, 8:16] ** 2
    ny = y[:, :, 0:8] ** 2 + y[:, :, 8:16] ** 2
    _close(ny, nx, 1e-12, "pair norms")
    if not np.array_equal(y[:, :, 16:], x[:, :, 16:]):
        raise AssertionError("dimensions past rope_dims changed")
    if np.allclose(y[:, 1:, 0:16], x[:, 1:, 0:16]):
        raise AssertionError("nothing was rotated")


def rope_pin_relative_positions(rope, attn):
    """Rotating queries and keys by their positions makes every logit depend
    on the position difference only: shifting all positions leaves the
    attention output unchanged."""
    r = _rng(45)
    q = r.standard_normal((2, 30, 16)) * 0.8
    k = r.standard_normal((2, 30, 16)) * 0.8
    v = r.standard_normal((2, 30, 16))
    a = attn(rope(q, 16, 100.0, None, 0), rope(k, 16, 100.0, None, 0), v)
    b = attn(rope(q, 16, 100.0, None, 97), rope(k, 16, 100.0, None, 97), v)
    _close(a, b, 1e-11, "shifted positions")
    c = attn(q, k, v)
    if np.allclose(a, c, atol=1e-3):
        raise AssertionError("rotation had no effect on attention")


def rope_pin_attention_closed_form(rope, attn):
    """head_dim 2, rope_dims 2: q = k = (a, 0) at every position p rotate to
    a (cos p, sin p), so the logit of query p and key p' is a^2 cos(p - p')
    and the output is the softmax of those logits applied to V."""
    n, a = 12, 1.7
    x = np.zeros((1, n, 2))
    x[0, :, 0] = a
    v = _rng(46).standard_normal((1, n, 2))
    out = attn(rope(x, 2, 10000.0, None, 0), rope(x, 2, 10000.0, None, 0), v)
    p = np.arange(n, dtype=np.float64)
    logits = a * a * np.cos(p[:, None] - p[None, :])
    _close(out[0], softmax(logits, axis=1) @ v[0], 1e-13, "closed-form logits")


ROPE_PINS = [
    rope_pin_position_zero_is_identity,
    rope_pin_decimal_frequencies,
    rope_pin_unit_vector_traces_the_angle,
    rope_pin_page_backward_inverts,
    rope_pin_factors_divide_angles,
    rope_pin_pair_norms_and_passthrough,
    rope_pin_relative_positions,
    rope_pin_attention_closed_form,
]
