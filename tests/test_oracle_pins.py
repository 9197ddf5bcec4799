"""The CPU oracle against its pins, and the pins against broken oracles.

CPU only.  Part 1 runs every pin of ``oracle_pins`` against the oracle.
Part 2 compiles copies of ``oracle/vattn_oracle.c`` with one plausible
mistake planted each (dropped max subtraction, wrong sign, missing
normalisation, an extra scale, K used as V, ...) and checks that at least one
pin rejects every copy, i.e. the pins are strong enough to catch it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _oracle_attn(q, k, v):
    return oracle.attention_f64(q, k, v)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_oracle_attn)


def test_rows_variant_matches_full():
    q, k, v = workloads.make_custom(3, 70, 32, "normal", seed=21)
    full = oracle.attention_f64(q, k, v)
    rows = workloads.sample_rows(3, 70, 5)
    part = oracle.attention_rows_f64(q, k, v, rows)
    np.testing.assert_array_equal(part, full.reshape(-1, 32)[rows])


def test_thread_count_does_not_change_result():
    q, k, v = workloads.make_custom(2, 50, 16, "sharp", seed=22)
    a = oracle.attention_f64(q, k, v, n_threads=1)
    b = oracle.attention_f64(q, k, v, n_threads=4)
    np.testing.assert_array_equal(a, b)


def test_empty_shapes():
    for shape in [(0, 5, 4), (3, 0, 4)]:
        z = np.zeros(shape, np.float32)
        assert oracle.attention_f64(z, z, z).shape == shape


def test_bad_row_index_rejected():
    q, k, v = workloads.make_custom(1, 4, 4, "normal", seed=1)
    with pytest.raises(RuntimeError):
        oracle.attention_rows_f64(q, k, v, [4])


# ------------------------------------------------------------------ mutants
# (name, exact text in vattn_oracle.c, replacement).  Each replacement keeps
# every memory access in bounds.
MUTANTS = [
    ("no_max_subtraction", "s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    ("wrong_sign", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("base2_exp", "s[j] = exp(s[j] - m);", "s[j] = exp2(s[j] - m);"),
    ("no_normalisation", "out_row[c] /= l;", "out_row[c] /= 1.0;"),
    ("count_not_sum", "l += s[j];", "l += 1.0;"),
    ("scaled_logits", "acc += q_row[c] * k_head[j * d + c];",
     "acc += 0.125 * q_row[c] * k_head[j * d + c];"),
    ("keys_as_values", "out_row[c] += s[j] * v_head[j * d + c];",
     "out_row[c] += s[j] * k_head[j * d + c];"),
    ("drop_last_key_value", "for (long j = 0; j < n; ++j)\n        for (long c = 0; c < d; ++c)\n            out_row[c] +=",
     "for (long j = 0; j + 1 < n; ++j)\n        for (long c = 0; c < d; ++c)\n            out_row[c] +="),
    ("query_from_keys", "attend_row(q + head_base + i * head_dim,",
     "attend_row(k + head_base + i * head_dim,"),
    ("head_offset_wrong", "const long head_base = h * n_patches * head_dim;",
     "const long head_base = h * n_patches;"),
    ("min_not_max", "if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    ("first_key_only_dim", "acc += q_row[c] * k_head[j * d + c];",
     "acc += q_row[c] * k_head[j * d];"),
]

# Planted mistakes in the rotary transform.
ROPE_MUTANTS = [
    ("rope_sin_sign", "yr[i] = a * cs - b * sn;", "yr[i] = a * cs + b * sn;"),
    ("rope_adjacent_pairs", "const double b = xr[i + half];", "const double b = xr[i + 1];"),
    ("rope_exponent_halved", "-2.0 * (double)i / (double)rope_dims",
     "-1.0 * (double)i / (double)rope_dims"),
    ("rope_factors_multiply", "theta = theta / factors[i];", "theta = theta * factors[i];"),
    ("rope_offset_ignored", "const double pos = (double)(pos_offset + n);",
     "const double pos = (double)n;"),
    ("rope_cos_sin_swapped", "const double cs = cos(theta);", "const double cs = sin(theta);"),
    ("rope_half_from_head_dim", "const long half = rope_dims / 2;",
     "const long half = head_dim / 2;"),
    ("rope_second_half_sign", "yr[i + half] = a * sn + b * cs;",
     "yr[i + half] = b * cs - a * sn;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "vattn_oracle.c")).read()
    assert src.count(old) == 1, "mutation anchor for %s not unique" % name
    csrc = tmp_path / ("m_%s.c" % name)
    csrc.write_text(src.replace(old, new))
    (tmp_path / "vattn_oracle.h").write_text(
        open(os.path.join(ROOT, "oracle", "vattn_oracle.h")).read())
    so = tmp_path / ("m_%s.so" % name)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    str(csrc), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    dp = ctypes.POINTER(ctypes.c_double)
    cl = ctypes.c_long
    lib.vattn_oracle_f64.argtypes = [dp, dp, dp, dp, cl, cl, cl, ctypes.c_int]
    lib.vattn_oracle_f64.restype = ctypes.c_int
    lib.vattn_oracle_rope_f64.argtypes = [dp, dp, cl, cl, cl, cl, ctypes.c_double, dp, cl]
    lib.vattn_oracle_rope_f64.restype = ctypes.c_int

    def f64(x):
        return np.ascontiguousarray(x, np.float64)

    def attn(q, k, v):
        q, k, v = f64(q), f64(k), f64(v)
        out = np.empty(q.shape, np.float64)
        with np.errstate(all="ignore"):
            rc = lib.vattn_oracle_f64(q.ctypes.data_as(dp), k.ctypes.data_as(dp),
                                      v.ctypes.data_as(dp), out.ctypes.data_as(dp),
                                      *q.shape, 1)
        assert rc == 0
        return out

    def rope(x, rope_dims, base, factors, pos_offset):
        x = f64(x)
        y = np.empty_like(x)
        fac = None if factors is None else f64(factors)
        with np.errstate(all="ignore"):
            rc = lib.vattn_oracle_rope_f64(x.ctypes.data_as(dp), y.ctypes.data_as(dp),
                                           *x.shape, rope_dims, base,
                                           None if fac is None else fac.ctypes.data_as(dp),
                                           pos_offset)
        assert rc == 0
        return y
    return attn, rope


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m[0])
def test_pins_reject_planted_mistake(tmp_path, mutant):
    name, old, new = mutant
    attn, _ = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin detects the planted mistake %r" % name


def _oracle_rope(x, rope_dims, base, factors, pos_offset):
    return oracle.rope_neox_f64(x, rope_dims, base, factors, pos_offset)


@pytest.mark.parametrize("pin", oracle_pins.ROPE_PINS, ids=lambda p: p.__name__)
def test_rope_pin(pin):
    pin(_oracle_rope, _oracle_attn)


@pytest.mark.parametrize("mutant", ROPE_MUTANTS, ids=lambda m: m[0])
def test_rope_pins_reject_planted_mistake(tmp_path, mutant):
    name, old, new = mutant
    attn, rope = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in oracle_pins.ROPE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(rope, attn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no rotary pin detects the planted mistake %r" % name


def test_rope_rejects_bad_arguments():
    x = np.zeros((1, 4, 8))
    for kw in ({"rope_dims": 7}, {"rope_dims": 10}, {"rope_dims": -2},
               {"rope_dims": 8, "pos_offset": -1}):
        with pytest.raises(ValueError):
            oracle.rope_neox_f64(x, **kw)
    with pytest.raises(ValueError):
        oracle.rope_neox_f64(x, 8, factors=[1.0, 2.0])


def test_rope_zero_dims_is_identity():
    x = np.random.default_rng(3).standard_normal((2, 5, 6))
    assert np.array_equal(oracle.rope_neox_f64(x, 0), x)


def test_oracle_accepts_f16_and_f64_inputs_exactly():
    q, k, v = workloads.make_custom(2, 20, 8, "normal", seed=9)
    h = [x.astype(np.float16) for x in (q, k, v)]
    a = oracle.attention_f64(*h)
    b = oracle.attention_f64(*[x.astype(np.float64) for x in h])
    np.testing.assert_array_equal(a, b)
