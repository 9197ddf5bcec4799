"""GPU parity of the fused rotary (NeoX) path against the float64 oracle.

The oracle rotates Q and K in float64 (``oracle.rope_neox_f64``: patch n at
position pos_offset + n, pairs (i, i + rope_dims/2), angle
pos * base^(-2i/rope_dims) / factors[i]) and then evaluates the attention;
the GPU builds its (cos, sin) table with ``vattn_rope_table`` and rotates Q
and K inside the attention kernel.  Tolerance as for every other path:
max-abs <= 2e-3 and relative L2 <= 1e-3 over the compared elements.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads

from tests import full_size

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_L2 = 1e-3


@pytest.fixture(scope="module")
def vattn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import non_causal_flash_amd as m
    return m


def _assert_close(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(gpu)), "%s: non-finite output" % what
    diff = gpu - ref
    max_abs = float(np.max(np.abs(diff)))
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    print("%s: max_abs %.3e rel_l2 %.3e" % (what, max_abs, rel), flush=True)
    assert max_abs <= MAX_ABS and rel <= REL_L2, "%s: max_abs %.3e rel_l2 %.3e" % (what, max_abs, rel)


def _ref(q, k, v, rope_dims, base=10000.0, factors=None, pos_offset=0, rows=None):
    qr = oracle.rope_neox_f64(q, rope_dims, base, factors, pos_offset)
    kr = oracle.rope_neox_f64(k, rope_dims, base, factors, pos_offset)
    if rows is None:
        return oracle.attention_f64(qr, kr, v)
    return oracle.attention_rows_f64(qr, kr, v, rows)


def _device(x, layout="head", dtype=None):
    t = torch.from_numpy(workloads.to_layout(x, layout)).cuda()
    if dtype is not None:
        t = t.to(dtype)
    return t.transpose(0, 1) if layout == "patch" else t


def _run(vattn, q, k, v, table, precision, layout="head"):
    dq, dk, dv = (_device(x, layout) for x in (q, k, v))
    out = vattn.forward(dq, dk, dv, precision=precision, rope=table)
    torch.cuda.synchronize()
    return out.contiguous().float().cpu().numpy()


# ------------------------------------------------------------------ table

@pytest.mark.parametrize("rope_dims,base,factors,pos_offset", [
    (64, 10000.0, None, 0),
    (8, 10000.0, None, 5000),
    (32, 500000.0, np.linspace(1.0, 8.0, 16), 3),
    (2, 10.0, None, 123456),
])
def test_table_matches_float64_angles(vattn, rope_dims, base, factors, pos_offset):
    """Table entry (n, i) is (cos, sin) of (pos_offset + n) * base^(-2i/d) /
    factors[i], evaluated in float64 and rounded to float32: within one f32
    rounding of the float64 value."""
    n = 1000
    table = vattn.rope_table(n, rope_dims, base, factors, pos_offset)
    torch.cuda.synchronize()
    got = table.cpu().numpy().astype(np.float64)
    half = rope_dims // 2
    i = np.arange(half, dtype=np.float64)
    w = np.power(float(np.float32(base)), -2.0 * i / rope_dims)
    if factors is not None:
        w = w / np.asarray(factors, np.float32).astype(np.float64)
    theta = (np.arange(n, dtype=np.float64) + pos_offset)[:, None] * w[None, :]
    assert got.shape == (n, half, 2)
    assert np.max(np.abs(got[:, :, 0] - np.cos(theta))) <= 6.0e-8
    assert np.max(np.abs(got[:, :, 1] - np.sin(theta))) <= 6.0e-8


# ------------------------------------------------------------- workloads

@pytest.mark.parametrize("precision", ["fast", "auto", "split"])
def test_rope_workload_10_full(vattn, precision):
    w = workloads.WORKLOADS[10]
    q, k, v = workloads.make_inputs(10)
    table = vattn.rope_table(w.n_patches, w.rope_dims, w.rope_base)
    _assert_close(_run(vattn, q, k, v, table, precision), _ref(q, k, v, w.rope_dims),
                  "workload 10 %s" % precision)


@pytest.mark.parametrize("precision", ["auto", "split"])
def test_rope_sharp_workload_11_full_tensor(vattn, precision):
    """Workload 11 (sharp 128 x 4096 x 64, rotated) as the benchmark launches
    it; every output element against the oracle."""
    w = workloads.WORKLOADS[11]
    q, k, v = workloads.make_inputs(11)
    table = vattn.rope_table(w.n_patches, w.rope_dims, w.rope_base)
    _assert_close(_run(vattn, q, k, v, table, precision), full_size.reference(11),
                  "workload 11 %s" % precision)


# ---------------------------------------------------------------- shapes

SHAPES = [  # (head_dim, rope_dims)
    (64, 64), (64, 32), (64, 16), (64, 8), (32, 32), (32, 8), (40, 40), (40, 24),
    (48, 16), (17, 8), (8, 8),
]


@pytest.mark.parametrize("d,rope_dims", SHAPES)
@pytest.mark.parametrize("n", [1, 63, 300])
def test_rope_shapes_head_major(vattn, d, rope_dims, n):
    q, k, v = workloads.make_custom(3, n, d, "normal", seed=31 * d + n + rope_dims)
    table = vattn.rope_table(n, rope_dims, 100.0)
    for precision in ("fast", "auto"):
        print("d %d rope %d N %d %s" % (d, rope_dims, n, precision), flush=True)
        _assert_close(_run(vattn, q, k, v, table, precision), _ref(q, k, v, rope_dims, 100.0),
                      "d=%d rope=%d N=%d %s" % (d, rope_dims, n, precision))


@pytest.mark.parametrize("d,rope_dims", [(64, 64), (64, 32), (40, 24), (33, 16)])
@pytest.mark.parametrize("n", [100, 1000])
def test_rope_patch_major(vattn, d, rope_dims, n):
    q, k, v = workloads.make_custom(4, n, d, "normal", seed=17 * d + n)
    table = vattn.rope_table(n, rope_dims)
    for precision in ("fast", "split"):
        print("patch-major d %d rope %d N %d %s" % (d, rope_dims, n, precision), flush=True)
        _assert_close(_run(vattn, q, k, v, table, precision, "patch"), _ref(q, k, v, rope_dims),
                      "patch-major d=%d rope=%d N=%d %s" % (d, rope_dims, n, precision))


def test_rope_wide_grid_with_ragged_tail(vattn):
    """130 heads x 300 patches: the 16-wave rotary kernel (>= 128 wide
    blocks) with a partial last key tile and a partial last query block."""
    q, k, v = workloads.make_custom(130, 300, 64, "normal", seed=77)
    table = vattn.rope_table(300, 64)
    for precision in ("fast", "auto"):
        _assert_close(_run(vattn, q, k, v, table, precision), _ref(q, k, v, 64),
                      "130x300 %s" % precision)


def test_rope_sharp_small(vattn):
    """Sharp logits with rotation: the split correction must see the rotated K."""
    q, k, v = workloads.make_custom(4, 700, 64, "sharp", seed=91)
    table = vattn.rope_table(700, 64)
    for precision in ("auto", "split"):
        _assert_close(_run(vattn, q, k, v, table, precision), _ref(q, k, v, 64),
                      "sharp 4x700 %s" % precision)


def test_rope_factors_and_offset(vattn):
    q, k, v = workloads.make_custom(2, 500, 64, "normal", seed=55)
    factors = np.linspace(1.0, 40.0, 16)
    table = vattn.rope_table(500, 32, 10000.0, factors, 250)
    _assert_close(_run(vattn, q, k, v, table, "auto"),
                  _ref(q, k, v, 32, 10000.0, np.asarray(factors, np.float32), 250),
                  "factors + offset")


def test_rope_longer_table_and_inputs_unchanged(vattn):
    """A table with more rows than patches is fine (rows past n_patches are
    not used); q and k are read only."""
    q, k, v = workloads.make_custom(3, 200, 64, "normal", seed=56)
    table = vattn.rope_table(4096, 64)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = vattn.forward(dq, dk, dv, rope=table)
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy(), q) and np.array_equal(dk.cpu().numpy(), k)
    _assert_close(out.cpu().numpy(), _ref(q, k, v, 64), "long table")


@pytest.mark.parametrize("d,rope_dims,n", [(64, 64, 1024), (64, 32, 300), (40, 24, 500)])
def test_rope_f16(vattn, d, rope_dims, n):
    """f16 tensors: the oracle reads the same f16 values; the output is f16."""
    q, k, v = (x.astype(np.float16) for x in workloads.make_custom(3, n, d, "normal", seed=d + n))
    table = vattn.rope_table(n, rope_dims)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    for precision in ("fast", "auto", "split"):
        out = vattn.forward(dq, dk, dv, precision=precision, rope=table)
        torch.cuda.synchronize()
        assert out.dtype == torch.float16
        _assert_close(out.float().cpu().numpy(), _ref(q, k, v, rope_dims),
                      "f16 d=%d rope=%d N=%d %s" % (d, rope_dims, n, precision))


def test_rope_f16_sharp(vattn):
    q, k, v = (x.astype(np.float16) for x in workloads.make_custom(4, 600, 64, "sharp", seed=92))
    table = vattn.rope_table(600, 64)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    for precision in ("auto", "split"):
        out = vattn.forward(dq, dk, dv, precision=precision, rope=table)
        torch.cuda.synchronize()
        _assert_close(out.float().cpu().numpy(), _ref(q, k, v, 64), "f16 sharp %s" % precision)


def test_rope_c_abi_direct(vattn):
    """vattn_rope_table and vattn_forward_rope with raw pointers, patch-major
    with a padded patch stride; the padding of out stays untouched."""
    h, n, d, rd = 3, 200, 32, 16
    q, k, v = workloads.make_custom(h, n, d, "normal", seed=23)
    sn = h * d + 8
    bufs = []
    for x in (q, k, v):
        b = torch.zeros(n, sn, device="cuda")
        b[:, :h * d] = torch.from_numpy(workloads.to_layout(x, "patch").reshape(n, h * d)).cuda()
        bufs.append(b)
    ob = torch.full((n, sn), float("nan"), device="cuda")
    table = torch.empty(n * rd // 2 * 2, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert vattn.rope_table_raw(table.data_ptr(), n, rd, 10000.0, None, 0, s) == 0
    rc = vattn.forward_rope_raw(bufs[0].data_ptr(), bufs[1].data_ptr(), bufs[2].data_ptr(),
                                ob.data_ptr(), h, n, d, d, sn, rd, table.data_ptr(), s, "auto")
    assert rc == 0
    torch.cuda.synchronize()
    host = ob.cpu().numpy()
    assert np.all(np.isnan(host[:, h * d:]))
    got = host[:, :h * d].reshape(n, h, d).transpose(1, 0, 2)
    _assert_close(got, _ref(q, k, v, rd), "rope c-abi")


def test_rope_deterministic(vattn):
    q, k, v = workloads.make_custom(16, 1000, 64, "sharp", seed=3)
    table = vattn.rope_table(1000, 64)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    a = vattn.forward(dq, dk, dv, rope=table)
    b = vattn.forward(dq, dk, dv, rope=table)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
