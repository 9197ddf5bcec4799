"""GPU parity at large sizes: long heads, many heads, wide patch strides.

The C ABI bounds each head's addressed span ((n_patches + 63) * stride_patch
+ head_dim < 2^28 elements) and the grid (n_heads * blocks < 2^31); these
cases sit well inside the bounds but far beyond the workloads, so 32-bit
offset arithmetic, the XCD block remap over large grids and wide strides
are exercised.  The oracle computes sampled rows (float64); tolerance as
everywhere: max-abs <= 2e-3 and relative L2 <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vattn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import non_causal_flash_amd as m
    return m


def _rows(h, n, count, seed):
    rng = np.random.default_rng(seed)
    rows = {0, h * n - 1, n - 1, (h - 1) * n}
    rows.update(int(x) for x in rng.integers(0, h * n, size=count))
    return np.array(sorted(rows), dtype=np.int64)


def _check(got_rows, ref, what):
    got_rows = np.asarray(got_rows, np.float64)
    assert np.all(np.isfinite(got_rows)), what
    diff = got_rows - ref
    max_abs = float(np.max(np.abs(diff)))
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    print("%s: max_abs %.3e rel_l2 %.3e" % (what, max_abs, rel), flush=True)
    assert max_abs <= 2e-3 and rel <= 1e-3, what


def test_two_million_patches_one_head(vattn):
    """H = 1, N = 2^21, d = 64: 8192 blocks of one head, a 128M-element span."""
    h, n, d = 1, 1 << 21, 64
    print("H=%d N=%d d=%d" % (h, n, d), flush=True)
    q, k, v = workloads.make_custom(h, n, d, "normal", seed=61)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = vattn.forward(dq, dk, dv)
    torch.cuda.synchronize()
    del dq, dk, dv
    rows = _rows(h, n, 24, seed=1)
    got = out.view(-1, d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    _check(got, oracle.attention_rows_f64(q, k, v, rows), "N=2^21")


def test_sixty_five_thousand_heads(vattn):
    """H = 65536, N = 64, d = 32: a 65536-workgroup grid."""
    h, n, d = 65536, 64, 32
    print("H=%d N=%d d=%d" % (h, n, d), flush=True)
    q, k, v = workloads.make_custom(h, n, d, "normal", seed=62)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    for precision in ("fast", "auto"):
        out = vattn.forward(dq, dk, dv, precision=precision)
        torch.cuda.synchronize()
        rows = _rows(h, n, 400, seed=2)
        got = out.view(-1, d)[torch.from_numpy(rows).cuda()].cpu().numpy()
        _check(got, oracle.attention_rows_f64(q, k, v, rows), "H=65536 %s" % precision)


def test_wide_patch_stride(vattn):
    """Patch-major with 4096 heads of 64 dims: stride_patch = 262144 elements."""
    h, n, d = 4096, 100, 64
    print("patch-major H=%d N=%d d=%d" % (h, n, d), flush=True)
    q, k, v = workloads.make_custom(h, n, d, "sharp", seed=63)
    views = [torch.from_numpy(workloads.to_layout(x, "patch")).cuda().transpose(0, 1)
             for x in (q, k, v)]
    assert views[0].stride() == (d, h * d, 1)
    out = vattn.forward(*views)
    torch.cuda.synchronize()
    rows = _rows(h, n, 300, seed=3)
    got = out.contiguous().view(-1, d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    _check(got, oracle.attention_rows_f64(q, k, v, rows), "stride_patch 262144")


def test_long_f16_rotary_head(vattn):
    """f16 tensors with rotary positions up to 2^18: H = 2, N = 2^18, d = 64."""
    h, n, d = 2, 1 << 18, 64
    print("f16 rotary H=%d N=%d d=%d" % (h, n, d), flush=True)
    q, k, v = (x.astype(np.float16) for x in workloads.make_custom(h, n, d, "normal", seed=64))
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    table = vattn.rope_table(n, 64)
    out = vattn.forward(dq, dk, dv, rope=table)
    torch.cuda.synchronize()
    rows = _rows(h, n, 24, seed=4)
    got = out.view(-1, d)[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref = oracle.attention_rows_f64(oracle.rope_neox_f64(q, 64), oracle.rope_neox_f64(k, 64), v, rows)
    _check(got, ref, "f16 rotary N=2^18")
