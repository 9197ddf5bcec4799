"""GPU parity of the strided access modes and of head_dim values other than
32 and 64, against the float64 oracle (which always reads head-major
arrays: a patch-major case gives the oracle the same values transposed on
the host).

Tolerance as for the head-major cases: max-abs <= 2e-3 and relative L2
<= 1e-3 over the compared elements.
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


def _patch_major_views(x):
    """Contiguous [N][H][d] device copy of a head-major array, seen as [H, N, d]."""
    t = torch.from_numpy(workloads.to_layout(x, "patch")).cuda()
    return t.transpose(0, 1)


def _run_patch_major(vattn, q, k, v, precision):
    dq, dk, dv = (_patch_major_views(x) for x in (q, k, v))
    out = vattn.forward(dq, dk, dv, precision=precision)
    torch.cuda.synchronize()
    assert out.stride() == dq.stride()
    return out.contiguous().cpu().numpy()


HEAD_DIMS = [1, 3, 8, 16, 20, 24, 33, 40, 48, 56, 63]


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("n", [1, 65, 300])
def test_any_head_dim_head_major(vattn, d, n):
    for h, precision in ((2, "fast"), (3, "auto")):
        print("head_dim %d N %d H %d %s" % (d, n, h, precision), flush=True)
        q, k, v = workloads.make_custom(h, n, d, "normal", seed=13 * d + n + h)
        dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
        out = vattn.forward(dq, dk, dv, precision=precision)
        torch.cuda.synchronize()
        _assert_close(out.cpu().numpy(), oracle.attention_f64(q, k, v),
                      "d=%d N=%d H=%d %s" % (d, n, h, precision))


@pytest.mark.parametrize("d", [32, 64, 40, 41])
@pytest.mark.parametrize("n", [1, 100, 257, 1000, 4097])
def test_patch_major(vattn, d, n):
    for precision in ("fast", "auto", "split"):
        print("patch-major d %d N %d %s" % (d, n, precision), flush=True)
        q, k, v = workloads.make_custom(3, n, d, "normal", seed=7 * d + n)
        _assert_close(_run_patch_major(vattn, q, k, v, precision), oracle.attention_f64(q, k, v),
                      "patch-major d=%d N=%d %s" % (d, n, precision))


@pytest.mark.parametrize("d", [32, 64])
def test_patch_major_equals_head_major_bitwise(vattn, d):
    """With head_dim 32 or 64 the strided kernels run the same arithmetic in
    the same order as the contiguous fast path: the outputs agree exactly."""
    q, k, v = workloads.make_custom(4, 777, d, "sharp", seed=5 + d)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    for precision in ("fast", "auto"):
        dense = vattn.forward(dq, dk, dv, precision=precision)
        torch.cuda.synchronize()
        strided = _run_patch_major(vattn, q, k, v, precision)
        assert np.array_equal(dense.cpu().numpy(), strided), precision


@pytest.mark.parametrize("d,pitch", [(40, 48), (64, 72), (33, 36), (17, 17)])
def test_padded_rows_untouched(vattn, d, pitch):
    """Rows with a pitch larger than head_dim and NaN in the padding columns:
    nothing outside the [H][N][d] elements is read (the output stays finite)
    or written (the padding of out stays NaN)."""
    h, n = 2, 300
    q, k, v = workloads.make_custom(h, n, d, "normal", seed=d + pitch)

    def padded(x):
        buf = torch.full((h, n, pitch), float("nan"), device="cuda")
        buf[:, :, :d] = torch.from_numpy(x).cuda()
        return buf

    bufs = [padded(x) for x in (q, k, v)]
    obuf = torch.full((h, n, pitch), float("nan"), device="cuda")
    views = [b[:, :, :d] for b in bufs]
    out = vattn.forward(*views, out=obuf[:, :, :d], precision="auto")
    torch.cuda.synchronize()
    host = obuf.cpu().numpy()
    if pitch > d:
        assert np.all(np.isnan(host[:, :, d:]))
    _assert_close(host[:, :, :d], oracle.attention_f64(q, k, v), "pitch %d d %d" % (pitch, d))
    assert out.data_ptr() == obuf.data_ptr()


def test_patch_major_sharp_workload_full_tensor(vattn):
    """Workload 6 (the sharp 128 x 4096 x 64 case stored patch-major) as the
    benchmark launches it; every output element against the oracle."""
    q, k, v = workloads.make_inputs(6)
    _assert_close(_run_patch_major(vattn, q, k, v, "auto"), full_size.reference(6),
                  "workload 6")


def test_head_dim_40_workload_full(vattn):
    w = workloads.WORKLOADS[7]
    q, k, v = workloads.make_inputs(7)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = vattn.forward(dq, dk, dv)
    torch.cuda.synchronize()
    _assert_close(out.cpu().numpy(), oracle.attention_f64(q, k, v), "workload 7")


def test_strided_c_abi_direct(vattn):
    """vattn_forward_strided with raw pointers: patch-major with a padded
    patch stride (heads packed, 8 floats of padding after each patch)."""
    h, n, d = 3, 200, 32
    q, k, v = workloads.make_custom(h, n, d, "normal", seed=21)
    sn = h * d + 8
    bufs = []
    for x in (q, k, v):
        b = torch.zeros(n, sn, device="cuda")
        b[:, :h * d] = torch.from_numpy(workloads.to_layout(x, "patch").reshape(n, h * d)).cuda()
        bufs.append(b)
    ob = torch.full((n, sn), float("nan"), device="cuda")
    rc = vattn.forward_strided_raw(bufs[0].data_ptr(), bufs[1].data_ptr(), bufs[2].data_ptr(),
                                   ob.data_ptr(), h, n, d, d, sn,
                                   torch.cuda.current_stream().cuda_stream, "auto")
    assert rc == 0
    torch.cuda.synchronize()
    host = ob.cpu().numpy()
    assert np.all(np.isnan(host[:, h * d:]))
    got = host[:, :h * d].reshape(n, h, d).transpose(1, 0, 2)
    _assert_close(got, oracle.attention_f64(q, k, v), "strided c-abi")


# Grids that select each kernel shape: 16-wave blocks (256 rows) when there
# are more than 128 of them, 8-wave blocks while 2x that reaches 256; below,
# the split-key kernel while there are at most 256 64-row blocks, else
# 8-wave blocks again (the rotary kernels use 4-wave blocks there).  The 16-wave kernel stores tiles two steps ahead and
# synchronises after every odd step, so it also runs with 1, 2, 3 and 5 key
# tiles (ragged and exact).
WORKGROUP_SHAPES = [("split keys", 2, 1000, 1), ("split keys ragged", 3, 333, 1),
                    ("8 waves below the CU count", 20, 1000, 8), ("8 waves", 32, 1000, 8),
                    ("16 waves above half the CUs", 40, 1000, 16), ("16 waves", 70, 1000, 16),
                    ("16 waves one tile", 300, 64, 16), ("16 waves two tiles", 300, 128, 16),
                    ("16 waves three tiles ragged", 300, 150, 16),
                    ("16 waves five tiles ragged", 260, 300, 16)]


@pytest.mark.parametrize("label,h,n,shape", WORKGROUP_SHAPES,
                         ids=[s[0] for s in WORKGROUP_SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_every_workgroup_shape(vattn, label, h, n, shape, dtype):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    chosen = vattn.launch_shape(h, n, 64, False, cus)
    print("%s: H=%d N=%d, %d CUs, shape %d" % (label, h, n, cus, chosen), flush=True)
    if cus == 256:
        assert chosen == shape
    q, k, v = workloads.make_custom(h, n, 64, "sharp", seed=h + n)
    if dtype == "f16":
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    rows = workloads.sample_rows(h, n, per_head=12)
    ref = oracle.attention_rows_f64(q, k, v, rows)
    for precision in ("auto", "split"):
        out = vattn.forward(dq, dk, dv, precision=precision)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().reshape(-1, 64)[rows]
        _assert_close(got, ref, "%s %s %s" % (label, dtype, precision))
