"""GPU parity of the f16-tensor entry point (vattn_forward_f16) against the
float64 oracle.  Inputs are the f32 draws rounded to f16; the oracle reads
those f16 values promoted exactly to float64.  The GPU result is f16, so the
comparison includes its final rounding (at most 2^-12 relative), inside the
usual tolerance: max-abs <= 2e-3 and relative L2 <= 1e-3.
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


def _f16(h, n, d, kind, seed):
    return tuple(x.astype(np.float16) for x in workloads.make_custom(h, n, d, kind, seed=seed))


def _run(vattn, q, k, v, precision, layout="head"):
    dev = [torch.from_numpy(workloads.to_layout(x, layout)).cuda() for x in (q, k, v)]
    if layout == "patch":
        dev = [t.transpose(0, 1) for t in dev]
    out = vattn.forward(*dev, precision=precision)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    return out.contiguous().cpu().numpy()


@pytest.mark.parametrize("wid", [8])
@pytest.mark.parametrize("precision", ["fast", "auto", "split"])
def test_f16_workload_full(vattn, wid, precision):
    q, k, v = workloads.make_inputs(wid)
    assert q.dtype == np.float16
    _assert_close(_run(vattn, q, k, v, precision), oracle.attention_f64(q, k, v),
                  "workload %d %s" % (wid, precision))


@pytest.mark.parametrize("precision", ["auto", "split"])
def test_f16_sharp_workload_full_tensor(vattn, precision):
    """Workload 9 (sharp 128 x 4096 x 64, f16 tensors) as the benchmark
    launches it; every output element against the oracle."""
    q, k, v = workloads.make_inputs(9)
    _assert_close(_run(vattn, q, k, v, precision), full_size.reference(9),
                  "workload 9 %s" % precision)


@pytest.mark.parametrize("d", [32, 64, 40, 17])
@pytest.mark.parametrize("n", [1, 63, 65, 257, 1000])
@pytest.mark.parametrize("layout", ["head", "patch"])
def test_f16_shapes(vattn, d, n, layout):
    for precision in ("fast", "auto"):
        print("f16 d %d N %d %s %s" % (d, n, layout, precision), flush=True)
        q, k, v = _f16(3, n, d, "normal", seed=3 * d + n)
        _assert_close(_run(vattn, q, k, v, precision, layout), oracle.attention_f64(q, k, v),
                      "f16 d=%d N=%d %s %s" % (d, n, layout, precision))


def test_f16_sharp_small(vattn):
    q, k, v = _f16(4, 777, 64, "sharp", seed=77)
    _assert_close(_run(vattn, q, k, v, "auto"), oracle.attention_f64(q, k, v), "f16 sharp small")


def test_f16_constant_v_is_exact(vattn):
    rng = np.random.default_rng(8)
    h, n, d = 2, 300, 64
    q = (rng.standard_normal((h, n, d)) * 0.3).astype(np.float16)
    k = rng.standard_normal((h, n, d)).astype(np.float16)
    v = np.full((h, n, d), 0.75, np.float16)
    out = _run(vattn, q, k, v, "auto")
    assert np.all(out == np.float16(0.75))


def test_f16_c_abi_direct(vattn):
    h, n, d = 2, 300, 64
    q, k, v = _f16(h, n, d, "normal", seed=31)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = torch.empty_like(dq)
    rc = vattn.forward_f16_raw(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), out.data_ptr(),
                               h, n, d, n * d, d, torch.cuda.current_stream().cuda_stream, "auto")
    assert rc == 0
    torch.cuda.synchronize()
    _assert_close(out.cpu().numpy(), oracle.attention_f64(q, k, v), "f16 c-abi")
