"""HIP-graph capture of the C-ABI launches (what bench.py times).

A graph captured from ``forward`` must recompute on every replay: the
inputs are overwritten between replays, with eager launches and
synchronisations in between, and every replay is compared with an eager
call on the same inputs (bit for bit: the kernels are deterministic) and
with the float64 oracle.
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


CASES = [  # (H, N, d, kind, rope_dims, dtype, layout)
    (16, 1024, 64, "normal", 0, "f32", "head"),   # split-key kernel
    (128, 300, 64, "sharp", 0, "f32", "head"),    # 16-wave kernel
    (16, 1024, 64, "normal", 64, "f32", "head"),  # rotary
    (128, 300, 64, "sharp", 0, "f16", "head"),    # f16 entry
    (16, 300, 40, "normal", 0, "f32", "patch"),   # strided entry, padded head_dim
]


def _device(x, dtype, layout):
    """[H][N][d] host array as a device view in the workload's storage order."""
    x = workloads.to_layout(x.astype(np.float16) if dtype == "f16" else x, layout)
    t = torch.from_numpy(x).cuda()
    return t.transpose(0, 1) if layout == "patch" else t


@pytest.mark.parametrize("h,n,d,kind,rope_dims,dtype,layout", CASES)
def test_graph_replays_match_eager(vattn, h, n, d, kind, rope_dims, dtype, layout):
    seeds = [3, 4, 5]
    dq, dk, dv = (_device(x, dtype, layout)
                  for x in workloads.make_custom(h, n, d, kind, seed=seeds[0]))
    out = torch.empty_strided(dq.shape, dq.stride(), dtype=dq.dtype, device=dq.device)
    table = vattn.rope_table(n, rope_dims) if rope_dims else None
    vattn.forward(dq, dk, dv, out=out, rope=table)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vattn.forward(dq, dk, dv, out=out, rope=table)
    for i, seed in enumerate(seeds):
        x = workloads.make_custom(h, n, d, kind, seed=seed)
        for dst, src in zip((dq, dk, dv), x):
            dst.copy_(_device(src, dtype, layout))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = vattn.forward(dq, dk, dv, rope=table)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), "replay %d differs from the eager call" % i
        if i == 0:
            qq, kk, vv = (a.astype(np.float16) if dtype == "f16" else a for a in x)
            if rope_dims:
                qq, kk = oracle.rope_neox_f64(qq, rope_dims), oracle.rope_neox_f64(kk, rope_dims)
            rows = workloads.sample_rows(h, n, per_head=2)
            ref = oracle.attention_rows_f64(qq, kk, vv, rows)
            host = got.float().contiguous().cpu().numpy().reshape(-1, d)
            diff = host[rows].astype(np.float64) - ref
            assert np.max(np.abs(diff)) <= 2e-3
            assert np.linalg.norm(diff) / np.linalg.norm(ref) <= 1e-3
