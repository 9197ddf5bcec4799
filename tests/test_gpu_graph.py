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


CASES = [  # (H, N, d, kind, rope_dims): split-key, 16-wave and rotary kernels
    (16, 1024, 64, "normal", 0),
    (128, 300, 64, "sharp", 0),
    (16, 1024, 64, "normal", 64),
]


@pytest.mark.parametrize("h,n,d,kind,rope_dims", CASES)
def test_graph_replays_match_eager(vattn, h, n, d, kind, rope_dims):
    seeds = [3, 4, 5]
    q, k, v = workloads.make_custom(h, n, d, kind, seed=seeds[0])
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = torch.empty_like(dq)
    table = vattn.rope_table(n, rope_dims) if rope_dims else None
    vattn.forward(dq, dk, dv, out=out, rope=table)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vattn.forward(dq, dk, dv, out=out, rope=table)
    for i, seed in enumerate(seeds):
        x = workloads.make_custom(h, n, d, kind, seed=seed)
        for dst, src in zip((dq, dk, dv), x):
            dst.copy_(torch.from_numpy(src))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = vattn.forward(dq, dk, dv, rope=table)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), "replay %d differs from the eager call" % i
        if i == 0:
            qq, kk, vv = x
            if rope_dims:
                qq, kk = oracle.rope_neox_f64(qq, rope_dims), oracle.rope_neox_f64(kk, rope_dims)
            rows = workloads.sample_rows(h, n, per_head=2)
            ref = oracle.attention_rows_f64(qq, kk, vv, rows)
            diff = got.cpu().numpy().reshape(-1, d)[rows].astype(np.float64) - ref
            assert np.max(np.abs(diff)) <= 2e-3
            assert np.linalg.norm(diff) / np.linalg.norm(ref) <= 1e-3
