"""Seeded random parity sweep across the option space: element type, layout,
head_dim (padded or not), rotary dims, precision mode and grid size.  The
head counts are drawn around the grid sizes where the launcher switches
kernels (16-wave, 8-wave, split-key and 4-wave workgroups), so every kernel
meets every option.  The oracle computes sampled rows in float64; tolerance
as everywhere: max-abs <= 2e-3 and relative L2 <= 1e-3.  FAST runs only on
normal-scale logits (sharp logits need the split product, see the precision
modes in include/vattn.h)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _cases(count=48, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        n = int(rng.choice([1, 63, 64, 65, 200, 257, 300, 511]))
        # 256-row blocks per head, and the grid sizes where the kernel changes
        wide = (n + 255) // 256
        target = int(rng.choice([1, 60, 127, 128, 129, 255, 256, 300]))
        h = max(1, min(400, target // wide))
        d = int(rng.choice([64, 32, 40, 17, 48, 8]))
        dtype = str(rng.choice(["f32", "f16"]))
        layout = str(rng.choice(["head", "patch"]))
        rope_choices = [0] + [r for r in (8, 16, 32, 64) if r <= d]
        rope_dims = int(rng.choice(rope_choices))
        kind = str(rng.choice(["normal", "sharp"]))
        precision = str(rng.choice(["auto", "split", "fast"] if kind == "normal"
                                   else ["auto", "split"]))
        cases.append((i, h, n, d, dtype, layout, rope_dims, kind, precision))
    return cases


CASES = _cases()


@pytest.fixture(scope="module")
def vattn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import non_causal_flash_amd as m
    return m


@pytest.mark.parametrize("i,h,n,d,dtype,layout,rope_dims,kind,precision", CASES,
                         ids=["%d-H%d-N%d-d%d-%s-%s-r%d-%s-%s" % c for c in CASES])
def test_random_option_mix(vattn, i, h, n, d, dtype, layout, rope_dims, kind, precision):
    q, k, v = workloads.make_custom(h, n, d, kind, seed=7000 + i)
    if dtype == "f16":
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
    dev = []
    for x in (q, k, v):
        t = torch.from_numpy(workloads.to_layout(x, layout)).cuda()
        dev.append(t.transpose(0, 1) if layout == "patch" else t)
    table = vattn.rope_table(n, rope_dims) if rope_dims else None
    out = vattn.forward(*dev, precision=precision, rope=table)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(h, n, per_head=3, seed=i)
    qq, kk = q, k
    if rope_dims:
        qq, kk = oracle.rope_neox_f64(q, rope_dims), oracle.rope_neox_f64(k, rope_dims)
    ref = oracle.attention_rows_f64(qq, kk, v, rows)
    got = out.float().contiguous().cpu().numpy().reshape(-1, d)[rows].astype(np.float64)
    assert np.all(np.isfinite(got))
    diff = got - ref
    max_abs = float(np.max(np.abs(diff)))
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    assert max_abs <= 2e-3 and rel <= 1e-3, (max_abs, rel)
