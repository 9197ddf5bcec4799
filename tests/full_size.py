"""Float64 oracle outputs of whole benchmark workloads, computed once per
test process: several GPU test modules compare full-size results with the
same workload.  The rotary workloads get the oracle's NeoX rotation of Q
and K first (patch n at position n)."""
from __future__ import annotations

import functools

import oracle
import workloads


@functools.lru_cache(maxsize=None)
def reference(wid: int):
    w = workloads.WORKLOADS[wid]
    q, k, v = workloads.make_inputs(wid)
    if w.rope_dims:
        q = oracle.rope_neox_f64(q, w.rope_dims, w.rope_base)
        k = oracle.rope_neox_f64(k, w.rope_dims, w.rope_base)
    out = oracle.attention_f64(q, k, v)
    out.setflags(write=False)
    return out
