"""The top-K-versus-dense comparison (paged_sparse_attention_amd.approx) against
the same comparison computed with the fp64 oracle on a small problem."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from synth import Problem
import gpu_harness as H
from parity import check_selection

pytestmark = pytest.mark.gpu


def test_sparse_vs_dense_metrics(ora):
    from paged_sparse_attention_amd import approx
    p = Problem(hq=8, hkv=2, d=64, ps=16, c=64, n=40, k=6)
    x = synth.make_inputs(p, 61)
    q, kp, vp, do = (H.dev(x[n], p.dtype) for n in ("q", "k_pool", "v_pool", "do"))
    pt = H.dev(x["page_table"])
    shape = dict(hq=p.hq, hkv=p.hkv, d=p.d, ps=p.ps, c=p.c, n=p.n, n_slots=p.slots, dtype=p.dtype)
    dense = approx.run(q, kp, vp, pt, do, top_k=p.n, **shape)
    sparse = approx.run(q, kp, vp, pt, do, top_k=p.k, **shape)
    got = approx.compare(sparse, dense)

    sel = sparse[5].cpu().numpy()
    _, scores = ora.selection(p, x["q"], x["k_pool"], x["page_table"])
    check_selection(sel, scores, p.keff)                       # valid choice (exact or within the tie band)
    full = np.tile(np.arange(p.n, dtype=np.int32), (p.hkv, 1))
    want = {}
    res = {}
    for name, s in (("sparse", sel), ("dense", full)):
        q_ = Problem(p.hq, p.hkv, p.d, p.ps, p.c, p.n, p.n if name == "dense" else p.k, p.dtype)
        o, lse = ora.fwd(q_, x["q"], x["k_pool"], x["v_pool"], x["page_table"], s)
        dq, dk, dv = ora.bwd(q_, x["q"], x["k_pool"], x["v_pool"], x["page_table"], s, x["do"])
        pool_k = np.zeros((p.slots, p.hkv, p.ps, p.d))
        pool_v = np.zeros_like(pool_k)
        slot, row = ora.key_slots(q_, x["page_table"], s)
        for h in range(p.hkv):
            np.add.at(pool_k, (slot[h], h, row[h]), dk[h])
            np.add.at(pool_v, (slot[h], h, row[h]), dv[h])
        res[name] = (o, lse, dq, pool_k, pool_v)
    rel = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))
    (o_s, l_s, dq_s, k_s, v_s), (o_d, l_d, dq_d, k_d, v_d) = res["sparse"], res["dense"]
    want = {"rel_err_O": rel(o_s, o_d), "rel_err_dQ": rel(dq_s, dq_d), "rel_err_dK": rel(k_s, k_d),
            "rel_err_dV": rel(v_s, v_d), "mass_mean": float(np.exp(l_s - l_d).mean()),
            "mass_min": float(np.exp(l_s - l_d).min())}
    H.say(f"  gpu {got}\n  oracle {want}")
    for key, w in want.items():
        # the metrics are norms of differences of bf16-rounded outputs: agree to a few 1e-3 relative
        assert abs(got[key] - w) <= 2e-2 * abs(w) + 2e-3, (key, got[key], w)
