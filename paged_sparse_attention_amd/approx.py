"""How far top-K page attention is from dense attention on the same inputs.

The OOMB page keeps only the top-K pages of the earlier context per chunk and
kv-head ("Page-level Sparse Attention", technical summary, section 2) and
reports that the approximation preserves accuracy (section 4).  This module
measures the approximation itself for one chunk step: the same inputs run once
with top-K selection and once with every prior page selected (dense), both
through the library, and the outputs and gradients are compared.

Reported per K:
  - rel_err of O, dQ, dK, dV: ||sparse - dense|| / ||dense|| (Frobenius; dK and
    dV over the whole gradient pools);
  - mass_mean / mass_min: the share of each row's dense softmax mass that the
    sparse key set holds, exp(LSE_sparse - LSE_dense), averaged / minimised over
    rows (the sparse keys are a subset of the dense ones, so this is <= 1).

    python -m paged_sparse_attention_amd.approx [--workload sparse-256k] [--k 64,128]
"""
from __future__ import annotations

import argparse
import json

import torch

from .step import ChunkStep


def _norm(t):
    return float(torch.linalg.vector_norm(t.double()))


def run(q, k_pool, v_pool, page_table, dO, *, hq, hkv, d, ps, c, n, top_k, n_slots, dtype, scale=0.0):
    """One chunk step with the given top_k; fresh zero gradient pools.
    Returns (O, LSE, dQ, dK pool, dV pool, selected pages) as device tensors."""
    st = ChunkStep(hq, hkv, d, ps, c, n, top_k, n_slots, dtype=dtype, softmax_scale=scale)
    dk = torch.zeros(k_pool.shape, dtype=torch.float32, device=k_pool.device)
    dv = torch.zeros_like(dk)
    st.rep_update(k_pool, page_table, 0, n + c // ps)
    st.select(q, keep_scores=False)
    st.fwd(q, k_pool, v_pool, page_table)
    st.bwd(q, k_pool, v_pool, page_table, dO, dk, dv)
    torch.cuda.synchronize()
    return st.o.clone(), st.lse.clone(), st.dq.clone(), dk, dv, st.sel[:, :st.keff].clone()


def compare(sparse, dense):
    """Relative errors of (O, dQ, dK, dV) and the softmax mass the sparse keys keep."""
    o_s, lse_s, dq_s, dk_s, dv_s = sparse[:5]
    o_d, lse_d, dq_d, dk_d, dv_d = dense[:5]
    mass = torch.exp((lse_s - lse_d).double())
    rel = lambda a, b: _norm(a.float() - b.float()) / max(_norm(b), 1e-300)
    return {"rel_err_O": rel(o_s, o_d), "rel_err_dQ": rel(dq_s, dq_d), "rel_err_dK": rel(dk_s, dk_d),
            "rel_err_dV": rel(dv_s, dv_d), "mass_mean": float(mass.mean()), "mass_min": float(mass.min())}


def main():
    import numpy as np

    import synth

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="sparse-256k")
    ap.add_argument("--k", default="64,128", help="comma-separated top-K values")
    args = ap.parse_args()
    seed, p = synth.WORKLOADS[args.workload]
    x = synth.make_inputs(p, seed)
    bf = p.dtype == "bf16"

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf else t).cuda()

    q, kp, vp, do, pt = dev(x["q"]), dev(x["k_pool"]), dev(x["v_pool"]), dev(x["do"]), \
        torch.from_numpy(x["page_table"]).cuda()
    shape = dict(hq=p.hq, hkv=p.hkv, d=p.d, ps=p.ps, c=p.c, n=p.n, n_slots=p.slots, dtype=p.dtype, scale=p.scale)
    dense = run(q, kp, vp, pt, do, top_k=p.n, **shape)
    for k in (int(v) for v in args.k.split(",")):
        r = compare(run(q, kp, vp, pt, do, top_k=k, **shape), dense)
        r.update({"workload": args.workload, "top_k": k, "prior_pages": p.n,
                  "selected_fraction": min(k, p.n) / max(p.n, 1)})
        print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
