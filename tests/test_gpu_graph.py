"""A whole chunk step captured in a HIP graph (torch.cuda.graph over the
library's stream-ordered entry points) replays to the same bytes as the eager
calls: the entry points enqueue kernels only, with no memset, copy,
allocation or synchronisation that a capture would record or break.  Each
replay follows eager work of the program (pool reset, output poisoning) and a
synchronisation, and every replay is checked, not just the first."""
import numpy as np
import pytest
import torch

import synth
from synth import Problem
import gpu_harness as H

pytestmark = pytest.mark.gpu

CASES = {
    "xcd-pairs-g3": (39, Problem(hq=12, hkv=4, d=128, ps=64, c=512, n=30, k=6)),
    "d64-bf16-g7": (30, Problem(hq=14, hkv=2, d=64, ps=16, c=112, n=31, k=9)),
    "mha-fp32-d128": (26, Problem(hq=2, hkv=2, d=128, ps=32, c=64, n=9, k=3, dtype="f32")),
}


def _bytes(t):
    return t.view(torch.uint8) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    seed, p = CASES[name]
    H.say(f"[graph] {name}")
    x = synth.make_inputs(p, seed)
    d = H.Device(p, x)
    st = H.make_step(p)
    st.rep_update(d.k, d.pt, 0, p.n)  # prior pages' rep vectors: set-up, outside the step

    def run_step():
        st.step(d.q, d.k, d.v, d.pt, d.do, d.dk, d.dv)

    def outputs():
        return [t.clone() for t in (st.rep, st.sel, st.o, st.lse, st.dq, d.dk, d.dv)]

    def reset():
        d.dk.fill_(0.5)
        d.dv.fill_(-0.25)
        st.o.fill_(3.0)
        st.lse.fill_(3.0)
        st.dq.fill_(3.0)

    reset()
    run_step()
    torch.cuda.synchronize()
    want = outputs()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_step()
    torch.cuda.synchronize()

    names = ("rep", "sel", "o", "lse", "dq", "dk_pool", "dv_pool")
    for r in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(names, want, outputs()):
            assert torch.equal(_bytes(a), _bytes(b)), f"replay {r}: {n} differs from the eager step"
