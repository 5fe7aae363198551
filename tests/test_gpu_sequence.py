"""Chunk-recurrent attention over a whole sequence (ChunkedSequence, the C ABI
called chunk by chunk) against the whole-sequence oracle, element by element.

Per chunk: the selected pages (identical, or inside the near-tie band), O, LSE
and dQ; for the whole sequence: the dK/dV pools, which every chunk's backward
adds into (compared as pool after minus the seeded prefill).  The driver's
recompute modes (the forward re-run in the backward with the saved selection:
serially with one activation buffer, or on a second stream alongside the next
chunk's backward with two) must give bitwise the results of the mode that keeps
every chunk's O and LSE."""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import synth
from synth import Sequence
import gpu_harness as H
from parity import check_selection, compare, compare_lse

pytestmark = pytest.mark.gpu

SEQ = {
    "seq-bf16-ps16": (51, Sequence(hq=4, hkv=2, d=64, ps=16, c=64, chunks=4, k=3, n0=2)),
    "seq-fp32-no-context": (52, Sequence(hq=4, hkv=2, d=64, ps=16, c=32, chunks=5, k=2, n0=0, dtype="f32")),
    "seq-qwen-shape": (53, Sequence(hq=28, hkv=4, d=128, ps=128, c=512, chunks=4, k=2, n0=4)),
    "seq-dense-all-pages": (54, Sequence(hq=8, hkv=2, d=128, ps=64, c=128, chunks=3, k=1000, n0=1)),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")


def run_sequence(s, seed, keep=True, raw=None, overlap=True, stream=None):
    """Forward and backward over the sequence.  raw, if a dict, receives every
    chunk's O and LSE (copied as the forward produces them) and the pools."""
    from paged_sparse_attention_amd.sequence import ChunkedSequence
    x = synth.make_sequence_inputs(s, seed)
    last = s.step(s.chunks - 1)
    q, k, v, do = (H.dev(x[n], s.dtype) for n in ("q", "k_pool", "v_pool", "do"))
    pt = H.dev(x["page_table"])
    dk0, dv0 = synth.canary(last, seed, "k"), synth.canary(last, seed, "v")
    dk, dv = H.dev(dk0), H.dev(dv0)
    drv = ChunkedSequence(s.hq, s.hkv, s.d, s.ps, s.c, s.chunks, s.k, n_initial_pages=s.n0, dtype=s.dtype,
                          softmax_scale=s.scale, keep_activations=keep, overlap_recompute=overlap)
    outs = []
    st = stream if stream is not None else torch.cuda.current_stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        drv.forward(q, k, v, pt, stream=stream, on_chunk=lambda i, o, lse: outs.append((o.clone(), lse.clone())))
        drv.backward(q, k, v, pt, do, dk, dv, stream=stream)
    torch.cuda.synchronize()
    if raw is not None:
        raw.update(o=[o for o, _ in outs], lse=[l for _, l in outs], dk=dk, dv=dv)
    return x, drv, dk.cpu().numpy().astype(np.float64) - dk0, dv.cpu().numpy().astype(np.float64) - dv0


@pytest.mark.parametrize("name", list(SEQ))
def test_sequence_elementwise(ora, name):
    seed, s = SEQ[name]
    H.say(f"case {name}: {s}")
    x, drv, gdk, gdv = run_sequence(s, seed)
    r = ora.sequence(s, x)
    sels, exact = [], True
    for i in range(s.chunks):
        keff = drv.keff(i)
        g = drv.sel[i][:, :keff].cpu().numpy() if keff else np.zeros((s.hkv, 0), np.int32)
        if keff:
            exact &= check_selection(g, r["scores"][i], keff)
        sels.append(g)
    if not exact:                                  # near ties: the oracle takes the GPU's pages
        r = ora.sequence(s, x, sels=sels)
    report = {"sel_exact": bool(exact)}
    for i in range(s.chunks):
        rep_i = {}
        compare("O", H.host(drv.o[i]).reshape(-1, s.d), r["o"][i], s.dtype, rep_i)
        compare_lse(drv.lse[i].cpu().numpy().T.reshape(-1), r["lse"][i], s.dtype, rep_i)
        compare("dQ", drv.dq[i].cpu().numpy().reshape(-1, s.d), r["dq"][i], s.dtype, rep_i)
        report[f"chunk{i}"] = rep_i
    compare("dK pool", gdk, r["dk"], s.dtype, report)
    compare("dV pool", gdv, r["dv"], s.dtype, report)
    H.say(f"  {json.dumps(report, default=float)}")


@pytest.mark.parametrize("name", ["seq-bf16-ps16", "seq-fp32-no-context", "seq-qwen-shape"])
def test_recompute_matches_kept_activations(name):
    seed, s = SEQ[name]
    H.say(f"case {name} recompute: {s}")
    kept = {}
    _, a, _, _ = run_sequence(s, seed, keep=True, raw=kept)
    for overlap, nbuf in ((False, 1), (True, 2)):
        redo = {}
        _, b, _, _ = run_sequence(s, seed, keep=False, raw=redo, overlap=overlap)
        assert b.o.shape[0] == nbuf and b.lse.shape[0] == nbuf     # activations of one or two chunks only
        for i in range(s.chunks):
            assert torch.equal(a.sel[i], b.sel[i]), f"chunk {i} selection"
            assert torch.equal(kept["o"][i], redo["o"][i]), f"chunk {i} O"
            assert torch.equal(kept["o"][i], a.o[i]), f"chunk {i} O handed to the callback"
            assert torch.equal(kept["lse"][i], redo["lse"][i]), f"chunk {i} LSE"
            assert torch.equal(a.dq[i], b.dq[i]), f"chunk {i} dQ (overlap {overlap})"
        assert torch.equal(kept["dk"], redo["dk"]) and torch.equal(kept["dv"], redo["dv"]), \
            f"dK/dV pools (overlap {overlap})"


def test_overlapped_recompute_on_a_caller_stream():
    """The overlapped re-run backward ordered on a stream the caller passes
    (not the default one) gives bitwise the results of kept activations."""
    seed, s = SEQ["seq-qwen-shape"]
    H.say("case seq-qwen-shape, recompute on a caller stream")
    kept, redo = {}, {}
    _, a, _, _ = run_sequence(s, seed, keep=True, raw=kept)
    _, b, _, _ = run_sequence(s, seed, keep=False, raw=redo, overlap=True, stream=torch.cuda.Stream())
    for i in range(s.chunks):
        assert torch.equal(kept["o"][i], redo["o"][i]), f"chunk {i} O"
        assert torch.equal(a.dq[i], b.dq[i]), f"chunk {i} dQ"
    assert torch.equal(kept["dk"], redo["dk"]) and torch.equal(kept["dv"], redo["dv"]), "dK/dV pools"
