"""HIP path against the fp64 oracle on an MI355X, through the C ABI.

Small problems: every output element by element (they span several tiles and
have ragged tails).  Full-size workloads: exact rep vectors and selection,
O/LSE/dQ on sampled rows (one in every row block and query head; every row at
sparse-256k), the last chunk keys,
invariants, and every key's dK/dV under a dO supported on sampled rows.  Bars:
see parity.py."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from synth import Problem, WORKLOADS
import gpu_harness as H
from parity import ZERO_REF

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny-fp32": (1, WORKLOADS["tiny-fp32"][1]),
    "gqa7-ps64-ragged": (21, Problem(hq=28, hkv=4, d=128, ps=64, c=320, n=24, k=6)),
    "qwen-ps128": (22, Problem(hq=28, hkv=4, d=128, ps=128, c=256, n=12, k=4)),
    "dense-k-ge-n": (23, Problem(hq=8, hkv=2, d=128, ps=64, c=128, n=6, k=10)),
    "k0-local-only": (24, Problem(hq=4, hkv=1, d=128, ps=16, c=48, n=5, k=0)),
    "n0-no-prior": (25, Problem(hq=4, hkv=2, d=64, ps=32, c=96, n=0, k=4)),
    "mha-fp32-d128": (26, Problem(hq=2, hkv=2, d=128, ps=32, c=64, n=9, k=3, dtype="f32")),
    "one-page-chunk": (27, Problem(hq=12, hkv=3, d=64, ps=16, c=16, n=40, k=7)),
    "extra-slots": (28, Problem(hq=6, hkv=2, d=64, ps=32, c=64, n=10, k=4, n_slots=30)),
    "scale-override-fp32": (29, Problem(hq=4, hkv=2, d=64, ps=16, c=32, n=8, k=3, dtype="f32", scale=0.05)),
    "d64-bf16-g7": (30, Problem(hq=14, hkv=2, d=64, ps=16, c=112, n=31, k=9)),
    # more key pages than the kernels' LDS page-slot cache holds (1024): slots
    # are then read from the page table for every tile
    "uncached-pages-dense": (31, Problem(hq=4, hkv=1, d=64, ps=16, c=32, n=1100, k=2000)),
    "uncached-pages-topk": (32, Problem(hq=8, hkv=2, d=128, ps=16, c=64, n=1500, k=1100)),
    "mha-bf16": (33, Problem(hq=4, hkv=4, d=128, ps=64, c=128, n=10, k=3)),
    "gqa32-d64": (34, Problem(hq=32, hkv=1, d=64, ps=32, c=64, n=12, k=5)),
    "ps32-d128": (35, Problem(hq=8, hkv=2, d=128, ps=32, c=96, n=20, k=7)),
    "k-one-below-n": (36, Problem(hq=4, hkv=2, d=64, ps=16, c=32, n=9, k=8)),
    "scale-override-bf16": (37, Problem(hq=6, hkv=3, d=128, ps=128, c=128, n=5, k=2, scale=0.05)),
    # work orders over the XCDs: one XCD per kv-head (8 kv-heads), with 8 row
    # splits of dK/dV, so 8 row-share groups per XCD
    "kv8-xcd-per-head": (38, Problem(hq=16, hkv=8, d=128, ps=32, c=256, n=24, k=5)),
    # two XCDs per kv-head taking its 6 row blocks in turn, and 4 dK/dV
    # row-share groups per XCD
    "xcd-pairs-g3": (39, Problem(hq=12, hkv=4, d=128, ps=64, c=512, n=30, k=6)),
}

FULL = ["dense-32k", "sparse-1m", "sparse-4m"]     # sampled rows
EVERY_ROW = ["sparse-256k"]                         # every row of O, LSE and dQ

# Known limit of R16 (P and dS rounded to bf16 before their MFMAs): with a
# softmax scale of 0.2 (2.3 x 1/sqrt(128)) dQ and dK reach 5.0 and 5.9 in
# magnitude, and the rounding of dS is relative (at most 2^-8 of each term),
# so their max-abs error (0.0247 and 0.0246 measured on MI355X) exceeds the
# absolute 2e-2 bar, which the benchmark workloads (outputs below 1) meet with
# a wide margin.  O, dV, LSE and the selection still meet the official bars.
LARGE_SCALE = (37, Problem(hq=6, hkv=3, d=128, ps=128, c=128, n=5, k=2, scale=0.2))
LARGE_SCALE_REL = 4 * 2.0 ** -8   # dQ, dK: max-abs <= 4 u max|ref|, u = 2^-8 (bf16 unit roundoff)

REPORT_DIR = os.environ.get("OOMB_PARITY_REPORT_DIR")


def _save(name, report):
    if REPORT_DIR:
        os.makedirs(REPORT_DIR, exist_ok=True)
        with open(os.path.join(REPORT_DIR, f"parity_{name}.json"), "w") as f:
            json.dump(report, f, indent=1, default=float)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import paged_sparse_attention_amd as P
    assert len(P.hip_runtimes_loaded()) == 1, P.hip_runtimes_loaded()


@pytest.mark.parametrize("name", list(SMALL))
def test_small_elementwise(ora, name):
    seed, p = SMALL[name]
    H.say(f"case {name}: {p}")
    report, *_ = H.run_full(p, seed, ora)
    H.say(f"  {json.dumps(report, default=float)}")
    _save(name, report)


# Every value vector of a kv-head set to that head's first stored value row:
# O is that vector on every row and dQ = dK = 0 exactly (dO . V_j equals
# Dt = dO . O for every key), so the kernels' Dt and dS must cancel to within
# their rounding.
CONST_V = {
    "const-v-bf16": (51, Problem(hq=28, hkv=4, d=128, ps=128, c=256, n=12, k=4)),
    "const-v-fp32": (52, Problem(hq=4, hkv=2, d=64, ps=16, c=64, n=9, k=3, dtype="f32")),
}


# Q = 0: every score of a row is 0, so the weights are uniform over its visible
# keys (ties everywhere for the running maximum) and O is their mean value.
ZERO_Q = {
    "zero-q-bf16": (53, Problem(hq=28, hkv=4, d=128, ps=128, c=256, n=12, k=4)),
    "zero-q-fp32": (54, Problem(hq=4, hkv=2, d=64, ps=16, c=64, n=9, k=3, dtype="f32")),
}


@pytest.mark.parametrize("name", list(ZERO_Q))
def test_zero_queries(ora, name):
    seed, p = ZERO_Q[name]
    H.say(f"case {name}: {p}")

    def tweak(x):
        x["q"][...] = 0

    report, *_ = H.run_full(p, seed, ora, tweak=tweak)
    H.say(f"  {json.dumps(report, default=float)}")
    _save(name, report)


# Scores that rise along the key list: every query has a component a along one
# unit vector u and key j one of B * j / J, so a row's largest score grows by
# about B (in natural-log units) from the first key to the last and the
# forward's running maximum moves up tile after tile, past its rescaling slack
# several times, instead of settling in the first tiles as with random data.
RISING = (55, Problem(hq=7, hkv=1, d=128, ps=64, c=128, n=32, k=32), 14.0)


def test_rising_scores(ora):
    seed, p, B = RISING
    H.say(f"case rising-scores: {p}, B {B}")
    rng = np.random.default_rng(seed)
    u = rng.normal(size=p.d)
    u /= np.linalg.norm(u)
    nkeys = p.n * p.ps + p.c

    def tweak(x):
        pt = x["page_table"]
        k = synth.as_float(x["k_pool"], p.dtype)
        for m in range(p.n + p.chunk_pages):   # logical page m holds key positions m*ps .. m*ps+ps-1
            j = m * p.ps + np.arange(p.ps)
            k[pt[m]] += (B * j / nkeys)[None, :, None] * u
        x["k_pool"][...] = synth.bf16_bits(k)
        q = synth.as_float(x["q"], p.dtype) + np.sqrt(p.d) * u
        x["q"][...] = synth.bf16_bits(q)

    report, *_ = H.run_full(p, seed, ora, tweak=tweak)
    H.say(f"  {json.dumps(report, default=float)}")
    _save("rising-scores", report)


@pytest.mark.parametrize("name", list(CONST_V))
def test_constant_values(ora, name):
    seed, p = CONST_V[name]
    H.say(f"case {name}: {p}")

    def tweak(x):
        v = x["v_pool"]
        v[...] = v[:1, :, :1, :]   # [slots][hkv][ps][d]: slot 0, row 0 of each head everywhere

    report, st, d, x, sel = H.run_full(p, seed, ora, tweak=tweak)
    H.say(f"  {json.dumps(report, default=float)}")
    # the oracle's dQ and dK are zero up to fp64 rounding, so only the absolute bar applied to them
    assert report["dQ"]["rms_ref"] <= ZERO_REF and report["dK"]["rms_ref"] <= ZERO_REF, report
    _save(name, report)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(ora, name):
    seed, p = WORKLOADS[name]
    H.say(f"workload {name}: {p}")
    report = H.run_sampled(p, seed, ora)
    H.say(f"  {json.dumps(report, default=float)}")
    _save(name, report)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", EVERY_ROW)
def test_full_size_every_row(ora, name):
    """O, LSE and dQ of every row against the oracle at full size, and the keys'
    summed dK against its error model (gpu_harness.sum_dk_model)."""
    seed, p = WORKLOADS[name]
    H.say(f"workload {name} (every row): {p}")
    report = H.run_sampled(p, seed, ora, every_row=True)
    H.say(f"  {json.dumps(report, default=float)}")
    _save(name, report)
    torch.cuda.empty_cache()


def test_bf16_large_scale_known_limit(ora):
    """The documented bf16 limit at a large softmax scale: official bars for the
    selection, O, LSE and dV; dQ and dK held to 4 u max|ref| (u = 2^-8), the
    form that a relative rounding error of dS takes."""
    seed, p = LARGE_SCALE
    H.say(f"case scale-0.2-bf16 (known limit): {p}")
    report, *_ = H.run_full(p, seed, ora, rel_limits={"dQ": LARGE_SCALE_REL, "dK": LARGE_SCALE_REL})
    H.say(f"  {json.dumps(report, default=float)}")
    _save("scale-0.2-bf16-known-limit", report)


def test_deterministic_and_stream(ora):
    """Repeated runs give identical bits; a non-default stream gives the same bits."""
    seed, p = SMALL["gqa7-ps64-ragged"]
    x = synth.make_inputs(p, seed)
    outs = []
    for use_stream in (False, False, True):
        d = H.Device(p, x, canary_seed=seed)
        st = H.make_step(p)
        s = torch.cuda.Stream() if use_stream else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            st.rep_update(d.k, d.pt, 0, p.n + p.chunk_pages)
            st.select(d.q)
            st.fwd(d.q, d.k, d.v, d.pt)
            st.bwd(d.q, d.k, d.v, d.pt, d.do, d.dk, d.dv)
        s.synchronize()
        outs.append([t.cpu().clone() for t in (st.rep, st.scores, st.sel, st.o, st.lse, st.dq, d.dk, d.dv)])
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    for a, b in zip(outs[0], outs[2]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


# Selection alone at page counts around the top-K kernel's variants: every
# score held in registers (up to 2048, 8192 and 32768 pages a head) or read
# again from memory in each radix pass (more pages than that).
SELECT_ONLY = {
    "sel-2048": (41, Problem(hq=4, hkv=2, d=64, ps=16, c=16, n=2048, k=64)),
    "sel-2049-k1": (42, Problem(hq=4, hkv=2, d=64, ps=16, c=16, n=2049, k=1)),
    "sel-8193-k2048": (43, Problem(hq=4, hkv=2, d=64, ps=16, c=16, n=8193, k=2048)),
    "sel-32768": (44, Problem(hq=4, hkv=2, d=64, ps=16, c=16, n=32768, k=128)),
    "sel-40000": (45, Problem(hq=4, hkv=2, d=64, ps=16, c=16, n=40000, k=500)),
}


@pytest.mark.parametrize("name", list(SELECT_ONLY))
def test_select_page_counts(ora, name):
    """Rep vectors, scores and the top-K pages against the oracle."""
    from parity import check_selection
    seed, p = SELECT_ONLY[name]
    H.say(f"[select] {name}")
    x = synth.make_inputs(p, seed)
    st = H.make_step(p)
    k = H.dev(x["k_pool"], p.dtype)
    pt = H.dev(x["page_table"])
    q = H.dev(x["q"], p.dtype)
    st.rep_update(k, pt, 0, p.n + p.chunk_pages)
    st.select(q)
    torch.cuda.synchronize()
    orep = ora.rep(p, x["k_pool"], x["page_table"], 0, p.n + p.chunk_pages)
    oscores = ora.scores(p, ora.qmean(p, x["q"]), orep[: p.n])
    gscores = st.scores[:, : p.n].cpu().numpy()
    assert np.max(np.abs(gscores - oscores)) <= 1e-5 * max(1.0, float(np.max(np.abs(oscores))))
    check_selection(st.sel[:, : p.keff].cpu().numpy(), oscores, p.keff)


def test_rep_update_range_only(ora):
    """oomb_rep_update writes exactly rows [first, first + count) of the rep table."""
    seed, p = SMALL["qwen-ps128"]
    x = synth.make_inputs(p, seed)
    d = H.Device(p, x)
    st = H.make_step(p)
    st.rep.fill_(7.0)
    first, count = p.n - 3, 3 + p.chunk_pages
    st.rep_update(d.k, d.pt, first, count)
    torch.cuda.synchronize()
    rep = st.rep.cpu().numpy()
    assert np.all(rep[:first] == 7.0)
    want = ora.rep(p, x["k_pool"], x["page_table"], first, count)
    assert np.max(np.abs(rep[first:first + count] - want)) <= 1e-5


def test_bwd_accumulates(ora):
    """Two backward calls add twice the gradient to the pools (in-place accumulation)."""
    seed, p = SMALL["qwen-ps128"]
    x = synth.make_inputs(p, seed)
    d = H.Device(p, x)
    st = H.make_step(p)
    st.rep_update(d.k, d.pt, 0, p.n + p.chunk_pages)
    st.select(d.q)
    st.fwd(d.q, d.k, d.v, d.pt)
    st.bwd(d.q, d.k, d.v, d.pt, d.do, d.dk, d.dv)
    once_k, once_v = d.dk.clone() - 0.5, d.dv.clone() + 0.25
    st.bwd(d.q, d.k, d.v, d.pt, d.do, d.dk, d.dv)
    torch.cuda.synchronize()
    twice_k, twice_v = d.dk - 0.5, d.dv + 0.25
    assert torch.allclose(twice_k, 2 * once_k, atol=1e-6, rtol=1e-5)
    assert torch.allclose(twice_v, 2 * once_v, atol=1e-6, rtol=1e-5)
