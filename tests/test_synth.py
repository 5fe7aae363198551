"""The seeded input generator: counter-based reproducibility, distribution,
single-step bf16 rounding, page-table permutation and pool placement."""
from fractions import Fraction
import math
import struct

import numpy as np

import synth
from synth import Problem


def bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def nearest_even_bf16(x):
    """Exact round-to-nearest-even of a float to bf16, by rational arithmetic."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    ax = Fraction(abs(x))
    e = math.floor(math.log2(abs(x)))
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    m = ax / ulp                       # in [128, 256)
    lo = math.floor(m)
    r = m - lo
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    val = float(lo * ulp)
    return sign | (struct.unpack("<I", struct.pack("<f", val))[0] >> 16)


def test_counter_based_chunks_agree():
    whole = synth.normals(7, 3, 10001)
    parts = np.concatenate([synth.normals(7, 3, 4000, 0), synth.normals(7, 3, 6001, 4000)])
    assert np.array_equal(whole, parts)
    assert not np.array_equal(whole[:100], synth.normals(8, 3, 100))
    assert not np.array_equal(whole[:100], synth.normals(7, 4, 100))


def test_normal_moments():
    x = synth.normals(1, 1, 400000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(np.mean(x ** 3)) < 0.03 and abs(np.mean(x ** 4) - 3) < 0.05


def test_bf16_rounding_exact():
    lib = synth.lib()
    vals = list(synth.normals(2, 9, 3000) * 7.3) + [1.0, -2.5, 3.0000001, 1 + 2 ** -8, 1 + 3 * 2 ** -8,
                                                     1 + 2 ** -8 + 2 ** -40, 255.5, 1e-30, -65504.0]
    for v in vals:
        assert lib.synth_round_bf16(float(v)) == nearest_even_bf16(float(v)), v


def test_problem_inputs_layout():
    p = Problem(hq=4, hkv=2, d=8, ps=4, c=8, n=5, k=2, dtype="bf16", n_slots=9)
    x = synth.make_inputs(p, 3)
    pt = x["page_table"]
    assert sorted(pt.tolist()) == sorted(set(pt.tolist())) and len(pt) == p.n + p.chunk_pages
    assert x["k_pool"].shape == (9, 2, 4, 8) and x["q"].shape == (8, 4, 8)
    # token (n, h, r, x) of K = N(0,1) draw + 0.5 * per-(page, head) offset, rounded once
    n, h, r, xx = 3, 1, 2, 5
    tok = synth.normals(3, synth.S_K, 1, ((n * p.hkv + h) * p.ps + r) * p.d + xx)[0]
    off = synth.normals(3, synth.S_KOFF, 1, (n * p.hkv + h) * p.d + xx)[0]
    assert x["k_pool"][pt[n], h, r, xx] == synth.lib().synth_round_bf16(tok + 0.5 * off)
    unmapped = sorted(set(range(9)) - set(pt.tolist()))
    assert all(bf16_value(b) == 64.0 for b in x["k_pool"][unmapped].ravel())


def test_sequence_inputs_cover_every_page():
    s = synth.Sequence(hq=4, hkv=2, d=16, ps=4, c=8, chunks=3, k=2, n0=2)
    x = synth.make_sequence_inputs(s, 9)
    assert x["q"].shape == (3, 8, 4, 16) and x["do"].shape == (3, 8, 4, 16)
    assert x["k_pool"].shape == (s.pages, 2, 4, 16)
    assert sorted(x["page_table"].tolist()) == list(range(s.pages))
    assert s.step(0).n == 2 and s.step(2).n == 2 + 2 * 2 and s.step(2).slots == s.pages
    y = synth.make_sequence_inputs(s, 9)
    assert all(np.array_equal(x[k], y[k]) for k in x)
