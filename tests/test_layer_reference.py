"""Pins of the fp64 decoder-layer reference (oracle/layer.py), on the CPU.

Each pin checks the reference against something other than itself:
- its autograd backward against central finite differences (gradcheck);
- its paged top-K attention, with every earlier page selected, against
  torch's causal scaled-dot-product attention;
- its page selection against the C attention oracle's rep -> mean query ->
  scores -> top-K chain on the same fp64 keys and queries;
- the rotary positions against the closed form of one pair, (cos t, sin t),
  and two properties of a rotation by position: norms are kept, and q.k
  depends only on the distance of the positions;
- RMSNorm against its defining property (unit root-mean-square).
Planted in a copy of the reference, a flipped rotation sign, a causal mask
with u < t, and a chunk-mean query over one head of the group each fail at
least one of these.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import layer as R

TINY = synth.Layer(hidden=8, hq=2, hkv=1, d=4, inter=8, ps=2, c=4, chunks=3, k=1)
SMALL = synth.Layer(hidden=32, hq=4, hkv=2, d=8, inter=48, ps=2, c=8, chunks=4, k=2)


def weights(s, seed):
    bits = synth.make_layer_inputs(s, seed)
    return bits, {n: R.widen(bits[n]) for n in R.NAMES}, R.widen(bits["x"])


def test_backward_matches_finite_differences():
    s = TINY
    _, w, x = weights(s, 1)
    with torch.no_grad():
        q, k, _ = R.project(s, w, x)
    sels, _ = R.select(s, q, k)
    names = ("wq", "wk", "wv", "wo", "wg", "wd", "ln1", "ln2", "bq")

    def f(x_, *ws):
        ww = dict(w)
        ww.update(zip(names, ws))
        return R.layer_forward(s, ww, x_, sels)

    args = [x.clone().requires_grad_(True)] + [w[n].clone().requires_grad_(True) for n in names]
    assert torch.autograd.gradcheck(f, args, eps=1e-6, atol=1e-6, rtol=1e-5)


def test_dense_selection_is_causal_attention():
    s = SMALL
    _, w, x = weights(s, 2)
    cp = s.c // s.ps
    every = [np.tile(np.arange(i * cp), (s.hkv, 1)) for i in range(s.chunks)]
    y = R.layer_forward(s, w, x, every)
    q, k, v = R.project(s, w, x)
    g = s.hq // s.hkv
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.repeat_interleave(g, dim=1).transpose(0, 1),
                                       v.repeat_interleave(g, dim=1).transpose(0, 1), is_causal=True)
    o = o.transpose(0, 1).reshape(x.shape[0], s.hq * s.d)
    x1 = x + o @ w["wo"]
    h2 = R.rms_norm(x1, w["ln2"], s.eps)
    ref = x1 + (F.silu(h2 @ w["wg"]) * (h2 @ w["wu"])) @ w["wd"]
    assert torch.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_selection_matches_attention_oracle(ora):
    s = SMALL
    _, w, x = weights(s, 3)
    with torch.no_grad():
        q, k, _ = R.project(s, w, x)
    sels, scores = R.select(s, q, k)
    pages = s.chunks * (s.c // s.ps)
    pool = k.numpy().reshape(pages, s.ps, s.hkv, s.d).transpose(0, 2, 1, 3).copy()
    pt = np.arange(pages, dtype=np.int32)
    for i in range(1, s.chunks):
        p = synth.Problem(s.hq, s.hkv, s.d, s.ps, s.c, i * (s.c // s.ps), s.k, dtype="f64", n_slots=pages)
        qc = q.numpy()[i * s.c:(i + 1) * s.c].copy()
        sel, sc = ora.selection(p, qc, pool, pt, "f64")
        assert np.array_equal(sel, sels[i])
        assert np.allclose(sc, scores[i], rtol=1e-12, atol=1e-12)


def test_rotary_is_a_rotation_by_position():
    d, t_len = 8, 12
    gen = torch.Generator().manual_seed(0)
    qv, kv = torch.randn(d, generator=gen, dtype=torch.float64), torch.randn(d, generator=gen, dtype=torch.float64)
    q = R.rotary(qv.expand(t_len, 1, d).clone(), 1.0e4)[:, 0]
    k = R.rotary(kv.expand(t_len, 1, d).clone(), 1.0e4)[:, 0]
    assert torch.allclose(q.norm(dim=-1), qv.norm().expand(t_len), rtol=1e-13)
    for m, n, shift in ((5, 3, 4), (9, 2, 1), (3, 7, 2)):
        assert abs(float(q[m] @ k[n] - q[m + shift] @ k[n + shift])) < 1e-12
    assert torch.equal(q[0], qv)  # position 0 is not rotated


def test_rms_norm_has_unit_rms():
    x = torch.randn(5, 16, dtype=torch.float64, generator=torch.Generator().manual_seed(1)) * 3.0
    y = R.rms_norm(x, torch.ones(16, dtype=torch.float64), 0.0)
    assert torch.allclose((y * y).mean(dim=-1), torch.ones(5, dtype=torch.float64), rtol=1e-13)


def test_layer_inputs_are_seeded_and_shaped():
    s = synth.LAYERS["layer-tiny"][1]
    a = synth.make_layer_inputs(s, 11)
    b = synth.make_layer_inputs(s, 11)
    for n, (shape, _) in synth.layer_tensors(s).items():
        assert a[n].shape == shape and a[n].dtype == np.uint16
        assert np.array_equal(a[n], b[n])
    assert not np.array_equal(a["wq"], synth.make_layer_inputs(s, 12)["wq"])


def test_rotary_closed_form_of_one_pair():
    # one pair (D = 2): the frequency is 1 whatever theta, so (1, 0) at
    # position t becomes (cos t, sin t) and (0, 1) becomes (-sin t, cos t)
    t = torch.arange(7, dtype=torch.float64)
    e0 = torch.tensor([1.0, 0.0], dtype=torch.float64).expand(7, 1, 2).clone()
    e1 = torch.tensor([0.0, 1.0], dtype=torch.float64).expand(7, 1, 2).clone()
    assert torch.allclose(R.rotary(e0, 1.0e6)[:, 0], torch.stack([t.cos(), t.sin()], -1), atol=1e-15)
    assert torch.allclose(R.rotary(e1, 1.0e6)[:, 0], torch.stack([-t.sin(), t.cos()], -1), atol=1e-15)
