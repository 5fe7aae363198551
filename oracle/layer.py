"""fp64 CPU reference of a decoder layer around the paged top-K attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite may import this
module.  It shares no code with the HIP library or its Python package and
never imports them.

What it computes: a Qwen2-style decoder block (RMSNorm, QKV projections with
bias, rotary positions with the rotate-half pairing, output projection,
RMSNorm, SwiGLU MLP, two residual adds) over a whole sequence, whose attention
is the chunk-recurrent paged top-K attention of the page "Out of the Memory
Barrier" (OOMB), technical summary, section 2: token t of chunk i attends to
the keys of the pages chosen for chunk i and its kv-head, and causally to the
tokens of its own chunk.  The page selection follows the same readings as the
attention oracle: one set per (chunk, kv-head), score = (mean query of the
chunk over its tokens and the group's query heads) . (mean key of the page),
the K best by (score desc, page asc), among the pages of earlier chunks.

Every step is written for the whole sequence at once in fp64 with plain torch
operations, and the backward pass is torch's autograd of that forward (pinned
against finite differences in the tests), so there is no chunking, paging or
recomputation in here to get wrong.  Inputs are the bf16 values the device
sees, widened exactly.
"""
from __future__ import annotations

import numpy as np
import torch

NAMES = ("ln1", "wq", "bq", "wk", "bk", "wv", "bv", "wo", "ln2", "wg", "wu", "wd")


def widen(bits: np.ndarray) -> torch.Tensor:
    """bf16 bits (uint16) -> fp64 tensor with the same values."""
    return torch.from_numpy((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def rms_norm(x, gain, eps):
    return x * torch.rsqrt((x * x).mean(dim=-1, keepdim=True) + eps) * gain


def rotary(x, theta):
    """x [T][heads][D]: pair (j, j + D/2) of token t is rotated by the angle
    t * theta^(-2j/D)."""
    t_len, _, d = x.shape
    half = d // 2
    freq = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    ang = torch.arange(t_len, dtype=torch.float64)[:, None] * freq[None, :]
    c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def project(s, w, x):
    """q [T][Hq][D], k, v [T][Hkv][D] of the layer input x [T][hidden]."""
    h = rms_norm(x, w["ln1"], s.eps)
    t_len = x.shape[0]
    q = (h @ w["wq"] + w["bq"]).reshape(t_len, s.hq, s.d)
    k = (h @ w["wk"] + w["bk"]).reshape(t_len, s.hkv, s.d)
    v = (h @ w["wv"] + w["bv"]).reshape(t_len, s.hkv, s.d)
    return rotary(q, s.rope_theta), rotary(k, s.rope_theta), v


def select(s, q, k):
    """Per chunk i, per kv-head: the K_eff = min(K, i*C/ps) best earlier pages,
    ascending, with their scores; q, k as from project (fp64)."""
    g = s.hq // s.hkv
    cp = s.c // s.ps
    rep = k.detach().reshape(s.chunks * cp, s.ps, s.hkv, s.d).mean(dim=1)  # [pages][Hkv][D]
    sels, scores = [], []
    for i in range(s.chunks):
        n = i * cp
        keff = min(s.k, n)
        qc = q.detach()[i * s.c:(i + 1) * s.c].reshape(s.c, s.hkv, g, s.d)
        qbar = qc.mean(dim=(0, 2))  # [Hkv][D]
        sc = torch.einsum("hd,phd->hp", qbar, rep[:n])  # [Hkv][n]
        sel = np.zeros((s.hkv, keff), dtype=np.int64)
        for h in range(s.hkv):
            order = sorted(range(n), key=lambda p: (-float(sc[h, p]), p))
            sel[h] = np.sort(order[:keff])
        sels.append(sel)
        scores.append(sc.numpy())
    return sels, scores


def mask(s, sels):
    """allowed [Hkv][T][T]: token t (chunk i) sees the tokens of pages
    sels[i][h] and the tokens u <= t of chunk i."""
    t_len = s.chunks * s.c
    m = torch.zeros((s.hkv, t_len, t_len), dtype=torch.bool)
    idx = torch.arange(s.c)
    for i in range(s.chunks):
        rows = slice(i * s.c, (i + 1) * s.c)
        m[:, rows, rows] = idx[None, :, None] >= idx[None, None, :]
        for h in range(s.hkv):
            for p in sels[i][h]:
                m[h, rows, p * s.ps:(p + 1) * s.ps] = True
    return m


def layer_forward(s, w, x, sels):
    """y [T][hidden] of the layer, with the given selections."""
    q, k, v = project(s, w, x)
    g = s.hq // s.hkv
    allowed = mask(s, sels)
    scale = 1.0 / np.sqrt(s.d)
    outs = []
    for head in range(s.hq):
        h = head // g
        sc = (q[:, head, :] @ k[:, h, :].T) * scale
        sc = sc.masked_fill(~allowed[h], float("-inf"))
        outs.append(torch.softmax(sc, dim=-1) @ v[:, h, :])
    o = torch.stack(outs, dim=1).reshape(x.shape[0], s.hq * s.d)
    x1 = x + o @ w["wo"]
    h2 = rms_norm(x1, w["ln2"], s.eps)
    gate = h2 @ w["wg"]
    return x1 + (gate * torch.sigmoid(gate) * (h2 @ w["wu"])) @ w["wd"]


def run(s, bits: dict, sels=None) -> dict:
    """The layer's forward and backward on the widened bf16 inputs of
    synth.make_layer_inputs.  sels: the selections to attend with (default:
    this reference's own).  Returns y, dx, the weight gradients, and the
    reference's own selections and page scores."""
    w = {n: widen(bits[n]).requires_grad_(True) for n in NAMES}
    x = widen(bits["x"]).requires_grad_(True)
    dy = widen(bits["dy"])
    with torch.no_grad():
        q, k, _ = project(s, w, x)
    own, scores = select(s, q, k)
    y = layer_forward(s, w, x, own if sels is None else sels)
    y.backward(dy)
    return {"y": y.detach().numpy(), "dx": x.grad.numpy(), "grads": {n: w[n].grad.numpy() for n in NAMES},
            "sel": own, "scores": scores}
