"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch.
They use closed forms, special cases that reduce to textbook attention
(written here as a masked dense softmax over the whole logical sequence, in
numpy, or differentiated by torch autograd in fp64), brute-force sorting,
central finite differences and invariants of softmax attention.  The method
is the OOMB page's ("Out of the Memory Barrier", technical summary, section 2:
paged KV cache and gradients, top-K pages by representative vectors reused in
the backward pass); the readings are those stated in the oracle's source.

``tests/test_oracle_pins.py`` runs every pin; ``tests/test_oracle_mutants.py``
plants plausible mistakes in copies of the oracle and checks that some pin
catches each one.
"""
from __future__ import annotations

import math

import numpy as np

import synth
from synth import Problem


def tiny(seed=11, **kw):
    base = dict(hq=2, hkv=1, d=8, ps=4, c=8, n=6, k=3, dtype="f64")
    base.update(kw)
    p = Problem(**base)
    return p, synth.make_inputs(p, seed)


def scale_of(p):
    return p.scale if p.scale > 0 else 1.0 / math.sqrt(p.d)


def logical_seq(p, pool, pt):
    """[hkv][(n + C/ps) * ps][d] in logical token order: logical page m is pool slot pt[m]."""
    m = p.n + p.chunk_pages
    return np.asarray(pool)[np.asarray(pt)[:m]].transpose(1, 0, 2, 3).reshape(p.hkv, m * p.ps, p.d)


def visibility(p, sel):
    """[hkv][C][P + C] mask: prior token j is visible iff its page is selected for
    the kv-head; chunk token u is visible to chunk token t iff u <= t."""
    P = p.n * p.ps
    vis = np.zeros((p.hkv, p.c, P + p.c), dtype=bool)
    t = np.arange(p.c)[:, None]
    u = np.arange(p.c)[None, :]
    for h in range(p.hkv):
        pages = np.zeros(p.n, dtype=bool)
        pages[np.asarray(sel[h], dtype=np.int64)] = True
        vis[h, :, :P] = np.repeat(pages, p.ps)[None, :]
        vis[h, :, P:] = u <= t
    return vis


def masked_attention(p, q, kseq, vseq, vis):
    """Textbook softmax attention with a boolean mask, fp64.  O [C][Hq][D], LSE [Hq][C]."""
    G = p.hq // p.hkv
    sc = scale_of(p)
    O = np.zeros((p.c, p.hq, p.d))
    L = np.zeros((p.hq, p.c))
    for g in range(p.hq):
        h = g // G
        S = sc * q[:, g, :] @ kseq[h].T
        S = np.where(vis[h], S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
        O[:, g, :] = np.exp(S - lse[:, None]) @ vseq[h]
        L[g] = lse
    return O, L


def rows_to_grid(p, a):
    """Oracle per-row output [C*Hq][...] -> [C][Hq][...]."""
    return a.reshape((p.c, p.hq) + a.shape[1:])


def torch_masked_grads(p, x, sel):
    """dQ, dK_seq, dV_seq of L = sum(dO * O) for the masked attention, by torch autograd, fp64 CPU."""
    import torch
    pt = x["page_table"]
    q = torch.tensor(np.asarray(x["q"], dtype=np.float64), requires_grad=True)
    ks = torch.tensor(logical_seq(p, x["k_pool"], pt), requires_grad=True)
    vs = torch.tensor(logical_seq(p, x["v_pool"], pt), requires_grad=True)
    dout = torch.tensor(np.asarray(x["do"], dtype=np.float64))
    vis = torch.tensor(visibility(p, sel))
    G = p.hq // p.hkv
    sc = scale_of(p)
    outs = []
    for g in range(p.hq):
        h = g // G
        S = sc * q[:, g, :] @ ks[h].T
        S = S.masked_fill(~vis[h], float("-inf"))
        outs.append(torch.softmax(S, dim=1) @ vs[h])
    O = torch.stack(outs, dim=1)
    (O * dout).sum().backward()
    return q.grad.numpy(), ks.grad.numpy(), vs.grad.numpy()


def key_grads_to_seq(p, sel, dk):
    """Oracle dk [hkv][nkeys][d] -> [hkv][P + C][d] in logical token order."""
    keff = p.keff
    P = p.n * p.ps
    out = np.zeros((p.hkv, P + p.c, p.d))
    for h in range(p.hkv):
        for i, page in enumerate(np.asarray(sel[h], dtype=np.int64)):
            out[h, page * p.ps:(page + 1) * p.ps] = dk[h, i * p.ps:(i + 1) * p.ps]
        out[h, P:] = dk[h, keff * p.ps:]
    return out


def close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * ref, f"{what}: max err {err:.3e} > {tol:.1e} * {ref:.3g}"


# ---------------------------------------------------------------------------
# representative vectors
# ---------------------------------------------------------------------------
def pin_rep_constant_page(ora):
    """A page whose ps keys are one vector has that vector as its representative."""
    p, x = tiny()
    kp = x["k_pool"].copy()
    pt = x["page_table"]
    for n in range(p.n):
        kp[pt[n]] = kp[pt[n], :, :1, :]          # every row := row 0
    rep = ora.rep(p, kp, pt)
    close(rep, np.stack([kp[pt[n], :, 0, :] for n in range(p.n)]), 1e-15, "rep(const page)")


def pin_rep_ramp(ora):
    """Keys r*e + b for r = 0..ps-1 have mean (ps-1)/2 * e + b."""
    p, x = tiny(ps=8)
    kp = x["k_pool"].copy()
    pt = x["page_table"]
    e = np.linspace(-1.0, 2.0, p.d)
    b = np.arange(p.d, dtype=np.float64) * 0.25
    for n in range(p.n):
        for h in range(p.hkv):
            kp[pt[n], h] = np.arange(p.ps)[:, None] * e[None, :] + b[None, :] + n
    rep = ora.rep(p, kp, pt)
    want = np.stack([[(p.ps - 1) / 2 * e + b + n for _ in range(p.hkv)] for n in range(p.n)])
    close(rep, want, 1e-14, "rep(ramp)")


def pin_rep_bruteforce(ora):
    """Representative vectors equal numpy's mean over the page's rows, for a
    bf16 pool with extra unmapped slots and two kv-heads; also for a page range."""
    p = Problem(hq=4, hkv=2, d=16, ps=8, c=16, n=9, k=4, dtype="bf16", n_slots=15)
    x = synth.make_inputs(p, 5)
    kseq = logical_seq(p, synth.as_float(x["k_pool"], "bf16"), x["page_table"])
    want = kseq.reshape(p.hkv, p.n + p.chunk_pages, p.ps, p.d).mean(axis=2).transpose(1, 0, 2)
    close(ora.rep(p, x["k_pool"], x["page_table"]), want[:p.n], 1e-12, "rep(bf16)")
    close(ora.rep(p, x["k_pool"], x["page_table"], first=p.n, count=p.chunk_pages),
          want[p.n:], 1e-12, "rep(chunk pages)")


def pin_rep_slot_permutation(ora):
    """Moving pages to other physical slots (and updating the table) changes nothing."""
    p, x = tiny(n_slots=12)
    pt = x["page_table"]
    rep0 = ora.rep(p, x["k_pool"], pt)
    perm = np.random.default_rng(3).permutation(p.slots)
    kp2 = np.empty_like(x["k_pool"])
    kp2[perm] = x["k_pool"]                       # slot s moves to perm[s]
    close(ora.rep(p, kp2, perm[pt].astype(np.int32)), rep0, 0.0, "rep(permuted slots)")


# ---------------------------------------------------------------------------
# chunk-mean query, scores, top-K
# ---------------------------------------------------------------------------
def pin_score_identity(ora):
    """score(n, h) equals the mean over chunk tokens t and group heads g of the
    per-row dot products q[t][g] . rep[n][h] (linearity of the mean)."""
    p, x = tiny(hq=6, hkv=2, n=10, c=12)
    rep = ora.rep(p, x["k_pool"], x["page_table"])
    sc = ora.scores(p, ora.qmean(p, x["q"]), rep)
    G = p.hq // p.hkv
    want = np.zeros((p.hkv, p.n))
    for h in range(p.hkv):
        rows = [x["q"][t, g] for t in range(p.c) for g in range(h * G, (h + 1) * G)]
        want[h] = np.mean([[r @ rep[n, h] for n in range(p.n)] for r in rows], axis=0)
    close(sc, want, 1e-13, "scores")


def pin_select_bruteforce(ora):
    """Top-K equals a full sort by (score desc, page asc), written ascending,
    for random scores with planted exact ties, K < N, K = N, K > N and K = 0."""
    rng = np.random.default_rng(7)
    for n, k in [(40, 7), (40, 1), (40, 40), (17, 30), (25, 0), (64, 63)]:
        p = Problem(hq=3, hkv=3, d=4, ps=4, c=4, n=n, k=k, dtype="f64")
        sc = np.round(rng.normal(size=(p.hkv, n)) * 4) / 4     # many exact ties
        got = ora.select(p, sc)
        keff = min(k, n)
        assert got.shape == (p.hkv, keff)
        for h in range(p.hkv):
            order = sorted(range(n), key=lambda m: (-sc[h, m], m))
            assert list(got[h]) == sorted(order[:keff]), (n, k, h)


def pin_select_duplicates(ora):
    """Pages planted as exact duplicates resolve to the lower page index."""
    p = Problem(hq=1, hkv=1, d=4, ps=4, c=4, n=8, k=2, dtype="f64")
    sc = np.array([[0.0, 5.0, 1.0, 5.0, 3.0, 5.0, -1.0, 2.0]])
    assert list(ora.select(p, sc)[0]) == [1, 3]
    sc = np.array([[9.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0]])
    assert list(ora.select(p, sc)[0]) == [0, 1]


def pin_selection_end_to_end(ora):
    """rep -> mean query -> scores -> top-K against numpy on a bf16 problem."""
    p = Problem(hq=4, hkv=2, d=16, ps=8, c=16, n=20, k=5, dtype="bf16")
    x = synth.make_inputs(p, 9)
    kseq = logical_seq(p, synth.as_float(x["k_pool"], "bf16"), x["page_table"])
    rep = kseq[:, : p.n * p.ps].reshape(p.hkv, p.n, p.ps, p.d).mean(axis=2)
    q = synth.as_float(x["q"], "bf16").reshape(p.c, p.hkv, p.group, p.d)
    qbar = q.mean(axis=(0, 2))
    sc = np.einsum("hd,hnd->hn", qbar, rep)
    sel, sco = ora.selection(p, x["q"], x["k_pool"], x["page_table"])
    close(sco, sc, 1e-12, "scores(bf16)")
    for h in range(p.hkv):
        assert list(sel[h]) == sorted(np.argsort(-sc[h], kind="stable")[: p.k]), h


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
def _fwd_vs_masked(ora, p, x, sel, tol):
    o, lse = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel)
    pt = x["page_table"]
    kseq = logical_seq(p, synth.as_float(x["k_pool"], p.dtype), pt)
    vseq = logical_seq(p, synth.as_float(x["v_pool"], p.dtype), pt)
    O, L = masked_attention(p, synth.as_float(x["q"], p.dtype), kseq, vseq, visibility(p, sel))
    close(rows_to_grid(p, o), O, tol, "O")
    close(rows_to_grid(p, lse).T, L, tol, "LSE")


def pin_fwd_dense_textbook(ora):
    """With K >= N every prior page is attended: the result is textbook dense
    causal attention over the whole sequence (prior tokens, then the chunk)."""
    p, x = tiny(k=6, hq=4, hkv=2, n_slots=11)
    _fwd_vs_masked(ora, p, x, np.tile(np.arange(p.n, dtype=np.int32), (p.hkv, 1)), 1e-12)


def pin_fwd_sparse_masked(ora):
    """With K < N the result is softmax attention restricted to the selected pages
    plus the causal chunk (same masked dense formulation), for an arbitrary selection."""
    p, x = tiny(hq=6, hkv=3, n=9, k=4, ps=4, c=12, d=8)
    sel = np.array([[0, 2, 5, 8], [1, 3, 4, 7], [2, 3, 6, 8]], dtype=np.int32)
    _fwd_vs_masked(ora, p, x, sel, 1e-12)


def pin_fwd_bf16_widening(ora):
    """bf16 and fp32 inputs are the exact widened values: same result as fp64
    storage of those values."""
    for dt in ("bf16", "f32"):
        p = Problem(hq=4, hkv=2, d=8, ps=4, c=8, n=5, k=2, dtype=dt)
        x = synth.make_inputs(p, 2)
        sel = np.array([[0, 3], [1, 4]], dtype=np.int32)
        o, lse = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel)
        p64 = Problem(hq=4, hkv=2, d=8, ps=4, c=8, n=5, k=2, dtype="f64")
        o2, lse2 = ora.fwd(p64, *(synth.as_float(x[a], dt) for a in ("q", "k_pool", "v_pool")),
                           x["page_table"], sel)
        close(o, o2, 0.0, "O(%s)" % dt)
        close(lse, lse2, 0.0, "LSE(%s)" % dt)
        _fwd_vs_masked(ora, p, x, sel, 1e-12)


def pin_fwd_rows_sum_to_one(ora):
    """Softmax weights of every row sum to 1: with every value vector = 1, O = 1."""
    p, x = tiny(hq=4, hkv=2, n=7, k=3)
    vp = np.ones_like(x["v_pool"])
    sel = np.array([[0, 3, 6], [1, 2, 5]], dtype=np.int32)
    o, _ = ora.fwd(p, x["q"], x["k_pool"], vp, x["page_table"], sel)
    close(o, np.ones_like(o), 1e-14, "sum p")


def pin_fwd_zero_query(ora):
    """Q = 0 gives uniform weights: O = mean of the visible values, LSE = ln |J|."""
    p, x = tiny(hq=2, hkv=1, n=6, k=2, c=8)
    sel = np.array([[1, 4]], dtype=np.int32)
    q0 = np.zeros_like(x["q"])
    o, lse = ora.fwd(p, q0, x["k_pool"], x["v_pool"], x["page_table"], sel)
    vseq = logical_seq(p, x["v_pool"], x["page_table"])
    P = p.n * p.ps
    prior = np.concatenate([vseq[0, s * p.ps:(s + 1) * p.ps] for s in (1, 4)])
    for t in range(p.c):
        vis = np.concatenate([prior, vseq[0, P:P + t + 1]])
        for g in range(p.hq):
            close(o[t * p.hq + g], vis.mean(axis=0), 1e-14, "O(q=0)")
            close(lse[t * p.hq + g], math.log(len(vis)), 1e-14, "LSE(q=0)")


def pin_fwd_single_key(ora):
    """No prior pages (K = 0): chunk token 0 sees only itself, O = v_0, LSE = s_0."""
    p, x = tiny(k=0)
    o, lse = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], np.zeros((1, 0), np.int32),
                     rows=np.arange(p.hq))
    slot = x["page_table"][p.n]
    for g in range(p.hq):
        k0 = x["k_pool"][slot, 0, 0]
        close(o[g], x["v_pool"][slot, 0, 0], 1e-15, "O(single key)")
        close(lse[g], scale_of(p) * x["q"][0, g] @ k0, 1e-14, "LSE(single key)")


def pin_fwd_two_key_closed_form(ora):
    """Hand-worked case: D = 2, one prior page of one token, chunk of one token.
    q = (1, 0), prior key (sqrt(2) ln 2, 0), own key 0, scale 1/sqrt(2):
    scores ln 2 and 0, weights 2/3 and 1/3, LSE = ln 3, O = (2 v_prior + v_own) / 3."""
    p = Problem(hq=1, hkv=1, d=2, ps=1, c=1, n=1, k=1, dtype="f64")
    q = np.array([[[1.0, 0.0]]])
    kp = np.zeros((2, 1, 1, 2))
    vp = np.zeros((2, 1, 1, 2))
    pt = np.array([1, 0], dtype=np.int32)          # prior page in slot 1, chunk page in slot 0
    kp[1, 0, 0] = [math.sqrt(2) * math.log(2), 0.0]
    vp[1, 0, 0] = [3.0, -6.0]
    vp[0, 0, 0] = [0.0, 3.0]
    o, lse = ora.fwd(p, q, kp, vp, pt, np.array([[0]], dtype=np.int32))
    close(lse, [math.log(3.0)], 1e-15, "LSE(closed form)")
    close(o, [[2.0, -3.0]], 1e-14, "O(closed form)")


def pin_fwd_lse_bounds(ora):
    """max_j s_j <= LSE <= max_j s_j + ln |J| for every row."""
    p, x = tiny(hq=4, hkv=2, n=8, k=3, c=8)
    sel = np.array([[0, 1, 7], [2, 5, 6]], dtype=np.int32)
    _, lse = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel)
    kseq = logical_seq(p, x["k_pool"], x["page_table"])
    vis = visibility(p, sel)
    for t in range(p.c):
        for g in range(p.hq):
            h = g // p.group
            s = scale_of(p) * kseq[h][vis[h, t]] @ x["q"][t, g]
            L = lse[t * p.hq + g]
            assert s.max() - 1e-13 <= L <= s.max() + math.log(len(s)) + 1e-13


def pin_scale_override(ora):
    """A given softmax scale s equals the default scale with Q multiplied by s * sqrt(D)."""
    p, x = tiny(scale=0.3)
    p0 = Problem(**{**p.__dict__, "scale": 0.0})
    sel = np.array([[0, 2, 4]], dtype=np.int32)
    o1, l1 = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel)
    o2, l2 = ora.fwd(p0, x["q"] * (0.3 * math.sqrt(p.d)), x["k_pool"], x["v_pool"], x["page_table"], sel)
    close(o1, o2, 1e-13, "O(scale)")
    close(l1, l2, 1e-13, "LSE(scale)")


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def _pool_grads(ora, p, x, sel, dk, dv):
    """Oracle dk/dv per key of J(h) -> pool-shaped arrays."""
    slot, row = ora.key_slots(p, x["page_table"], sel)
    gk = np.zeros(x["k_pool"].shape)
    gv = np.zeros(x["v_pool"].shape)
    for h in range(p.hkv):
        gk[slot[h], h, row[h]] += dk[h]
        gv[slot[h], h, row[h]] += dv[h]
    return gk, gv


def pin_bwd_finite_differences(ora):
    """dQ, dK, dV equal central differences of L = sum(dO * O) with the selection
    held fixed, for every element of Q and of the K and V pools (unmapped and
    unselected slots included: their gradient is 0)."""
    p, x = tiny(hq=2, hkv=1, d=8, ps=4, c=8, n=6, k=3, n_slots=10)
    sel = np.array([[0, 2, 5]], dtype=np.int32)
    pt, dout = x["page_table"], x["do"]

    def loss(q, kp, vp):
        o, _ = ora.fwd(p, q, kp, vp, pt, sel)
        return float(np.sum(rows_to_grid(p, o) * dout))

    dq, dk, dv = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], pt, sel, dout)
    gk, gv = _pool_grads(ora, p, x, sel, dk, dv)
    h = 1e-6
    for name, grad in (("q", rows_to_grid(p, dq)), ("k_pool", gk), ("v_pool", gv)):
        base = x[name]
        fd = np.zeros(base.shape)
        for i in range(base.size):
            plus, minus = base.copy(), base.copy()
            plus.flat[i] += h
            minus.flat[i] -= h
            args = {a: x[a] for a in ("q", "k_pool", "v_pool")}
            args[name] = plus
            lp = loss(args["q"], args["k_pool"], args["v_pool"])
            args[name] = minus
            lm = loss(args["q"], args["k_pool"], args["v_pool"])
            fd.flat[i] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - grad))
        assert err <= 1e-7 * max(1.0, np.max(np.abs(grad))), f"FD {name}: {err:.3e}"


def _bwd_vs_autograd(ora, p, x, sel, tol):
    dq, dk, dv = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"])
    tq, tk, tv = torch_masked_grads(p, x, sel)
    close(rows_to_grid(p, dq), tq, tol, "dQ")
    gk, gv = key_grads_to_seq(p, sel, dk), key_grads_to_seq(p, sel, dv)
    close(gk, tk, tol, "dK")
    close(gv, tv, tol, "dV")


def pin_bwd_dense_autograd(ora):
    """K >= N: gradients equal torch autograd (fp64, CPU) of dense causal attention."""
    p, x = tiny(hq=4, hkv=2, n=5, k=9, c=8)
    _bwd_vs_autograd(ora, p, x, np.tile(np.arange(p.n, dtype=np.int32), (p.hkv, 1)), 1e-12)


def pin_bwd_sparse_autograd(ora):
    """K < N: gradients equal torch autograd of the masked formulation; unselected
    prior tokens get exactly zero gradient."""
    p, x = tiny(hq=6, hkv=2, n=9, k=3, c=12, ps=4)
    sel = np.array([[0, 4, 8], [2, 3, 7]], dtype=np.int32)
    _bwd_vs_autograd(ora, p, x, sel, 1e-12)


def pin_bwd_invariants(ora):
    """Per kv-head: sum over keys of dK is 0 (softmax is shift-invariant in the
    scores), and sum over keys of dV equals the sum of dO over the head's rows."""
    p, x = tiny(hq=6, hkv=2, n=10, k=4, c=16, ps=4, d=16)
    sel, _ = ora.selection(p, x["q"], x["k_pool"], x["page_table"])
    _, dk, dv = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"])
    G = p.group
    for h in range(p.hkv):
        close(dk[h].sum(axis=0), np.zeros(p.d), 1e-12, "sum dK")
        close(dv[h].sum(axis=0), x["do"][:, h * G:(h + 1) * G].sum(axis=(0, 1)), 1e-12, "sum dV")


def pin_bwd_constant_values(ora):
    """Every value vector of a kv-head equal to one vector v_h: each row's
    output is v_h whatever the weights, so dO . V_j equals Dt = dO . O for
    every visible key j, every dS is zero, and with it dQ and dK; dV_j is then
    the sum over rows of P_rj dO_r, whose sum over keys is the sum of dO."""
    p, x = tiny(hq=4, hkv=2, n=8, k=3, c=8, ps=4, d=8)
    rng = np.random.default_rng(5)
    vh = rng.normal(size=(p.hkv, p.d))
    v = np.empty_like(x["v_pool"])
    for h in range(p.hkv):
        v[:, h] = vh[h]
    sel, _ = ora.selection(p, x["q"], x["k_pool"], x["page_table"])
    o, _ = ora.fwd(p, x["q"], x["k_pool"], v, x["page_table"], sel)
    G = p.group
    want_o = np.stack([vh[g // G] for _ in range(p.c) for g in range(p.hq)])
    close(o, want_o, 1e-13, "O = v")
    dq, dk, dv = ora.bwd(p, x["q"], x["k_pool"], v, x["page_table"], sel, x["do"])
    close(dq, np.zeros_like(dq), 1e-13, "dQ = 0")
    close(dk, np.zeros_like(dk), 1e-13, "dK = 0")
    for h in range(p.hkv):
        close(dv[h].sum(axis=0), x["do"][:, h * G:(h + 1) * G].sum(axis=(0, 1)), 1e-12, "sum dV")


def pin_bwd_linearity(ora):
    """Gradients are linear in dO."""
    p, x = tiny(hq=4, hkv=2, n=6, k=2)
    sel = np.array([[0, 5], [2, 3]], dtype=np.int32)
    a = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"])
    b = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, -2.5 * x["do"])
    for u, v, nm in zip(a, b, ("dq", "dk", "dv")):
        close(v, -2.5 * u, 1e-13, nm)


def pin_bwd_row_additivity(ora):
    """Driving the backward with rows A and B separately sums to driving it with
    A and B together, and dq of a row does not depend on the other rows."""
    p, x = tiny(hq=4, hkv=2, n=6, k=2, c=8)
    sel = np.array([[1, 4], [0, 3]], dtype=np.int32)
    rows = np.arange(p.c * p.hq)
    A, B = rows[::3], np.setdiff1d(rows, rows[::3])
    args = (p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"])
    qa, ka, va = ora.bwd(*args, rows=A)
    qb, kb, vb = ora.bwd(*args, rows=B)
    q, k, v = ora.bwd(*args)
    close(ka + kb, k, 1e-13, "dk additivity")
    close(va + vb, v, 1e-13, "dv additivity")
    close(qa, q[A], 0.0, "dq rows")
    close(qb, q[B], 0.0, "dq rows")


def _seq(**kw):
    base = dict(hq=4, hkv=2, d=16, ps=4, c=8, chunks=3, k=3, n0=2, dtype="f64")
    base.update(kw)
    return synth.Sequence(**base)


def pin_sequence_dense_equals_one_long_chunk(ora):
    """With every earlier page selected, chunk-recurrent attention over a
    sequence is causal attention over the whole sequence: the same as one
    chunk step whose chunk is all the chunks' tokens (its own prior pages being
    the initial context).  Forward and backward, pool by pool."""
    s = _seq(k=1000)
    x = synth.make_sequence_inputs(s, 41)
    r = ora.sequence(s, x)
    big = Problem(hq=s.hq, hkv=s.hkv, d=s.d, ps=s.ps, c=s.chunks * s.c, n=s.n0, k=1000, dtype=s.dtype,
                  n_slots=s.pages)
    q = x["q"].reshape(s.chunks * s.c, s.hq, s.d)
    do = x["do"].reshape(s.chunks * s.c, s.hq, s.d)
    sel = np.tile(np.arange(s.n0, dtype=np.int32), (s.hkv, 1))
    o, lse = ora.fwd(big, q, x["k_pool"], x["v_pool"], x["page_table"], sel)
    dq, dk, dv = ora.bwd(big, q, x["k_pool"], x["v_pool"], x["page_table"], sel, do)
    rows = s.c * s.hq
    for i in range(s.chunks):
        close(r["o"][i], o[i * rows:(i + 1) * rows], 1e-12, f"O chunk {i}")
        close(r["lse"][i], lse[i * rows:(i + 1) * rows], 1e-12, f"LSE chunk {i}")
        close(r["dq"][i], dq[i * rows:(i + 1) * rows], 1e-12, f"dQ chunk {i}")
    dkp, dvp = _pool_grads(ora, big, x, sel, dk, dv)
    close(r["dk"], dkp, 1e-12, "dK pool")
    close(r["dv"], dvp, 1e-12, "dV pool")


def pin_sequence_selection_by_chunk(ora):
    """Chunk i picks among exactly the pages before it (initial context and
    chunks 0 .. i-1): its pages are numpy's top-K of (the chunk's mean query
    over tokens and group heads) . (page key means), ties to the lower page,
    listed ascending."""
    s = _seq(k=3, chunks=4, n0=2)
    x = synth.make_sequence_inputs(s, 42)
    r = ora.sequence(s, x)
    kseq = logical_seq(s.step(s.chunks - 1), x["k_pool"], x["page_table"])   # [hkv][pages*ps][d]
    page_mean = kseq.reshape(s.hkv, s.pages, s.ps, s.d).mean(axis=2)
    G = s.hq // s.hkv
    for i in range(s.chunks):
        n = s.n0 + i * s.c // s.ps
        keff = min(s.k, n)
        for h in range(s.hkv):
            qbar = x["q"][i][:, h * G:(h + 1) * G, :].mean(axis=(0, 1))
            sc = page_mean[h, :n] @ qbar
            order = sorted(range(n), key=lambda m: (-sc[m], m))[:keff]
            assert list(r["sel"][i][h]) == sorted(order), (i, h, r["sel"][i][h], sorted(order))


def pin_sequence_invariants(ora):
    """Over the whole sequence: per kv-head the dK contributions sum to zero
    (softmax shift invariance, chunk by chunk), and the dV contributions sum to
    the sum of dO over every chunk's tokens and the head's query group."""
    s = _seq(k=2, chunks=3, n0=3)
    x = synth.make_sequence_inputs(s, 43)
    r = ora.sequence(s, x)
    G = s.hq // s.hkv
    for h in range(s.hkv):
        close(r["dk"][:, h].sum(axis=(0, 1)), np.zeros(s.d), 1e-11, "sum dK")
        close(r["dv"][:, h].sum(axis=(0, 1)), x["do"][:, :, h * G:(h + 1) * G, :].sum(axis=(0, 1, 2)), 1e-11,
              "sum dV")


PINS = {name: fn for name, fn in globals().items() if name.startswith("pin_")}


def _golden_value(v):
    """A fixture entry: a number, or a closed form in sqrt, ln and rationals."""
    if isinstance(v, (int, float)):
        return float(v)
    return float(eval(v, {"__builtins__": {}}, {"sqrt": math.sqrt, "ln": math.log}))


def pin_golden_two_key_step(ora):
    """The hand-worked step in tests/golden/two_key_step.json: forward and backward."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "two_key_step.json")
    with open(path) as f:
        gd = json.load(f)
    vec = lambda name: np.array([_golden_value(v) for v in gd[name]])
    sh = gd["shape"]
    p = Problem(hq=sh["hq"], hkv=sh["hkv"], d=sh["d"], ps=sh["ps"], c=sh["c"], n=sh["n"], k=sh["k"], dtype="f64")
    pt = np.array(gd["page_table"], dtype=np.int32)
    sel = np.array(gd["sel"], dtype=np.int32)
    kp = np.zeros((2, 1, 1, 2))
    vp = np.zeros((2, 1, 1, 2))
    kp[pt[0], 0, 0], vp[pt[0], 0, 0] = vec("k_prior"), vec("v_prior")
    kp[pt[1], 0, 0], vp[pt[1], 0, 0] = vec("k_own"), vec("v_own")
    q = vec("q").reshape(1, 1, 2)
    do = vec("dO").reshape(1, 1, 2)
    ex = gd["expected"]
    o, lse = ora.fwd(p, q, kp, vp, pt, sel)
    close(lse, [_golden_value(ex["lse"])], 1e-15, "golden LSE")
    close(o[0], [_golden_value(v) for v in ex["o"]], 1e-14, "golden O")
    dq, dk, dv = ora.bwd(p, q, kp, vp, pt, sel, do)
    ev = lambda name: [_golden_value(v) for v in ex[name]]
    close(dq[0], ev("dq"), 1e-14, "golden dQ")
    close(dk[0, 0], ev("dk_prior"), 1e-14, "golden dK prior")
    close(dk[0, 1], ev("dk_own"), 1e-14, "golden dK own")
    close(dv[0, 0], ev("dv_prior"), 1e-14, "golden dV prior")
    close(dv[0, 1], ev("dv_own"), 1e-14, "golden dV own")


PINS["pin_golden_two_key_step"] = pin_golden_two_key_step
