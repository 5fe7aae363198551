"""Run one chunk step through the C ABI on the GPU and check it against the
fp64 oracle (element by element on small problems; sampled rows, the last
chunk keys and invariants on full-size ones)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from parity import check_selection, compare, compare_lse


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return synth.widen_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def make_step(p):
    from paged_sparse_attention_amd.step import ChunkStep
    return ChunkStep(p.hq, p.hkv, p.d, p.ps, p.c, p.n, p.k, p.slots, dtype=p.dtype, softmax_scale=p.scale)


class Device:
    """The problem's inputs on the device."""

    def __init__(self, p, x, canary_seed=None):
        self.q = dev(x["q"], p.dtype)
        self.k = dev(x["k_pool"], p.dtype)
        self.v = dev(x["v_pool"], p.dtype)
        self.do = dev(x["do"], p.dtype)
        self.pt = dev(x["page_table"])
        if canary_seed is None:                       # constant prefill, checked on the device
            self.dk0 = self.dv0 = None
            self.dk = torch.full(tuple(x["k_pool"].shape), 0.5, dtype=torch.float32, device="cuda")
            self.dv = torch.full(tuple(x["k_pool"].shape), -0.25, dtype=torch.float32, device="cuda")
        else:                                         # seeded prefill, checked on the host
            self.dk0 = synth.canary(p, canary_seed, "k")
            self.dv0 = synth.canary(p, canary_seed, "v")
            self.dk = dev(self.dk0)
            self.dv = dev(self.dv0)


def touched_mask(p, ora, pt, sel):
    """[slots][hkv] bool: pool (slot, head) pairs that the backward may change."""
    slot, _ = ora.key_slots(p, pt, sel)
    m = np.zeros((p.slots, p.hkv), dtype=bool)
    for h in range(p.hkv):
        m[np.unique(slot[h]), h] = True
    return m


def run_full(p, seed, ora, report=None, rel_limits=None, tweak=None):
    """Every output against the oracle, element by element (small problems).
    rel_limits: {output name: r} replaces the official max-abs bar of that
    output by r * max |reference| (a documented known limit only).  tweak(x),
    if given, edits the generated inputs in place before both sides see them."""
    rel_limits = rel_limits or {}

    def bar(name, want):
        return rel_limits[name] * float(np.max(np.abs(want))) if name in rel_limits else None
    report = {} if report is None else report
    x = synth.make_inputs(p, seed)
    if tweak is not None:
        tweak(x)
    d = Device(p, x, canary_seed=seed)
    st = make_step(p)
    pages = p.n + p.chunk_pages
    st.rep_update(d.k, d.pt, 0, pages)
    st.select(d.q)
    st.fwd(d.q, d.k, d.v, d.pt)
    st.bwd(d.q, d.k, d.v, d.pt, d.do, d.dk, d.dv)
    torch.cuda.synchronize()

    rep = st.rep.cpu().numpy()
    orep = ora.rep(p, x["k_pool"], x["page_table"], 0, pages)
    err = float(np.max(np.abs(rep - orep))) if rep.size else 0.0
    report["rep"] = dict(max_abs=err)
    assert err <= 1e-5 * max(1.0, float(np.max(np.abs(orep))) if orep.size else 1.0), f"rep err {err:.3e}"

    keff = p.keff
    sel = st.sel[:, :keff].cpu().numpy() if keff else np.zeros((p.hkv, 0), np.int32)
    if p.n:
        qbar = ora.qmean(p, x["q"])
        oscores = ora.scores(p, qbar, orep[: p.n])
        gscores = st.scores[:, : p.n].cpu().numpy()
        serr = float(np.max(np.abs(gscores - oscores)))
        report["scores"] = dict(max_abs=serr)
        assert serr <= 1e-5 * max(1.0, float(np.max(np.abs(oscores)))), f"scores err {serr:.3e}"
        report["sel_exact"] = check_selection(sel, oscores, keff)

    oo, ol = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel)
    o = host(st.o).reshape(-1, p.d)
    lse = st.lse.cpu().numpy().T.reshape(-1)        # [Hq][C] -> row t*Hq + g
    compare("O", o, oo, p.dtype, report)
    compare_lse(lse, ol, p.dtype, report)

    odq, odk, odv = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"])
    compare("dQ", st.dq.cpu().numpy().reshape(-1, p.d), odq, p.dtype, report, max_abs=bar("dQ", odq))
    dk = d.dk.cpu().numpy()
    dv = d.dv.cpu().numpy()
    slot, row = ora.key_slots(p, x["page_table"], sel)
    gdk = np.stack([(dk[slot[h], h, row[h]].astype(np.float64) - d.dk0[slot[h], h, row[h]]) for h in range(p.hkv)])
    gdv = np.stack([(dv[slot[h], h, row[h]].astype(np.float64) - d.dv0[slot[h], h, row[h]]) for h in range(p.hkv)])
    compare("dK", gdk, odk, p.dtype, report, max_abs=bar("dK", odk))
    compare("dV", gdv, odv, p.dtype, report, max_abs=bar("dV", odv))
    untouched = ~touched_mask(p, ora, x["page_table"], sel)
    for name, after, before in (("dK", dk, d.dk0), ("dV", dv, d.dv0)):
        a = after[untouched]
        b = before[untouched]
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name}: an unselected slot changed"
    return report, st, d, x, sel


ROW_BLOCK = 256   # rows of a kv-head's C*G rows that one forward or dQ workgroup owns


def sample_rows(p, rng, n_extra=12, per_block=True):
    """Rows t*Hq + g covering the chunk's edges, page edges and every kv-head;
    with per_block, also one random row of every (row block, query head): the
    row blocks of kv-head h cover its rows t*G + gi (query head h*G + gi) in
    runs of ROW_BLOCK, and each workgroup writes one such run."""
    toks = {0, 1, p.ps - 1, min(p.ps, p.c - 1), p.c // 2, max(p.c - p.ps - 1, 0), max(p.c - 2, 0), p.c - 1}
    toks |= set(int(t) for t in rng.integers(0, p.c, n_extra))
    rows = []
    for i, t in enumerate(sorted(toks)):
        for g in {(i * 5) % p.hq, (i * 5 + p.group) % p.hq, p.hq - 1 - (i % p.hq)}:
            rows.append(t * p.hq + g)
    if per_block:
        G = p.group
        for b in range((p.c * G + ROW_BLOCK - 1) // ROW_BLOCK):
            r0, r1 = b * ROW_BLOCK, min((b + 1) * ROW_BLOCK, p.c * G) - 1
            for gi in range(G):
                lo, hi = -(-(r0 - gi) // G), (r1 - gi) // G   # tokens t with r0 <= t*G + gi <= r1
                if lo > hi:
                    continue
                t = int(lo + rng.integers(0, hi - lo + 1))
                for h in range(p.hkv):
                    rows.append(t * p.hq + h * G + gi)
    return np.array(sorted(set(rows)), dtype=np.int64)


def sum_dk_model(p, x, o_gpu, check, o_ref, lse_ref, slot, row, sample):
    """Error model of the per-kv-head sum over keys of the GPU's dK increments.

    Exactly, sum_j dS_rj = 0 for every row r (softmax shift invariance), so the
    keys' dK sum to zero.  Two roundings on the GPU leave a remainder:
    - Dt_r = dO_r . O_r is taken from the stored O, rounded to the input type
      (R15), while the backward's P_rj V_j sum to the unrounded O_r: each row's
      dS then sums to e_r = dO_r . (O_r - O_gpu,r), and the keys' dK gain
      scale * sum_r e_r Q_r over the rows r of the head's group.
    - each dS_rj is rounded to bf16 before its MFMA: round to nearest with 8
      significant bits leaves an error of mean zero and variance at most
      2^-16 dS_rj^2 / 3, so component d gains a term of standard deviation at
      most scale * sqrt(2^-16/3 * sum_r Q_rd^2 * sum_j dS_rj^2).
    With the oracle's O on every row (check == all rows) the first term is
    computed exactly (pred); otherwise it is taken as noise of variance
    scale^2 * mean(e_r^2) * sum_r Q_rd^2 (pred = 0).  sum_j dS_rj^2 and e_r^2
    are averaged over the rows `sample` (a subset of `check`), in fp64 from the
    oracle's LSE and O.  fp32 accumulation adds far less.  o_gpu: [C*Hq][D];
    o_ref, lse_ref: oracle values of the rows `check`; slot, row: the pool
    position of each key of J(h).  Returns (pred, sigma), each [Hkv][D]."""
    G = p.group
    scale = p.scale if p.scale else 1.0 / np.sqrt(p.d)
    do = synth.as_float(x["do"], p.dtype).reshape(p.c, p.hq, p.d)
    q = synth.as_float(x["q"], p.dtype).reshape(p.c, p.hq, p.d)
    pos = {int(r): i for i, r in enumerate(check)}
    every = len(check) == p.c * p.hq
    pk = p.keff * p.ps
    pred = np.zeros((p.hkv, p.d))
    sigma = np.zeros((p.hkv, p.d))
    if every:
        e = np.einsum("tgd,tgd->tg", do, (o_ref - o_gpu).reshape(p.c, p.hq, p.d))
    for h in range(p.hkv):
        sl = slice(h * G, (h + 1) * G)
        qq = np.sum(q[:, sl] ** 2, axis=(0, 1))
        kh = synth.as_float(x["k_pool"][slot[h], h, row[h]], p.dtype)
        vh = synth.as_float(x["v_pool"][slot[h], h, row[h]], p.dtype)
        ds2, e2 = [], []
        for r in sample:
            t, g = divmod(int(r), p.hq)
            if g // G != h:
                continue
            i = pos[int(r)]
            n = pk + t + 1                                    # prior keys, then chunk tokens u <= t
            pr = np.exp(scale * (kh[:n] @ q[t, g]) - lse_ref[i])
            dpr = vh[:n] @ do[t, g]
            ds2.append(np.sum((pr * (dpr - do[t, g] @ o_ref[i])) ** 2))
            e2.append(float(do[t, g] @ (o_ref[i] - o_gpu[r])) ** 2)
        var = (2.0 ** -16 if p.dtype == "bf16" else 2.0 ** -48) / 3 * float(np.mean(ds2)) * qq
        if every:
            pred[h] = scale * np.einsum("tg,tgd->d", e[:, sl], q[:, sl])
        else:
            var = var + float(np.mean(e2)) * qq
        sigma[h] = scale * np.sqrt(var)
    return pred, sigma


def run_sampled(p, seed, ora, report=None, n_local=32, every_row=False):
    """Full-size problem: rep and selection exactly; O/LSE/dQ on sampled rows
    (every row with every_row=True); dK/dV of the last n_local chunk tokens
    (only later rows see them); softmax invariants; then a second backward
    whose dO is zero outside the sampled rows, which makes dK/dV of every key
    exact from those rows alone."""
    report = {} if report is None else report
    rng = np.random.default_rng(seed)
    say(f"  generating inputs {p}")
    x = synth.make_inputs(p, seed)
    d = Device(p, x, canary_seed=None)
    st = make_step(p)
    pages = p.n + p.chunk_pages
    say("  gpu: rep, select, fwd, bwd")
    st.rep_update(d.k, d.pt, 0, pages)
    st.select(d.q)
    st.fwd(d.q, d.k, d.v, d.pt)
    st.bwd(d.q, d.k, d.v, d.pt, d.do, d.dk, d.dv)
    torch.cuda.synchronize()

    say("  oracle: rep and selection")
    rep = st.rep.cpu().numpy()
    orep = ora.rep(p, x["k_pool"], x["page_table"], 0, pages)
    err = float(np.max(np.abs(rep - orep)))
    report["rep"] = dict(max_abs=err)
    assert err <= 1e-5 * max(1.0, float(np.max(np.abs(orep)))), f"rep err {err:.3e}"
    keff = p.keff
    sel = st.sel[:, :keff].cpu().numpy()
    oscores = ora.scores(p, ora.qmean(p, x["q"]), orep[: p.n])
    gscores = st.scores[:, : p.n].cpu().numpy()
    serr = float(np.max(np.abs(gscores - oscores)))
    report["scores"] = dict(max_abs=serr)
    assert serr <= 1e-5 * max(1.0, float(np.max(np.abs(oscores)))), f"scores err {serr:.3e}"
    report["sel_exact"] = check_selection(sel, oscores, keff)

    rows = sample_rows(p, rng)
    check = ora.all_rows(p) if every_row else rows
    tag = "all rows" if every_row else "rows"
    say(f"  oracle: forward and dQ on {len(check)} rows")
    oo, ol = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, rows=check)
    o_gpu = host(st.o).reshape(-1, p.d)
    lse = st.lse.cpu().numpy().T.reshape(-1)[check]
    compare(f"O[{tag}]", o_gpu[check], oo, p.dtype, report)
    compare_lse(lse, ol, p.dtype, report)
    odq, _, _ = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"], rows=check, dkdv=False)
    compare(f"dQ[{tag}]", st.dq.cpu().numpy().reshape(-1, p.d)[check], odq, p.dtype, report)
    slot, row = ora.key_slots(p, x["page_table"], sel)
    model = sum_dk_model(p, x, o_gpu, check, oo, ol, slot, row, rows[:: max(1, len(rows) // 300)])
    del oo, ol, odq

    # last chunk tokens: seen only by rows t >= C - n_local
    say(f"  oracle: dK/dV of the last {n_local} chunk tokens")
    late = np.arange((p.c - n_local) * p.hq, p.c * p.hq, dtype=np.int64)
    _, odk, odv = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"], rows=late)
    jj = np.arange(keff * p.ps + p.c - n_local, keff * p.ps + p.c)
    dk = torch.stack([d.dk[torch.from_numpy(slot[h, jj]).cuda(), h, torch.from_numpy(row[h, jj]).cuda()]
                      for h in range(p.hkv)]).double().cpu().numpy() - 0.5
    dv = torch.stack([d.dv[torch.from_numpy(slot[h, jj]).cuda(), h, torch.from_numpy(row[h, jj]).cuda()]
                      for h in range(p.hkv)]).double().cpu().numpy() + 0.25
    compare("dK[last tokens]", dk, odk[:, jj], p.dtype, report)
    compare("dV[last tokens]", dv, odv[:, jj], p.dtype, report)

    # invariants over all keys, on the device
    touched = torch.from_numpy(touched_mask(p, ora, x["page_table"], sel)).cuda()
    G = p.group
    do_sum = torch.from_numpy(synth.as_float(x["do"], p.dtype).reshape(p.c, p.hkv, G, p.d).sum(axis=(0, 2)))
    inv_v = 0.0
    sum_dk = np.zeros((p.hkv, p.d))
    for h in range(p.hkv):
        m = touched[:, h]
        sum_dk[h] = (d.dk[m, h].double() - 0.5).sum(dim=(0, 1)).cpu().numpy()
        sv = (d.dv[m, h].double() + 0.25).sum(dim=(0, 1)).cpu()
        inv_v = max(inv_v, float((sv - do_sum[h]).abs().max()))
        assert bool((d.dk[~m, h] == 0.5).all()) and bool((d.dv[~m, h] == -0.25).all()), "untouched slot changed"
    inv_k = float(np.abs(sum_dk).max())
    report["sum_dK"] = inv_k
    report["sum_dV_minus_sum_dO"] = inv_v
    # the error model: what the Dt term leaves, within 5 standard deviations
    # of the rounding terms, component by component
    pred, sigma = model
    resid = sum_dk - pred
    report["sum_dK_model"] = dict(
        pred_max=float(np.abs(pred).max()), resid_max=float(np.abs(resid).max()),
        resid_rms=float(np.sqrt(np.mean(resid ** 2))), sigma_mean=float(np.mean(sigma)),
        resid_over_sigma_max=float(np.max(np.abs(resid) / sigma)))
    assert np.all(np.abs(resid) <= 5 * sigma), f"sum of dK: residual {report['sum_dK_model']}"
    assert inv_v <= 1e-3 * float(do_sum.abs().max()), f"sum of dV - sum of dO {inv_v:.3e}"

    # backward again with dO zero outside the sampled rows: every key is exact from them
    say("  gpu: backward with dO on sampled rows only")
    do_sparse = np.zeros_like(x["do"])
    flat_src = x["do"].reshape(-1, p.d)
    do_sparse.reshape(-1, p.d)[rows] = flat_src[rows]
    d.dk.fill_(0.5)
    d.dv.fill_(-0.25)
    st.bwd(d.q, d.k, d.v, d.pt, dev(do_sparse, p.dtype), d.dk, d.dv)
    torch.cuda.synchronize()
    say("  oracle: dK/dV of every key from the sampled rows")
    sdq, sdk, sdv = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, do_sparse, rows=rows)
    gdq = st.dq.cpu().numpy().reshape(-1, p.d)
    compare("dQ[sparse dO]", gdq[rows], sdq, p.dtype, report)
    others = np.setdiff1d(np.arange(p.c * p.hq), rows)
    assert not np.any(gdq[others]), "dQ of a row with dO = 0 is not 0"
    dk = torch.stack([d.dk[torch.from_numpy(slot[h]).cuda(), h, torch.from_numpy(row[h]).cuda()]
                      for h in range(p.hkv)]).double().cpu().numpy() - 0.5
    dv = torch.stack([d.dv[torch.from_numpy(slot[h]).cuda(), h, torch.from_numpy(row[h]).cuda()]
                      for h in range(p.hkv)]).double().cpu().numpy() + 0.25
    compare("dK[sparse dO]", dk, sdk, p.dtype, report)
    compare("dV[sparse dO]", dv, sdv, p.dtype, report)
    return report
