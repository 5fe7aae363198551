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


def run_full(p, seed, ora, report=None):
    """Every output against the oracle, element by element (small problems)."""
    report = {} if report is None else report
    x = synth.make_inputs(p, seed)
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
    compare("dQ", st.dq.cpu().numpy().reshape(-1, p.d), odq, p.dtype, report)
    dk = d.dk.cpu().numpy()
    dv = d.dv.cpu().numpy()
    slot, row = ora.key_slots(p, x["page_table"], sel)
    gdk = np.stack([(dk[slot[h], h, row[h]].astype(np.float64) - d.dk0[slot[h], h, row[h]]) for h in range(p.hkv)])
    gdv = np.stack([(dv[slot[h], h, row[h]].astype(np.float64) - d.dv0[slot[h], h, row[h]]) for h in range(p.hkv)])
    compare("dK", gdk, odk, p.dtype, report)
    compare("dV", gdv, odv, p.dtype, report)
    untouched = ~touched_mask(p, ora, x["page_table"], sel)
    for name, after, before in (("dK", dk, d.dk0), ("dV", dv, d.dv0)):
        a = after[untouched]
        b = before[untouched]
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name}: an unselected slot changed"
    return report, st, d, x, sel


def sample_rows(p, rng, n_extra=12):
    """Rows t*Hq + g covering the chunk's edges, page edges and every kv-head."""
    toks = {0, 1, p.ps - 1, min(p.ps, p.c - 1), p.c // 2, max(p.c - p.ps - 1, 0), max(p.c - 2, 0), p.c - 1}
    toks |= set(int(t) for t in rng.integers(0, p.c, n_extra))
    rows = []
    for i, t in enumerate(sorted(toks)):
        for g in {(i * 5) % p.hq, (i * 5 + p.group) % p.hq, p.hq - 1 - (i % p.hq)}:
            rows.append(t * p.hq + g)
    return np.array(sorted(set(rows)), dtype=np.int64)


def run_sampled(p, seed, ora, report=None, n_local=32):
    """Full-size problem: rep and selection exactly; O/LSE/dQ on sampled rows;
    dK/dV of the last n_local chunk tokens (only later rows see them); softmax
    invariants; then a second backward whose dO is zero outside the sampled rows,
    which makes dK/dV of every key exact from those rows alone."""
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
    say(f"  oracle: forward and dQ on {len(rows)} rows")
    oo, ol = ora.fwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, rows=rows)
    o = host(st.o).reshape(-1, p.d)[rows]
    lse = st.lse.cpu().numpy().T.reshape(-1)[rows]
    compare("O[rows]", o, oo, p.dtype, report)
    compare_lse(lse, ol, p.dtype, report)
    odq, _, _ = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"], rows=rows, dkdv=False)
    compare("dQ[rows]", st.dq.cpu().numpy().reshape(-1, p.d)[rows], odq, p.dtype, report)

    # last chunk tokens: seen only by rows t >= C - n_local
    say(f"  oracle: dK/dV of the last {n_local} chunk tokens")
    late = np.arange((p.c - n_local) * p.hq, p.c * p.hq, dtype=np.int64)
    _, odk, odv = ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], x["page_table"], sel, x["do"], rows=late)
    slot, row = ora.key_slots(p, x["page_table"], sel)
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
    inv_k, inv_v = 0.0, 0.0
    for h in range(p.hkv):
        m = touched[:, h]
        sk = (d.dk[m, h].double() - 0.5).sum(dim=(0, 1)).cpu()
        sv = (d.dv[m, h].double() + 0.25).sum(dim=(0, 1)).cpu()
        inv_k = max(inv_k, float(sk.abs().max()))
        inv_v = max(inv_v, float((sv - do_sum[h]).abs().max()))
        assert bool((d.dk[~m, h] == 0.5).all()) and bool((d.dv[~m, h] == -0.25).all()), "untouched slot changed"
    report["sum_dK"] = inv_k
    report["sum_dV_minus_sum_dO"] = inv_v
    assert inv_k <= 5e-2, f"sum of dK over keys {inv_k:.3e}"
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
