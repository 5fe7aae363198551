"""oomb_check_tables on the device: the counts of invalid selection and
page-table entries against the same counts taken in numpy, on valid tables
(all zero) and on tables with planted faults.  The check only reads the tables,
so the faulty ones are safe to hand to it (they are never given to the
attention kernels)."""
import numpy as np
import pytest
import torch

import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu


def expected(sel, pt, n, n_slots):
    c = [0, 0, 0, 0]
    if sel.size:
        c[0] = int(((sel < 0) | (sel >= n)).sum())
        c[1] = int((np.diff(sel, axis=1) <= 0).sum())
    seen = set()
    for s in pt:
        if s < 0 or s >= n_slots:
            c[2] += 1
        elif s in seen:
            c[3] += 1
        else:
            seen.add(int(s))
    return c


def run(p, sel, pt):
    import paged_sparse_attention_amd as P
    desc = P.make_desc(p.hq, p.hkv, p.d, p.ps, p.c, p.n, p.k, p.slots, dtype=p.dtype)
    counts = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((max(P.oomb_check_workspace_bytes(desc) // 4, 1),), 5, dtype=torch.int32, device="cuda")
    sel_d = H.dev(np.ascontiguousarray(sel, dtype=np.int32)) if sel.size else torch.zeros(1, dtype=torch.int32,
                                                                                          device="cuda")
    P.oomb_check_tables(desc, H.dev(np.ascontiguousarray(pt, dtype=np.int32)), sel_d, counts, ws)
    return counts.cpu().tolist()


CASES = {
    "qwen-ps128": (3, synth.Problem(hq=28, hkv=4, d=128, ps=128, c=512, n=40, k=8, dtype="bf16", n_slots=60)),
    "k0-local-only": (4, synth.Problem(hq=4, hkv=2, d=64, ps=16, c=64, n=10, k=0, dtype="f32")),
    "dense": (5, synth.Problem(hq=8, hkv=2, d=64, ps=32, c=64, n=12, k=100, dtype="bf16")),
}


@pytest.mark.parametrize("name", list(CASES))
def test_valid_and_planted_faults(name):
    seed, p = CASES[name]
    H.say(f"case check-tables {name}: {p}")
    rng = np.random.default_rng(seed)
    pt = synth.page_table(p, seed).astype(np.int64)
    keff = min(p.k, p.n)
    sel = np.stack([np.sort(rng.choice(p.n, keff, replace=False)) for _ in range(p.hkv)]) if keff else \
        np.zeros((p.hkv, 0), np.int64)
    assert run(p, sel, pt) == [0, 0, 0, 0]
    bad_pt = pt.copy()
    bad_pt[0] = p.slots                      # out of range
    bad_pt[-1] = -5                          # out of range
    bad_pt[1] = bad_pt[2]                    # a repeated slot
    want = expected(sel, bad_pt, p.n, p.slots)
    assert want[2] == 2 and want[3] >= 1
    assert run(p, sel, bad_pt) == want
    if keff >= 3:
        bad_sel = sel.copy()
        bad_sel[0, 0] = p.n                  # beyond the prior pages
        bad_sel[-1, 1], bad_sel[-1, 2] = bad_sel[-1, 2], bad_sel[-1, 1]   # out of order
        bad_sel[1 % p.hkv, -1] = -1
        want = expected(bad_sel, pt, p.n, p.slots)
        assert want[0] == 2 and want[1] >= 2
        assert run(p, bad_sel, pt) == want
