"""oomb_select_topk_noalloc -- the selection on the library's own per-device
scratch, for callers that cannot allocate -- against oomb_select_topk with a
caller workspace, through the C ABI.  Both run the same kernels on the same
inputs, so the selected pages and the scores must be identical bit for bit.
Two problems in a row, the second smaller, so that the second no-alloc call
runs on a scratch that still holds the first call's partial sums and scores;
then a problem too large for the scratch, which must be rejected."""
import numpy as np
import pytest
import torch

import synth
import paged_sparse_attention_amd as P

pytestmark = pytest.mark.gpu

# (name, seed, Hq, Hkv, D, ps, C, N, K, dtype): the sparse-256k selection, then a
# small ragged problem (D 64, 16-token pages, a chunk of 96 tokens)
CASES = [
    ("sparse-256k", 3, 28, 4, 128, 128, 4096, 2048, 64, "bf16"),
    ("small-d64", 41, 6, 2, 64, 16, 96, 300, 17, "bf16"),
]


def inputs(seed, hq, hkv, d, c, n, dtype):
    q = torch.from_numpy(synth.tensor(seed, 1, (c, hq, d), dtype))
    q = (q.view(torch.bfloat16) if dtype == "bf16" else q).cuda()
    rep = torch.from_numpy(synth.tensor(seed, 9, (n, hkv, d), "f32")).cuda()
    return q, rep


def test_noalloc_matches_workspace_selection_twice():
    for name, seed, hq, hkv, d, ps, c, n, k, dtype in CASES:
        print(f"case {name}", flush=True)
        desc = P.make_desc(hq, hkv, d, ps, c, n, k, n + c // ps, dtype=dtype)
        q, rep = inputs(seed, hq, hkv, d, c, n, dtype)
        keff = min(k, n)
        ws = torch.empty(P.oomb_select_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        sel_ws = torch.full((hkv, keff), -1, dtype=torch.int32, device="cuda")
        sc_ws = torch.full((hkv, n), float("nan"), dtype=torch.float32, device="cuda")
        P.oomb_select_topk(desc, q, rep, sel_ws, sc_ws, ws)
        sel_na = torch.full((hkv, keff), -2, dtype=torch.int32, device="cuda")
        sc_na = torch.full((hkv, n), float("inf"), dtype=torch.float32, device="cuda")
        P.oomb_select_topk_noalloc(desc, q, rep, sel_na, sc_na)
        # without scores_out the scores live in the scratch; the selection is the same
        sel_na2 = torch.full((hkv, keff), -3, dtype=torch.int32, device="cuda")
        P.oomb_select_topk_noalloc(desc, q, rep, sel_na2, None)
        torch.cuda.synchronize()
        assert torch.equal(sel_na, sel_ws), name
        assert torch.equal(sel_na2, sel_ws), name
        assert torch.equal(sc_na.view(torch.int32), sc_ws.view(torch.int32)), name
        s = sel_ws.cpu().numpy()
        assert np.all(np.diff(s, axis=1) > 0) and s.min() >= 0 and s.max() < n, name


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # Hkv * N = 1.2 million scores: more than the 4 MiB scratch holds
    desc = P.make_desc(8, 4, 128, 16, 64, 300000, 64, 300004)
    assert P.oomb_select_workspace_bytes(desc) > (4 << 20)
    q = torch.zeros((64, 8, 128), dtype=torch.bfloat16, device="cuda")
    rep = torch.zeros((16, 4, 128), dtype=torch.float32, device="cuda")   # never read: rejected first
    sel = torch.zeros((4, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(P.OombError) as e:
        P.oomb_select_topk_noalloc(desc, q, rep, sel)
    assert e.value.status == -9
