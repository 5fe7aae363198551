"""oomb_host_accumulate_grads on the CPU (host memory only, no HIP call): the
compact gradient blocks of one step added into the host dK/dV pools, against
the same adds done block by block in numpy; entries out of range are skipped,
untouched blocks keep their bits, and the thread count does not change the
result."""
import numpy as np
import pytest
import torch

import paged_sparse_attention_amd as P


def case(hkv, d, ps, c, n, k, slots, seed):
    rng = np.random.default_rng(seed)
    desc = P.make_desc(4 * hkv, hkv, d, ps, c, n, k, slots, dtype="bf16")
    keff = min(k, n)
    pt = rng.permutation(slots)[: n + c // ps].astype(np.int32)
    sel = np.stack([np.sort(rng.choice(n, keff, replace=False)) for _ in range(hkv)]).astype(np.int32) \
        if keff else np.zeros((hkv, 1), np.int32)
    nb = hkv * keff + (c // ps) * hkv
    delta_k = rng.standard_normal((nb, ps, d)).astype(np.float32)
    delta_v = rng.standard_normal((nb, ps, d)).astype(np.float32)
    hk = rng.standard_normal((slots, hkv, ps, d)).astype(np.float32)
    hv = rng.standard_normal((slots, hkv, ps, d)).astype(np.float32)
    return desc, keff, pt, sel, delta_k, delta_v, hk, hv


def expected(hkv, c, ps, n, keff, pt, sel, delta_k, delta_v, hk, hv):
    ek, ev = hk.copy(), hv.copy()
    for h in range(hkv):
        for j in range(keff):
            p = sel[h, j]
            if 0 <= p < n and 0 <= pt[p] < hk.shape[0]:
                ek[pt[p], h] += delta_k[h * keff + j]
                ev[pt[p], h] += delta_v[h * keff + j]
    for j in range(c // ps):
        for h in range(hkv):
            b = hkv * keff + j * hkv + h
            ek[pt[n + j], h] += delta_k[b]
            ev[pt[n + j], h] += delta_v[b]
    return ek, ev


@pytest.mark.parametrize("threads", [0, 1, 3, 8])
@pytest.mark.parametrize("shape", [(2, 64, 16, 32, 10, 3, 15), (4, 128, 128, 256, 6, 64, 9), (2, 64, 32, 64, 0, 4, 2)])
def test_matches_numpy(shape, threads):
    hkv, d, ps, c, n, k, slots = shape
    desc, keff, pt, sel, dk, dv, hk, hv = case(hkv, d, ps, c, n, k, slots, seed=threads + 10 * n)
    ek, ev = expected(hkv, c, ps, n, keff, pt, sel, dk, dv, hk, hv)
    tk, tv = torch.from_numpy(hk.copy()), torch.from_numpy(hv.copy())
    P.oomb_host_accumulate_grads(desc, torch.from_numpy(dk), torch.from_numpy(dv), torch.from_numpy(pt),
                                 torch.from_numpy(sel), tk, tv, threads)
    assert np.array_equal(tk.numpy(), ek) and np.array_equal(tv.numpy(), ev)


def test_out_of_range_entries_are_skipped():
    hkv, d, ps, c, n, k, slots = 2, 64, 16, 32, 10, 3, 15
    desc, keff, pt, sel, dk, dv, hk, hv = case(hkv, d, ps, c, n, k, slots, seed=5)
    sel[0, 1] = n + 3          # not a prior page
    sel[1, 2] = -1
    pt[n] = slots + 7          # chunk page 0 maps outside the pool
    ek, ev = hk.copy(), hv.copy()
    for h in range(hkv):
        for j in range(keff):
            p = sel[h, j]
            if 0 <= p < n:
                ek[pt[p], h] += dk[h * keff + j]
                ev[pt[p], h] += dv[h * keff + j]
    for j in range(1, c // ps):
        for h in range(hkv):
            b = hkv * keff + j * hkv + h
            ek[pt[n + j], h] += dk[b]
            ev[pt[n + j], h] += dv[b]
    tk, tv = torch.from_numpy(hk.copy()), torch.from_numpy(hv.copy())
    P.oomb_host_accumulate_grads(desc, torch.from_numpy(dk), torch.from_numpy(dv), torch.from_numpy(pt),
                                 torch.from_numpy(sel), tk, tv, 4)
    assert np.array_equal(tk.numpy(), ek) and np.array_equal(tv.numpy(), ev)


def test_rejects_bad_arguments():
    desc = P.make_desc(8, 2, 64, 16, 32, 10, 3, 15, dtype="bf16")
    a = torch.zeros(16)
    with pytest.raises(P.OombError):
        P.oomb_host_accumulate_grads(desc, a, a, a, a, a, a, 1000)
    assert P._L.oomb_host_accumulate_grads(P.ctypes.byref(desc), None, a.data_ptr(), a.data_ptr(), a.data_ptr(),
                                           a.data_ptr(), a.data_ptr(), 1) == -1
