"""CPU offloading of the KV cache and its gradients, through the C ABI.

1. The staging copy kernels (oomb_stage_gather, oomb_stage_offload_chunk,
   oomb_stage_flush_grads, oomb_stage_grads_out) and the host-side
   oomb_host_accumulate_grads against the same block moves done with numpy:
   bit-exact, including the blocks they must leave alone.
2. OffloadedSequence (K/V and dK/dV pools in pinned host memory, staging on the
   device, three streams) over whole sequences:
   - against the resident ChunkedSequence: selections, O, LSE and dQ bitwise;
     the dK/dV pools to fp32 rounding (each chunk's contribution is summed in
     staging before it is added to the host pool);
   - against the whole-sequence fp64 oracle, element by element;
   - the host K/V pools end up holding every chunk's pages bit for bit (they
     start poisoned with NaN there, so only the offload can fill them);
   - two and three staging buffers, kept or recomputed activations, copy
     streams with or without their own compute units, and gradients added on
     the host or over the link by the device give bitwise the same results.
"""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import synth
import gpu_harness as H
from parity import compare, compare_lse
from test_gpu_sequence import SEQ, run_sequence

pytestmark = pytest.mark.gpu

NAN_BITS = {"bf16": np.uint16(0x7FC0), "f32": np.float32(np.nan)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")


def pinned(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.pin_memory()


def host_bits(t):
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


# ---------------------------------------------------------------- 1. kernels

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stage_copy_kernels(dtype):
    import paged_sparse_attention_amd as P
    hq, hkv, d, ps, c, n, k = 4, 2, 64, 16, 32, 10, 3
    slots = n + c // ps + 3
    H.say(f"case stage kernels {dtype}: hkv {hkv} D {d} ps {ps} C {c} N {n} K {k} slots {slots}")
    rng = np.random.default_rng(7)
    desc = P.make_desc(hq, hkv, d, ps, c, n, k, slots, dtype=dtype)
    sd = P.oomb_stage_desc(desc)
    nsel, nst = hkv * k, sd.n_slots
    pt = rng.permutation(slots)[: n + c // ps].astype(np.int32)
    sel = np.array([[1, 4, 7], [1, 5, 9]], dtype=np.int32)   # page 1 selected by both kv-heads
    blk = (slots, hkv, ps, d)
    if dtype == "bf16":
        hk = rng.integers(0, 0x7F00, blk, dtype=np.uint16)
        hv = rng.integers(0, 0x7F00, blk, dtype=np.uint16)
    else:
        hk = rng.standard_normal(blk).astype(np.float32)
        hv = rng.standard_normal(blk).astype(np.float32)
    host_k, host_v = pinned(hk, dtype), pinned(hv, dtype)
    vk, vv = P.oomb_host_view(host_k), P.oomb_host_view(host_v)
    pt_d, sel_d = H.dev(pt), H.dev(sel)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    stage_k = torch.zeros((nst, hkv, ps, d), dtype=tdt, device="cuda")
    stage_v = torch.zeros_like(stage_k)
    P.oomb_stage_gather(desc, vk, vv, pt_d, sel_d, P.OOMB_STAGE_SELECTED | P.OOMB_STAGE_CHUNK, stage_k, stage_v)
    torch.cuda.synchronize()
    want_k = np.zeros((nst,) + blk[1:], dtype=hk.dtype)
    want_v = np.zeros_like(want_k)
    for h in range(hkv):
        for j in range(k):
            want_k[h * k + j, h] = hk[pt[sel[h, j]], h]
            want_v[h * k + j, h] = hv[pt[sel[h, j]], h]
    for j in range(c // ps):
        want_k[nsel + j] = hk[pt[n + j]]
        want_v[nsel + j] = hv[pt[n + j]]
    bits = lambda t: host_bits(t.cpu())
    assert np.array_equal(bits(stage_k), want_k.view(bits(stage_k).dtype)), "gathered K"
    assert np.array_equal(bits(stage_v), want_v.view(bits(stage_v).dtype)), "gathered V"

    # staging -> host: only the chunk's pages change
    out_k, out_v = pinned(np.zeros_like(hk), dtype), pinned(np.zeros_like(hv), dtype)
    P.oomb_stage_offload_chunk(desc, stage_k, stage_v, pt_d, P.oomb_host_view(out_k), P.oomb_host_view(out_v))
    torch.cuda.synchronize()
    exp_k = np.zeros_like(hk)
    exp_v = np.zeros_like(hv)
    for j in range(c // ps):
        exp_k[pt[n + j]] = hk[pt[n + j]]
        exp_v[pt[n + j]] = hv[pt[n + j]]
    assert np.array_equal(host_bits(out_k), exp_k.view(host_bits(out_k).dtype)), "offloaded K"
    assert np.array_equal(host_bits(out_v), exp_v.view(host_bits(out_v).dtype)), "offloaded V"

    # gradient flush: host += staging on the touched blocks, which then read zero
    g0k = rng.standard_normal(blk).astype(np.float32)
    g0v = rng.standard_normal(blk).astype(np.float32)
    s0k = rng.standard_normal((nst,) + blk[1:]).astype(np.float32)
    s0v = rng.standard_normal((nst,) + blk[1:]).astype(np.float32)
    gk, gv = pinned(g0k), pinned(g0v)
    sdk, sdv = H.dev(s0k), H.dev(s0v)
    P.oomb_stage_flush_grads(desc, sdk, sdv, pt_d, sel_d, P.oomb_host_view(gk), P.oomb_host_view(gv))
    torch.cuda.synchronize()
    ek, ev, esk, esv = g0k.copy(), g0v.copy(), s0k.copy(), s0v.copy()
    for h in range(hkv):
        for j in range(k):
            ek[pt[sel[h, j]], h] += s0k[h * k + j, h]
            ev[pt[sel[h, j]], h] += s0v[h * k + j, h]
            esk[h * k + j, h] = 0
            esv[h * k + j, h] = 0
    for j in range(c // ps):
        ek[pt[n + j]] += s0k[nsel + j]
        ev[pt[n + j]] += s0v[nsel + j]
        esk[nsel + j] = 0
        esv[nsel + j] = 0
    assert np.array_equal(gk.numpy(), ek) and np.array_equal(gv.numpy(), ev), "flushed host gradients"
    assert np.array_equal(sdk.cpu().numpy(), esk) and np.array_equal(sdv.cpu().numpy(), esv), "cleared staging"

    # gradients out to a compact host buffer, then added on the host: the same
    # host pools as the flush, and the same cleared staging
    nb = nsel + (c // ps) * hkv
    out_k = pinned(np.full((nb, ps, d), np.nan, np.float32))
    out_v = pinned(np.full((nb, ps, d), np.nan, np.float32))
    sdk, sdv = H.dev(s0k), H.dev(s0v)
    P.oomb_stage_grads_out(desc, sdk, sdv, P.oomb_host_view(out_k), P.oomb_host_view(out_v))
    torch.cuda.synchronize()
    want_k = np.stack([s0k[b, b // k] for b in range(nsel)] + [s0k[nsel + j // hkv, j % hkv] for j in range(nb - nsel)])
    want_v = np.stack([s0v[b, b // k] for b in range(nsel)] + [s0v[nsel + j // hkv, j % hkv] for j in range(nb - nsel)])
    assert np.array_equal(out_k.numpy(), want_k) and np.array_equal(out_v.numpy(), want_v), "gradient blocks out"
    assert np.array_equal(sdk.cpu().numpy(), esk) and np.array_equal(sdv.cpu().numpy(), esv), "cleared staging (out)"
    gk2, gv2 = torch.from_numpy(g0k.copy()), torch.from_numpy(g0v.copy())
    P.oomb_host_accumulate_grads(desc, out_k, out_v, torch.from_numpy(pt), torch.from_numpy(sel), gk2, gv2, 4)
    assert np.array_equal(gk2.numpy(), ek) and np.array_equal(gv2.numpy(), ev), "host-accumulated gradients"


# ------------------------------------------------------------- 2. sequences

def run_offloaded(s, seed, keep=False, nbuf=2, copy_cus=8, host_acc=False):
    from paged_sparse_attention_amd.offload import OffloadedSequence
    x = synth.make_sequence_inputs(s, seed)
    last = s.step(s.chunks - 1)
    pt = x["page_table"]
    q, do = H.dev(x["q"], s.dtype), H.dev(x["do"], s.dtype)
    chunk_slots = [pt[s.n0 + i * s.chunk_pages + np.arange(s.chunk_pages)] for i in range(s.chunks)]
    k_new = H.dev(np.stack([x["k_pool"][sl] for sl in chunk_slots]), s.dtype)
    v_new = H.dev(np.stack([x["v_pool"][sl] for sl in chunk_slots]), s.dtype)
    hk, hv = x["k_pool"].copy(), x["v_pool"].copy()
    poison = np.concatenate(chunk_slots)
    hk[poison] = NAN_BITS[s.dtype]
    hv[poison] = NAN_BITS[s.dtype]
    host_k, host_v = pinned(hk, s.dtype), pinned(hv, s.dtype)
    dk0, dv0 = synth.canary(last, seed, "k"), synth.canary(last, seed, "v")
    host_dk, host_dv = pinned(dk0), pinned(dv0)
    drv = OffloadedSequence(s.hq, s.hkv, s.d, s.ps, s.c, s.chunks, s.k, n_initial_pages=s.n0, dtype=s.dtype,
                            softmax_scale=s.scale, keep_activations=keep, n_buffers=nbuf, copy_cus=copy_cus,
                            host_accumulate=host_acc)
    outs = []
    pt_d = H.dev(pt)
    drv.forward(q, k_new, v_new, host_k, host_v, pt_d,
                on_chunk=lambda i, o, lse: outs.append((o.clone(), lse.clone())))
    drv.backward(q, do, host_k, host_v, host_dk, host_dv, pt_d)
    torch.cuda.synchronize()
    # every chunk page reached the host pools, bit for bit
    for name, t, ref in (("K", host_k, x["k_pool"]), ("V", host_v, x["v_pool"])):
        assert np.array_equal(host_bits(t), ref.view(host_bits(t).dtype)), f"host {name} pool after the forward"
    gdk = host_dk.numpy().astype(np.float64) - dk0
    gdv = host_dv.numpy().astype(np.float64) - dv0
    return x, drv, outs, gdk, gdv, host_dk.numpy().copy(), host_dv.numpy().copy()


@pytest.mark.parametrize("name", list(SEQ))
def test_offloaded_sequence(ora, name):
    seed, s = SEQ[name]
    H.say(f"case {name} offloaded: {s}")
    kept = {}
    _, res, rdk, rdv = run_sequence(s, seed, keep=True, raw=kept)
    x, drv, outs, gdk, gdv, _, _ = run_offloaded(s, seed, keep=False)
    for i in range(s.chunks):
        assert torch.equal(res.sel[i], drv.sel[i]), f"chunk {i} selection"
        assert torch.equal(kept["o"][i], outs[i][0]), f"chunk {i} O"
        assert torch.equal(kept["lse"][i], outs[i][1]), f"chunk {i} LSE"
        assert torch.equal(res.dq[i], drv.dq[i]), f"chunk {i} dQ"
    # dK/dV against the resident pools: the same sums, rounded in another order
    for nm, a, b in (("dK", gdk, rdk), ("dV", gdv, rdv)):
        err = float(np.max(np.abs(a - b)))
        bound = 2e-5 * max(1.0, float(np.max(np.abs(b))))
        assert err <= bound, f"{nm} pool: offloaded vs resident max |diff| {err:.3g} > {bound:.3g}"
    sels = [drv.sel[i][:, :drv.keff(i)].cpu().numpy() if drv.keff(i) else np.zeros((s.hkv, 0), np.int32)
            for i in range(s.chunks)]
    r = ora.sequence(s, x, sels=sels)
    report = {}
    for i in range(s.chunks):
        rep_i = {}
        compare("O", H.host(outs[i][0]).reshape(-1, s.d), r["o"][i], s.dtype, rep_i)
        compare_lse(outs[i][1].cpu().numpy().T.reshape(-1), r["lse"][i], s.dtype, rep_i)
        compare("dQ", drv.dq[i].cpu().numpy().reshape(-1, s.d), r["dq"][i], s.dtype, rep_i)
        report[f"chunk{i}"] = rep_i
    compare("dK pool", gdk, r["dk"], s.dtype, report)
    compare("dV pool", gdv, r["dv"], s.dtype, report)
    H.say(f"  {json.dumps(report, default=float)}")


def test_offload_buffers_streams_and_activations_do_not_change_results():
    seed, s = SEQ["seq-qwen-shape"]
    H.say(f"case seq-qwen-shape offloaded: 2 vs 3 staging buffers, masked vs unmasked streams, "
          f"host vs device gradient adds: {s}")
    _, a, outs_a, _, _, dk_a, dv_a = run_offloaded(s, seed, keep=False, nbuf=2, copy_cus=8, host_acc=True)
    _, b, outs_b, _, _, dk_b, dv_b = run_offloaded(s, seed, keep=True, nbuf=3, copy_cus=0, host_acc=False)
    for i in range(s.chunks):
        assert torch.equal(outs_a[i][0], outs_b[i][0]) and torch.equal(outs_a[i][1], outs_b[i][1]), f"chunk {i}"
        assert torch.equal(a.dq[i], b.dq[i]), f"chunk {i} dQ"
    assert np.array_equal(dk_a, dk_b) and np.array_equal(dv_a, dv_b), "host dK/dV pools"
