"""The C-ABI library on the CPU: it loads, exports every entry point that
include/oomb.h declares, and rejects bad descriptors, pointers and workspaces
with the documented status codes before any HIP call (the pointers below are
fake addresses; every case fails validation, so nothing is launched)."""
import os
import re
import subprocess

import pytest

import paged_sparse_attention_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oomb.h")

OK, NULL_PTR, BAD_SHAPE, UNSUPPORTED, BAD_DTYPE, MISALIGNED, WORKSPACE, LAUNCH = 0, -1, -2, -3, -4, -5, -6, -7
NOT_MAPPED = -8
SCRATCH_LIMIT = -9
A = 0x10000        # a fake, 16-byte aligned device address
B = 0x20000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oomb_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"oomb_rep_update", "oomb_select_topk", "oomb_attn_fwd", "oomb_attn_bwd"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    # nothing else leaks out of the library
    assert {e for e in exported if e.startswith("oomb")} == set(names)


def test_version_and_status_strings():
    assert P.oomb_abi_version() == P.ABI_VERSION == 2
    for code in (OK, NULL_PTR, BAD_SHAPE, UNSUPPORTED, BAD_DTYPE, MISALIGNED, WORKSPACE, LAUNCH, NOT_MAPPED,
                 SCRATCH_LIMIT):
        assert P.oomb_status_string(code) and P.oomb_status_string(code) != "unknown status"
    assert P.oomb_status_string(-99) == "unknown status"


def test_single_hip_runtime():
    assert len(P.hip_runtimes_loaded()) == 1


def good(**kw):
    base = dict(n_q_heads=28, n_kv_heads=4, head_dim=128, page_size=128, chunk_len=4096, n_prior_pages=2048,
                top_k=64, n_slots=2080)
    base.update(kw)
    return P.make_desc(**base)


def fwd(d, **ptrs):
    p = dict(q=A, k=A, v=A, pt=A, sel=A, o=A, lse=A)
    p.update(ptrs)
    return P._L.oomb_attn_fwd(P.ctypes.byref(d), p["q"], p["k"], p["v"], p["pt"], p["sel"], p["o"], p["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=28, n_kv_heads=5), BAD_SHAPE),
    (dict(n_q_heads=0), BAD_SHAPE),
    (dict(chunk_len=4000), BAD_SHAPE),
    (dict(chunk_len=0), BAD_SHAPE),
    (dict(n_slots=2079), BAD_SHAPE),
    (dict(rep_capacity=2000), BAD_SHAPE),
    (dict(n_prior_pages=-1), BAD_SHAPE),
    (dict(top_k=-3), BAD_SHAPE),
    (dict(softmax_scale=-1.0), BAD_SHAPE),
    (dict(softmax_scale=float("nan")), BAD_SHAPE),
    (dict(head_dim=96), UNSUPPORTED),
    (dict(page_size=256, chunk_len=4096), UNSUPPORTED),
    (dict(page_size=8, chunk_len=4096, n_slots=3000), UNSUPPORTED),
    (dict(n_kv_heads=28, n_q_heads=28), UNSUPPORTED),   # Hkv * D > 1024
])
def test_bad_descriptor(kw, code):
    assert fwd(good(**kw)) == code


def test_bad_dtype_and_null_desc():
    d = good()
    d.dtype = 7
    assert fwd(d) == BAD_DTYPE
    assert P._L.oomb_attn_fwd(None, A, A, A, A, A, A, A, None) == NULL_PTR
    assert P.oomb_select_workspace_bytes(d) == 0 and P.oomb_bwd_workspace_bytes(d) == 0


@pytest.mark.parametrize("name", ["q", "k", "v", "pt", "sel", "o", "lse"])
def test_null_and_misaligned_pointers(name):
    d = good(n_slots=0)  # also invalid: must report the descriptor first
    assert fwd(d, **{name: None}) == BAD_SHAPE
    # the descriptor is made valid but the pointer is NULL / misaligned: rejected before launch
    assert fwd(good(), **{name: None}) == NULL_PTR
    assert fwd(good(), **{name: A + 4}) == MISALIGNED


def test_sel_may_be_null_without_selection():
    # K_eff = 0 needs no sel pointer; a NULL q must still be caught
    assert fwd(good(top_k=0), sel=None, q=None) == NULL_PTR
    assert fwd(good(n_prior_pages=0, n_slots=32), sel=None, lse=A + 8) == MISALIGNED


def test_workspaces():
    d = good()
    ws = P.oomb_select_workspace_bytes(d)
    wb = P.oomb_bwd_workspace_bytes(d)
    assert ws > 0 and wb >= 28 * 4096 * 4
    L = P._L
    r = L.oomb_select_topk(P.ctypes.byref(d), A, A, A, None, A, ws - 1, None)
    assert r == WORKSPACE
    assert L.oomb_select_topk(P.ctypes.byref(d), A, A, A, None, None, ws, None) == WORKSPACE
    assert L.oomb_select_topk(P.ctypes.byref(d), A, A, A, None, A + 4, ws, None) == MISALIGNED
    args = [A] * 11
    assert L.oomb_attn_bwd(P.ctypes.byref(d), *args, A, wb - 1, None) == WORKSPACE
    assert L.oomb_attn_bwd(P.ctypes.byref(d), *args, None, wb, None) == WORKSPACE
    args[8] = None  # dq
    assert L.oomb_attn_bwd(P.ctypes.byref(d), *args, A, wb, None) == NULL_PTR


def test_select_noalloc_checks():
    """The allocation-free selection: the same argument checks as
    oomb_select_topk, and shapes whose workspace exceeds the library's 4 MiB
    scratch are rejected, all before any HIP call."""
    L = P._L
    d = good()
    assert L.oomb_select_topk_noalloc(P.ctypes.byref(d), None, A, A, None, None) == NULL_PTR
    assert L.oomb_select_topk_noalloc(P.ctypes.byref(d), A, A, None, None, None) == NULL_PTR
    assert L.oomb_select_topk_noalloc(P.ctypes.byref(d), A, A, A, A + 4, None) == MISALIGNED
    assert L.oomb_select_topk_noalloc(P.ctypes.byref(good(chunk_len=4000)), A, A, A, None, None) == BAD_SHAPE
    big = good(n_prior_pages=300000, n_slots=300032)       # Hkv * N = 1.2 million scores
    assert P.oomb_select_workspace_bytes(big) > 4 << 20
    assert L.oomb_select_topk_noalloc(P.ctypes.byref(big), A, A, A, None, None) == SCRATCH_LIMIT
    assert P.oomb_select_workspace_bytes(good(n_prior_pages=32768, n_slots=32800)) <= 4 << 20  # sparse-4m fits


def test_rep_update_ranges():
    d = good()
    L = P._L
    total = 2048 + 4096 // 128
    assert L.oomb_rep_update(P.ctypes.byref(d), A, A, -1, 4, A, None) == BAD_SHAPE
    assert L.oomb_rep_update(P.ctypes.byref(d), A, A, 0, total + 1, A, None) == BAD_SHAPE
    assert L.oomb_rep_update(P.ctypes.byref(d), A, A, total - 3, 4, A, None) == BAD_SHAPE
    assert L.oomb_rep_update(P.ctypes.byref(d), A, A, 0, -1, A, None) == BAD_SHAPE
    assert L.oomb_rep_update(P.ctypes.byref(d), None, A, 0, 4, A, None) == NULL_PTR
    assert L.oomb_rep_update(P.ctypes.byref(d), A, A, 0, 4, A + 2, None) == MISALIGNED


def test_binding_raises():
    with pytest.raises(P.OombError) as e:
        P.oomb_attn_fwd(good(head_dim=80), A, A, A, A, A, A, A, stream=0)
    assert e.value.status == UNSUPPORTED


# ---- offload entry points: the staged descriptor (host arithmetic only) and
# argument checks that fail before any HIP call

def test_stage_desc():
    d = good()                                    # Hkv 4, K 64 of N 2048, C/ps 32
    s = P.oomb_stage_desc(d)
    assert (s.n_prior_pages, s.top_k, s.n_slots, s.rep_capacity) == (256, 64, 288, 288)
    assert (s.n_q_heads, s.n_kv_heads, s.head_dim, s.page_size, s.chunk_len, s.dtype) == (28, 4, 128, 128, 4096, 1)
    s = P.oomb_stage_desc(good(n_prior_pages=10, top_k=64, n_slots=42))   # K_eff = N = 10
    assert (s.n_prior_pages, s.top_k, s.n_slots) == (40, 10, 72)
    s = P.oomb_stage_desc(good(n_prior_pages=0, n_slots=32))              # first chunk: no prior pages
    assert (s.n_prior_pages, s.top_k, s.n_slots) == (0, 0, 32)
    with pytest.raises(P.OombError) as e:
        P.oomb_stage_desc(good(chunk_len=4000))
    assert e.value.status == BAD_SHAPE
    assert P._L.oomb_stage_desc(P.ctypes.byref(good()), None) == NULL_PTR


def test_stage_calls_reject_bad_arguments():
    d = P.ctypes.byref(good())
    L = P._L
    g = lambda src=A, slots=2080, sel=A, parts=3, first=0, n=2048: L.oomb_stage_gather(
        d, src, A, slots, A, sel, parts, first, n, A, A, None)
    assert g(parts=0) == BAD_SHAPE                                  # no part
    assert g(parts=4) == BAD_SHAPE                                  # unknown part
    assert g(slots=0) == BAD_SHAPE
    assert g(first=-1) == BAD_SHAPE and g(n=-1) == BAD_SHAPE
    assert g(src=None) == NULL_PTR
    assert g(sel=None, parts=1) == NULL_PTR                         # selection needed
    assert g(src=A + 4) == MISALIGNED
    assert L.oomb_stage_offload_chunk(d, A, A, A, None, A, None) == NULL_PTR
    assert L.oomb_stage_flush_grads(d, A, A, A, None, A, A, None) == NULL_PTR
    assert L.oomb_stage_flush_grads(d, A, A, A, A, A, A + 8, None) == MISALIGNED
    assert L.oomb_stage_tables(d, A, None, None) == NULL_PTR
    assert L.oomb_stage_tables(P.ctypes.byref(good(head_dim=96)), A, A, None) == UNSUPPORTED
    out = P.ctypes.c_void_p()
    assert L.oomb_host_view(None, P.ctypes.byref(out)) == NULL_PTR
    assert L.oomb_host_view(A, None) == NULL_PTR


def test_check_tables_argument_checks():
    d = good()
    L = P._L
    assert P.oomb_check_workspace_bytes(d) == 4 * 2080
    assert P.oomb_check_workspace_bytes(good(chunk_len=4000)) == 0
    dr = P.ctypes.byref(d)
    assert L.oomb_check_tables(dr, A, A, None, B, 4 * 2080, None) == NULL_PTR
    assert L.oomb_check_tables(dr, A, None, A, B, 4 * 2080, None) == NULL_PTR    # K_eff > 0 needs sel
    assert L.oomb_check_tables(dr, A, A, A, B, 4 * 2080 - 4, None) == WORKSPACE
    assert L.oomb_check_tables(dr, A, A, A, None, 4 * 2080, None) == WORKSPACE
    assert L.oomb_check_tables(dr, A, A, A, B + 8, 4 * 2080, None) == MISALIGNED


def test_probe_argument_checks():
    L = P._L
    assert L.oomb_probe_mfma_peak(0, 1, A, None) == BAD_SHAPE
    assert L.oomb_probe_mfma_peak(65537, 1, A, None) == BAD_SHAPE
    assert L.oomb_probe_mfma_peak(1, 0, A, None) == BAD_SHAPE
    assert L.oomb_probe_mfma_peak(1, (1 << 20) + 1, A, None) == BAD_SHAPE
    assert L.oomb_probe_mfma_peak(1, 1, None, None) == NULL_PTR
    assert L.oomb_probe_mfma_peak(1, 1, A + 4, None) == MISALIGNED


def test_layer_op_argument_checks():
    L = P._L
    assert L.oomb_rmsnorm_fwd(None, A, 4, 256, 1e-6, B, A, None) == NULL_PTR
    assert L.oomb_rmsnorm_fwd(A, A, 4, 254, 1e-6, B, A, None) == BAD_SHAPE
    assert L.oomb_rmsnorm_fwd(A, A, 4, 8196, 1e-6, B, A, None) == BAD_SHAPE
    assert L.oomb_rmsnorm_fwd(A + 4, A, 4, 256, 1e-6, B, A, None) == MISALIGNED
    assert L.oomb_rmsnorm_bwd(A, A, A, A, None, 4, 256, None, None) == NULL_PTR
    assert L.oomb_rmsnorm_bwd(A, A, A, A, A + 8, 4, 256, B, None) == MISALIGNED
    assert L.oomb_rmsnorm_gain_grad(A, A, A, 4, 256, 0, B, None) == BAD_SHAPE
    assert L.oomb_rotary(A, 2, B, A, A, 4, 2, 64, 0, 0, None) == BAD_DTYPE
    assert L.oomb_rotary(A, 1, B, A, A, 4, 2, 63, 0, 0, None) == BAD_SHAPE
    assert L.oomb_rotary(A, 1, None, A, A, 4, 2, 64, 0, 0, None) == NULL_PTR
    assert L.oomb_swiglu_fwd(A, A, B, 6, None) == BAD_SHAPE
    assert L.oomb_swiglu_bwd(A, A, A, B, B + 2, 8, None) == MISALIGNED


@pytest.mark.parametrize("kw,splits,sub", [
    (dict(), 4, 2),                                            # 96 key blocks x 4 kv-heads: 4 splits
    (dict(chunk_len=8192, n_prior_pages=32768, top_k=128, n_slots=32832), 4, 2),  # 192 blocks: at least 4
    (dict(chunk_len=256, n_prior_pages=12, top_k=4, n_slots=14), 8, 2),          # 12 blocks: capped at 8
    (dict(chunk_len=2048, n_prior_pages=48, top_k=48, n_slots=64), 6, 2),           # 64 blocks: 1536 / 256
    (dict(n_q_heads=21, n_kv_heads=3), 6, 1),                # 288 blocks x heads: no whole groups per XCD
])
def test_bwd_workspace_holds_the_split_partials(kw, splits, sub):
    # Dt, lse*log2(e) and the rows' bias operands (32 bytes a row), then the
    # partial dK and dV sums of every row split but the first, each
    # [Hkv][K_eff*ps + C][D] fp32, every part rounded up to 256 bytes.
    # Rows of a key block are split over max(4, ceil(1536 / (key blocks x
    # kv-heads))) workgroups, at most 8; a key block is 128 keys (bf16).
    # When the (kv-head, split) groups divide evenly over 8 XCDs and an XCD
    # gets at most 128 chunk key blocks, each share of a chunk key block is
    # halved, and the second halves' sums take [splits][Hkv][chunk block keys][D]
    # more for dK and for dV.
    d = good(**kw)
    hq, hkv, dd, c = d.n_q_heads, d.n_kv_heads, d.head_dim, d.chunk_len
    pk = min(d.top_k, d.n_prior_pages) * d.page_size
    keys = pk + c
    blocks = -(-keys // 128)
    assert min(8, max(4, -(-1536 // (blocks * hkv)))) == splits
    nprior = min(blocks, -(-pk // 128))
    total = blocks * splits * hkv
    ordered = total % 8 == 0 and (total // 8) % blocks == 0 and 0 < nprior < blocks
    assert (2 if ordered and (total // 8 // blocks) * (blocks - nprior) <= 128 else 1) == sub
    up = lambda n: (n + 255) // 256 * 256
    part = up((splits - 1) * hkv * keys * dd * 4)
    part2 = up(splits * hkv * (keys - nprior * 128) * dd * 4) if sub == 2 else 0
    assert P.oomb_bwd_workspace_bytes(d) == 2 * up(hq * c * 4) + up(hq * c * 32) + 2 * part + 2 * part2


def test_trace_filter_arguments():
    # host-only state: the name is checked and copied, nothing is launched
    L = P._L
    assert L.oomb_trace_only(b"dkdv_kernel") == OK
    assert L.oomb_trace_only(b"") == BAD_SHAPE
    assert L.oomb_trace_only(b"k" * 63) == OK
    assert L.oomb_trace_only(b"k" * 64) == BAD_SHAPE
    assert L.oomb_trace_only(None) == OK
    P.oomb_trace_only("fwd_kernel")
    P.oomb_trace_only(None)
