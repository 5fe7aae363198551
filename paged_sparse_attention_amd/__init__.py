"""Python binding of liboomb.so, the gfx950 paged top-K chunk attention library.

Argument marshalling only: each function below has the name of the C entry
point it calls (declared in include/oomb.h), turns torch tensors into device
pointers and the current torch stream into a hipStream_t, and raises OombError
on a negative status.  Every step of the computation runs in the HIP kernels of
liboomb.so; there is no other code path.  Importing this module fails if the
library has not been built (python -m paged_sparse_attention_amd.build).

Method: page "Out of the Memory Barrier" (OOMB), technical summary, section 2
("Paged Memory Management", "Page-level Sparse Attention", "Specialized
Kernels").
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so liboomb.so binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboomb.so")

OOMB_F32, OOMB_BF16 = 0, 1
DTYPE_CODES = {"f32": OOMB_F32, "bf16": OOMB_BF16, torch.float32: OOMB_F32, torch.bfloat16: OOMB_BF16}
ABI_VERSION = 2
OOMB_STAGE_SELECTED, OOMB_STAGE_CHUNK = 1, 2


class OombError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class oomb_desc(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("chunk_len", ctypes.c_int32), ("n_prior_pages", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("rep_capacity", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


def make_desc(n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, n_prior_pages, top_k, n_slots,
              rep_capacity=None, dtype="bf16", softmax_scale=0.0) -> oomb_desc:
    pages = n_prior_pages + chunk_len // page_size
    return oomb_desc(n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, n_prior_pages, top_k, n_slots,
                     pages if rep_capacity is None else rep_capacity, DTYPE_CODES[dtype], softmax_scale)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_sparse_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(oomb_desc)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "oomb_rep_update": (ctypes.c_int, [P, vp, vp, i32, i32, vp, vp]),
        "oomb_select_workspace_bytes": (sz, [P]),
        "oomb_select_topk": (ctypes.c_int, [P, vp, vp, vp, vp, vp, sz, vp]),
        "oomb_select_topk_noalloc": (ctypes.c_int, [P, vp, vp, vp, vp, vp]),
        "oomb_attn_fwd": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp]),
        "oomb_bwd_workspace_bytes": (sz, [P]),
        "oomb_attn_bwd": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "oomb_check_workspace_bytes": (sz, [P]),
        "oomb_check_tables": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
        "oomb_host_view": (ctypes.c_int, [vp, ctypes.POINTER(vp)]),
        "oomb_stage_desc": (ctypes.c_int, [P, P]),
        "oomb_stage_tables": (ctypes.c_int, [P, vp, vp, vp]),
        "oomb_stage_gather": (ctypes.c_int, [P, vp, vp, i32, vp, vp, i32, i32, i32, vp, vp, vp]),
        "oomb_stage_offload_chunk": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp]),
        "oomb_stage_flush_grads": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp]),
        "oomb_stage_grads_out": (ctypes.c_int, [P, vp, vp, vp, vp, vp]),
        "oomb_host_accumulate_grads": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, i32]),
        "oomb_probe_mfma_peak": (ctypes.c_int, [i32, i32, vp, vp]),
        "oomb_rmsnorm_fwd": (ctypes.c_int, [vp, vp, i32, i32, ctypes.c_float, vp, vp, vp]),
        "oomb_rmsnorm_bwd": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, vp, vp]),
        "oomb_rmsnorm_gain_grad": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, vp]),
        "oomb_rotary": (ctypes.c_int, [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, vp]),
        "oomb_swiglu_fwd": (ctypes.c_int, [vp, vp, vp, ctypes.c_int64, vp]),
        "oomb_swiglu_bwd": (ctypes.c_int, [vp, vp, vp, vp, vp, ctypes.c_int64, vp]),
        "oomb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "oomb_abi_version": (ctypes.c_int, []),
        "oomb_trace_events": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
        "oomb_trace_only": (ctypes.c_int, [ctypes.c_char_p]),
        "oomb_trace_count": (ctypes.c_int, []),
        "oomb_trace_kernel": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    if L.oomb_abi_version() != ABI_VERSION:
        raise ImportError(f"liboomb.so ABI {L.oomb_abi_version()} != {ABI_VERSION}")
    return L


_L = _load()


def hip_runtimes_loaded() -> list[str]:
    """Paths of every libamdhip64 mapped into this process (one is expected)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return sorted(paths)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    raise TypeError(f"expected a tensor, an int address or None, got {type(x)}")


_IO_DTYPE = {0: torch.float32, 1: torch.bfloat16}   # oomb_dtype -> torch dtype of q, pools, o, dO


def _dev(x, dtype=None, name="argument"):
    """Address of a device buffer for the C ABI.  A tensor must be on the GPU,
    contiguous and (when given) of `dtype`, else ValueError: a host pointer, a
    strided view or a wrong element type would reach the kernels as a bad
    address or misread data.  An int passes through as an address, None as
    NULL (the library's own checks then apply)."""
    if x is None or isinstance(x, int):
        return x
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor, an int address or None, got {type(x)}")
    if not x.is_cuda:
        raise ValueError(f"{name}: expected a device tensor, got one on {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype}, expected {dtype}")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int):
    if status != 0:
        raise OombError(status, _L.oomb_status_string(status).decode())


def oomb_status_string(status: int) -> str:
    return _L.oomb_status_string(status).decode()


def oomb_abi_version() -> int:
    return _L.oomb_abi_version()


def oomb_rep_update(desc, k_pool, page_table, first_page, n_pages, rep, stream=None):
    io = _IO_DTYPE.get(desc.dtype)
    _check(_L.oomb_rep_update(ctypes.byref(desc), _dev(k_pool, io, "k_pool"), _dev(page_table, torch.int32, "page_table"),
                              first_page, n_pages, _dev(rep, torch.float32, "rep"), _stream(stream)))


def oomb_select_workspace_bytes(desc) -> int:
    return _L.oomb_select_workspace_bytes(ctypes.byref(desc))


def oomb_select_topk(desc, q, rep, sel, scores_out, workspace, workspace_bytes=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    io = _IO_DTYPE.get(desc.dtype)
    _check(_L.oomb_select_topk(ctypes.byref(desc), _dev(q, io, "q"), _dev(rep, torch.float32, "rep"),
                               _dev(sel, torch.int32, "sel"), _dev(scores_out, torch.float32, "scores_out"),
                               _dev(workspace, None, "workspace"), nbytes, _stream(stream)))


def oomb_select_topk_noalloc(desc, q, rep, sel, scores_out=None, stream=None):
    """oomb_select_topk on the library's own per-device scratch: no workspace
    argument, and nothing is allocated here either (see include/oomb.h)."""
    io = _IO_DTYPE.get(desc.dtype)
    _check(_L.oomb_select_topk_noalloc(ctypes.byref(desc), _dev(q, io, "q"), _dev(rep, torch.float32, "rep"),
                                       _dev(sel, torch.int32, "sel"), _dev(scores_out, torch.float32, "scores_out"),
                                       _stream(stream)))


def oomb_attn_fwd(desc, q, k_pool, v_pool, page_table, sel, o, lse, stream=None):
    io = _IO_DTYPE.get(desc.dtype)
    _check(_L.oomb_attn_fwd(ctypes.byref(desc), _dev(q, io, "q"), _dev(k_pool, io, "k_pool"), _dev(v_pool, io, "v_pool"),
                            _dev(page_table, torch.int32, "page_table"), _dev(sel, torch.int32, "sel"),
                            _dev(o, io, "o"), _dev(lse, torch.float32, "lse"), _stream(stream)))


def oomb_bwd_workspace_bytes(desc) -> int:
    return _L.oomb_bwd_workspace_bytes(ctypes.byref(desc))


def oomb_attn_bwd(desc, q, k_pool, v_pool, page_table, sel, o, lse, dO, dq, dk_pool, dv_pool, workspace,
                  workspace_bytes=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    io = _IO_DTYPE.get(desc.dtype)
    f32, i32 = torch.float32, torch.int32
    _check(_L.oomb_attn_bwd(ctypes.byref(desc), _dev(q, io, "q"), _dev(k_pool, io, "k_pool"), _dev(v_pool, io, "v_pool"),
                            _dev(page_table, i32, "page_table"), _dev(sel, i32, "sel"), _dev(o, io, "o"),
                            _dev(lse, f32, "lse"), _dev(dO, io, "dO"), _dev(dq, f32, "dq"),
                            _dev(dk_pool, f32, "dk_pool"), _dev(dv_pool, f32, "dv_pool"),
                            _dev(workspace, None, "workspace"), nbytes, _stream(stream)))


def oomb_check_workspace_bytes(desc) -> int:
    return _L.oomb_check_workspace_bytes(ctypes.byref(desc))


def oomb_check_tables(desc, page_table, sel, counts, workspace, workspace_bytes=None, stream=None):
    """counts: int32 [4] device tensor (see include/oomb.h)."""
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    i32 = torch.int32
    _check(_L.oomb_check_tables(ctypes.byref(desc), _dev(page_table, i32, "page_table"), _dev(sel, i32, "sel"),
                                _dev(counts, i32, "counts"), _dev(workspace, None, "workspace"), nbytes,
                                _stream(stream)))


def oomb_probe_mfma_peak(n_blocks, iters, out, stream=None):
    """Measurement helper: out is a float32 device tensor of n_blocks * 4 (see include/oomb.h)."""
    _check(_L.oomb_probe_mfma_peak(n_blocks, iters, _ptr(out), _stream(stream)))


def oomb_rmsnorm_fwd(x, gain, eps, h, rstd, stream=None):
    """x fp32 [rows][hidden], gain bf16 [hidden] -> h bf16, rstd fp32 [rows]."""
    rows, hidden = x.shape
    _check(_L.oomb_rmsnorm_fwd(_ptr(x), _ptr(gain), rows, hidden, eps, _ptr(h), _ptr(rstd), _stream(stream)))


def oomb_rmsnorm_bwd(x, gain, rstd, dh, dres, dx, stream=None):
    rows, hidden = x.shape
    _check(_L.oomb_rmsnorm_bwd(_ptr(x), _ptr(gain), _ptr(rstd), _ptr(dh), _ptr(dres), rows, hidden, _ptr(dx),
                               _stream(stream)))


def oomb_rmsnorm_gain_grad(x, rstd, dh, partial, stream=None):
    """partial: fp32 [segments][hidden]."""
    rows, hidden = x.shape
    _check(_L.oomb_rmsnorm_gain_grad(_ptr(x), _ptr(rstd), _ptr(dh), rows, hidden, partial.shape[0], _ptr(partial),
                                     _stream(stream)))


def oomb_rotary(x, out, cos_table, sin_table, first_position, inverse=False, stream=None):
    """x fp32 or bf16 [rows][heads][D] -> out bf16 of the same shape."""
    rows, heads, d = x.shape
    dt = 0 if x.dtype == torch.float32 else 1
    _check(_L.oomb_rotary(_ptr(x), dt, _ptr(out), _ptr(cos_table), _ptr(sin_table), rows, heads, d, first_position,
                          1 if inverse else 0, _stream(stream)))


def oomb_swiglu_fwd(gate, up, out, stream=None):
    _check(_L.oomb_swiglu_fwd(_ptr(gate), _ptr(up), _ptr(out), gate.numel(), _stream(stream)))


def oomb_swiglu_bwd(gate, up, dout, dgate, dup, stream=None):
    _check(_L.oomb_swiglu_bwd(_ptr(gate), _ptr(up), _ptr(dout), _ptr(dgate), _ptr(dup), gate.numel(),
                              _stream(stream)))


def oomb_host_view(host) -> int:
    """Device address of pinned host memory (a pinned CPU tensor or an int address)."""
    if isinstance(host, torch.Tensor) and (host.is_cuda or not host.is_pinned()):
        raise ValueError("oomb_host_view needs a pinned CPU tensor")
    out = ctypes.c_void_p()
    _check(_L.oomb_host_view(_ptr(host), ctypes.byref(out)))
    return out.value


def oomb_stage_desc(desc) -> oomb_desc:
    staged = oomb_desc()
    _check(_L.oomb_stage_desc(ctypes.byref(desc), ctypes.byref(staged)))
    return staged


def oomb_stage_tables(desc, sel_stage, pt_stage, stream=None):
    _check(_L.oomb_stage_tables(ctypes.byref(desc), _ptr(sel_stage), _ptr(pt_stage), _stream(stream)))


def oomb_stage_gather(desc, src_k, src_v, page_table, sel, parts, stage_k, stage_v, src_slots=None, first_page=0,
                      n_pages=None, stream=None):
    """src_k / src_v: device views (oomb_host_view) of the host pools, or device
    pools; src_slots defaults to the descriptor's n_slots, the page range to
    every prior page."""
    _check(_L.oomb_stage_gather(ctypes.byref(desc), _ptr(src_k), _ptr(src_v),
                                desc.n_slots if src_slots is None else src_slots, _ptr(page_table), _ptr(sel), parts,
                                first_page, desc.n_prior_pages if n_pages is None else n_pages, _ptr(stage_k),
                                _ptr(stage_v), _stream(stream)))


def oomb_stage_offload_chunk(desc, stage_k, stage_v, page_table, host_k, host_v, stream=None):
    _check(_L.oomb_stage_offload_chunk(ctypes.byref(desc), _ptr(stage_k), _ptr(stage_v), _ptr(page_table),
                                       _ptr(host_k), _ptr(host_v), _stream(stream)))


def oomb_stage_flush_grads(desc, stage_dk, stage_dv, page_table, sel, host_dk, host_dv, stream=None):
    _check(_L.oomb_stage_flush_grads(ctypes.byref(desc), _ptr(stage_dk), _ptr(stage_dv), _ptr(page_table), _ptr(sel),
                                     _ptr(host_dk), _ptr(host_dv), _stream(stream)))


def oomb_stage_grads_out(desc, stage_dk, stage_dv, out_dk, out_dv, stream=None):
    """out_dk / out_dv: device views (oomb_host_view) of pinned host buffers, or device buffers."""
    _check(_L.oomb_stage_grads_out(ctypes.byref(desc), _ptr(stage_dk), _ptr(stage_dv), _ptr(out_dk), _ptr(out_dv),
                                   _stream(stream)))


def oomb_host_accumulate_grads(desc, delta_dk, delta_dv, page_table, sel, host_dk, host_dv, n_threads=8):
    """Every argument is host memory (CPU tensors); returns when done.  The GIL
    is released during the call."""
    for t in (delta_dk, delta_dv, page_table, sel, host_dk, host_dv):
        if isinstance(t, torch.Tensor) and t.is_cuda:
            raise ValueError("oomb_host_accumulate_grads takes host tensors")
    _check(_L.oomb_host_accumulate_grads(ctypes.byref(desc), _ptr(delta_dk), _ptr(delta_dv), _ptr(page_table),
                                         _ptr(sel), _ptr(host_dk), _ptr(host_dv), n_threads))


def oomb_trace_events(events, capacity=None):
    """Start tracing into a ctypes array of hipEvent_t handles (None stops it)."""
    if events is None:
        _check(_L.oomb_trace_events(None, 0))
        return
    _check(_L.oomb_trace_events(ctypes.cast(events, ctypes.c_void_p), len(events) if capacity is None else capacity))


def oomb_trace_only(kernel):
    """Record only the launches of the named kernel (None: every launch)."""
    _check(_L.oomb_trace_only(None if kernel is None else kernel.encode()))


def oomb_trace_count() -> int:
    return _L.oomb_trace_count()


def oomb_trace_kernel(i: int):
    name = _L.oomb_trace_kernel(i)
    return name.decode() if name is not None else None
