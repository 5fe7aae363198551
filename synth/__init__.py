"""Seeded synthetic inputs for paged top-K chunk attention.

This module only draws numbers (see ``synth.c``); it holds none of the
attention method's arithmetic.  Both the HIP path's tests/benchmark and the CPU
oracle take their inputs from here, so the two see identical bits.

Workloads follow the shapes of the OOMB page ("Out of the Memory Barrier",
technical summary, section 2 and section 4): a Qwen2.5-7B-shaped attention
layer (28 query heads, 4 kv heads, head dim 128), 128-token pages, a chunk of
4096 or 8192 tokens attending to the top-K pages of 32K..4M tokens of prior
context, plus one tiny fp32 case.  Q, K, V and dO are N(0, 1); every (page,
kv-head) gets one N(0, 0.5) offset vector (standard deviation 0.5) added to all
of its keys so that page scores are well separated; the page table is a seeded
random permutation of the physical slots.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")

DTYPES = {"f32": 0, "bf16": 1, "f64": 2}
NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}

# stream ids of the counter-based generator
S_Q, S_K, S_V, S_DO, S_KOFF, S_PERM, S_DK0, S_DV0 = 1, 2, 3, 4, 5, 6, 7, 8


def build(force: bool = False) -> str:
    """Compile synth.c with gcc into libsynth.so (plain host code)."""
    src = os.path.join(HERE, "synth.c")
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(src):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               "-std=c11", src, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        L.synth_u64.restype = ctypes.c_uint64
        L.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        L.synth_normal.restype = ctypes.c_double
        L.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        L.synth_round_bf16.restype = ctypes.c_uint16
        L.synth_round_bf16.argtypes = [ctypes.c_double]
        L.synth_tensor.restype = None
        L.synth_tensor.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        L.synth_pool.restype = None
        L.synth_pool.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_double,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_int,
                                 ctypes.c_void_p]
        L.synth_permutation.restype = None
        L.synth_permutation.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p]
        _lib = L
    return _lib


@dataclasses.dataclass(frozen=True)
class Problem:
    """Shape of one chunk step.  n = prior pages, k = top-K, c = chunk tokens."""
    hq: int
    hkv: int
    d: int
    ps: int
    c: int
    n: int
    k: int
    dtype: str = "bf16"
    n_slots: int = 0          # 0 -> n + c // ps
    scale: float = 0.0        # 0 -> 1/sqrt(d)

    @property
    def slots(self) -> int:
        return self.n_slots if self.n_slots else self.n + self.c // self.ps

    @property
    def chunk_pages(self) -> int:
        return self.c // self.ps

    @property
    def keff(self) -> int:
        return max(0, min(self.k, self.n))

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def pairs(self) -> int:
        """Visible (query-head row, key) pairs of one step."""
        return self.hq * (self.c * self.keff * self.ps + self.c * (self.c + 1) // 2)


# The five workloads (shapes of the OOMB page's Qwen2.5-7B long-context runs),
# by name; the number is the default seed.
WORKLOADS = {
    "tiny-fp32": (1, Problem(hq=4, hkv=2, d=64, ps=16, c=64, n=64, k=8, dtype="f32")),
    "dense-32k": (2, Problem(hq=28, hkv=4, d=128, ps=128, c=4096, n=256, k=256)),
    "sparse-256k": (3, Problem(hq=28, hkv=4, d=128, ps=128, c=4096, n=2048, k=64)),
    "sparse-1m": (4, Problem(hq=28, hkv=4, d=128, ps=128, c=8192, n=8192, k=64)),
    "sparse-4m": (5, Problem(hq=28, hkv=4, d=128, ps=128, c=8192, n=32768, k=128)),
}


def tensor(seed: int, stream: int, shape, dtype: str, scale: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=NP_STORAGE[dtype])
    lib().synth_tensor(seed, stream, start, out.size, scale, DTYPES[dtype], out.ctypes.data)
    return out


def normals(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    return tensor(seed, stream, (count,), "f64", 1.0, start)


def page_table(p: Problem, seed: int) -> np.ndarray:
    perm = np.empty(p.slots, dtype=np.int32)
    lib().synth_permutation(seed, S_PERM, p.slots, perm.ctypes.data)
    return np.ascontiguousarray(perm[: p.n + p.chunk_pages])


def pool(p: Problem, seed: int, which: str, pt: np.ndarray, fill: float = 64.0) -> np.ndarray:
    """K or V pool [slots][hkv][ps][d]; K carries the per-page 0.5*N(0,1) offsets."""
    out = np.empty((p.slots, p.hkv, p.ps, p.d), dtype=NP_STORAGE[p.dtype])
    stream, off = (S_K, 0.5) if which == "k" else (S_V, 0.0)
    lib().synth_pool(seed, stream, S_KOFF, off, p.n + p.chunk_pages, p.hkv, p.ps, p.d,
                     pt.ctypes.data, p.slots, fill, DTYPES[p.dtype], out.ctypes.data)
    return out


def make_inputs(p: Problem, seed: int) -> dict:
    """All inputs of one chunk step as host arrays (bf16 stored as uint16 bits)."""
    pt = page_table(p, seed)
    return {
        "page_table": pt,
        "q": tensor(seed, S_Q, (p.c, p.hq, p.d), p.dtype),
        "k_pool": pool(p, seed, "k", pt),
        "v_pool": pool(p, seed, "v", pt),
        "do": tensor(seed, S_DO, (p.c, p.hq, p.d), p.dtype),
    }


@dataclasses.dataclass(frozen=True)
class Sequence:
    """A whole sequence of one layer processed chunk by chunk: n0 initial pages
    of context, then `chunks` chunks of c tokens; chunk i has n0 + i*c/ps prior
    pages.  The pools hold every page of the sequence."""
    hq: int
    hkv: int
    d: int
    ps: int
    c: int
    chunks: int
    k: int
    n0: int = 0
    dtype: str = "bf16"
    scale: float = 0.0

    @property
    def chunk_pages(self) -> int:
        return self.c // self.ps

    @property
    def pages(self) -> int:
        return self.n0 + self.chunks * self.chunk_pages

    def step(self, i: int) -> Problem:
        """The chunk step of chunk i (its pools span the whole sequence)."""
        return Problem(self.hq, self.hkv, self.d, self.ps, self.c, self.n0 + i * self.chunk_pages, self.k,
                       self.dtype, n_slots=self.pages, scale=self.scale)

    def pairs(self) -> int:
        return sum(self.step(i).pairs() for i in range(self.chunks))


# Whole sequences of the Qwen2.5-7B attention shape, chunk by chunk (name -> (seed, Sequence)).
SEQUENCES = {
    "seq-64k": (6, Sequence(hq=28, hkv=4, d=128, ps=128, c=4096, chunks=16, k=64)),
    "seq-256k": (7, Sequence(hq=28, hkv=4, d=128, ps=128, c=4096, chunks=64, k=64)),
}


def make_sequence_inputs(s: Sequence, seed: int) -> dict:
    """Inputs of a whole sequence: pools and page table of every page, and
    Q / dO of every chunk ([chunks][c][hq][d])."""
    last = s.step(s.chunks - 1)
    pt = page_table(last, seed)
    return {
        "page_table": pt,
        "q": tensor(seed, S_Q, (s.chunks, s.c, s.hq, s.d), s.dtype),
        "k_pool": pool(last, seed, "k", pt),
        "v_pool": pool(last, seed, "v", pt),
        "do": tensor(seed, S_DO, (s.chunks, s.c, s.hq, s.d), s.dtype),
    }


def canary(p: Problem, seed: int, which: str) -> np.ndarray:
    """Seeded fp32 prefill for a gradient pool (so untouched slots can be checked)."""
    return tensor(seed, S_DK0 if which == "k" else S_DV0, (p.slots, p.hkv, p.ps, p.d), "f32")


def widen_bf16(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> float32 values (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def as_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64 (exact widening)."""
    if dtype == "bf16":
        return widen_bf16(a).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# A decoder layer around the attention path (Qwen2-style block: RMSNorm,
# QKV projections with bias, rotary positions, output projection, RMSNorm,
# SwiGLU MLP).  Only its seeded inputs live here: weights, layer input and
# output gradient, all bf16.
# ---------------------------------------------------------------------------
S_LAYER = 40  # stream ids S_LAYER + i for the tensors of LAYER_TENSORS


@dataclasses.dataclass(frozen=True)
class Layer:
    hidden: int
    hq: int
    hkv: int
    d: int
    inter: int
    ps: int
    c: int
    chunks: int
    k: int
    rope_theta: float = 1.0e6
    eps: float = 1.0e-6

    @property
    def chunk_pages(self) -> int:
        return self.c // self.ps

    @property
    def pages(self) -> int:
        return self.chunks * self.chunk_pages

    @property
    def tokens(self) -> int:
        return self.chunks * self.c


def layer_tensors(s: Layer) -> dict:
    """name -> (shape, kind): 'w' weight N(0,1)/sqrt(fan in), 'b' bias
    0.1*N(0,1), 'g' norm gain 1 + 0.1*N(0,1), 'x' activation N(0,1)."""
    qd, kd = s.hq * s.d, s.hkv * s.d
    return {
        "ln1": ((s.hidden,), "g"), "wq": ((s.hidden, qd), "w"), "bq": ((qd,), "b"),
        "wk": ((s.hidden, kd), "w"), "bk": ((kd,), "b"), "wv": ((s.hidden, kd), "w"), "bv": ((kd,), "b"),
        "wo": ((qd, s.hidden), "w"), "ln2": ((s.hidden,), "g"), "wg": ((s.hidden, s.inter), "w"),
        "wu": ((s.hidden, s.inter), "w"), "wd": ((s.inter, s.hidden), "w"),
        "x": ((s.tokens, s.hidden), "x"), "dy": ((s.tokens, s.hidden), "x"),
    }


def make_layer_inputs(s: Layer, seed: int) -> dict:
    """bf16 bits (uint16) of every weight, of the layer input x [tokens][hidden]
    and of the output gradient dy [tokens][hidden]."""
    out = {}
    for i, (name, (shape, kind)) in enumerate(layer_tensors(s).items()):
        if kind == "g":
            g = 1.0 + 0.1 * normals(seed, S_LAYER + i, int(np.prod(shape)))
            out[name] = bf16_bits(g.reshape(shape))
        else:
            scale = {"w": 1.0 / np.sqrt(shape[0]), "b": 0.1, "x": 1.0}[kind]
            out[name] = tensor(seed, S_LAYER + i, shape, "bf16", scale)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# name -> (seed, Layer)
LAYERS = {
    "layer-tiny": (11, Layer(hidden=256, hq=4, hkv=2, d=64, inter=512, ps=16, c=64, chunks=4, k=2)),
    "layer-tiny-d128": (13, Layer(hidden=256, hq=2, hkv=1, d=128, inter=384, ps=32, c=64, chunks=5, k=3)),
    "layer-qwen-64k": (12, Layer(hidden=3584, hq=28, hkv=4, d=128, inter=18944, ps=128, c=4096, chunks=16, k=64)),
    "layer-qwen-256k": (14, Layer(hidden=3584, hq=28, hkv=4, d=128, inter=18944, ps=128, c=4096, chunks=64, k=64)),
}
