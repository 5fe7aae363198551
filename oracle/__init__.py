"""ctypes binding of the fp64 CPU oracle (oomb_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP library (paged_sparse_attention_amd) and never imports it.

Method: page "Out of the Memory Barrier" (OOMB), technical summary, section 2
(Methodology), "Paged Memory Management" and "Page-level Sparse Attention".
The readings the oracle takes are listed in oomb_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oomb_oracle.c")
LIB = os.path.join(HERE, "liboomb_oracle.so")

_DT = {"f32": 0, "bf16": 1, "f64": 2}
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}


def build(src: str = SRC, out: str = LIB, force: bool = False) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no FMA contraction, no fast-math."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < max(
            os.path.getmtime(src), os.path.getmtime(os.path.join(HERE, "oomb_oracle.h"))):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               "-std=c11", "-I", HERE, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Shape(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("ps", ctypes.c_int32), ("c", ctypes.c_int32), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_double)]


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


class Oracle:
    """fp64 oracle.  `p` is a synth.Problem-like object (hq, hkv, d, ps, c, n, k,
    slots, dtype, scale).  Arrays are numpy in the layouts of oomb_oracle.h."""

    def __init__(self, lib_path: str | None = None):
        path = lib_path or LIB
        if lib_path is None and not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.POINTER(_Shape)
        vp = ctypes.c_void_p
        L.ora_keff.restype = ctypes.c_int32
        L.ora_keff.argtypes = [P]
        L.ora_nkeys.restype = ctypes.c_int64
        L.ora_nkeys.argtypes = [P]
        L.ora_rep.restype = None
        L.ora_rep.argtypes = [P, vp, vp, ctypes.c_int32, ctypes.c_int32, vp]
        L.ora_qmean.restype = None
        L.ora_qmean.argtypes = [P, vp, vp]
        L.ora_scores.restype = None
        L.ora_scores.argtypes = [P, vp, vp, vp]
        L.ora_select.restype = ctypes.c_int32
        L.ora_select.argtypes = [P, vp, vp]
        L.ora_fwd.restype = None
        L.ora_fwd.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int64, vp, vp, vp]
        L.ora_bwd.restype = None
        L.ora_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp, vp, vp, vp]
        L.ora_threads.restype = ctypes.c_int
        L.ora_threads.argtypes = []
        L.ora_key_offset.restype = ctypes.c_int64
        L.ora_key_offset.argtypes = [P, vp, vp, ctypes.c_int32, ctypes.c_int64]
        self.L = L

    def threads(self) -> int:
        return self.L.ora_threads()

    @staticmethod
    def shape(p, dtype: str | None = None) -> _Shape:
        return _Shape(p.hq, p.hkv, p.d, p.ps, p.c, p.n, p.k, p.slots, _DT[dtype or p.dtype],
                      float(p.scale))

    def _check(self, a, dtype):
        a = np.ascontiguousarray(a)
        assert a.dtype == _STORAGE[dtype], (a.dtype, dtype)
        return a

    # --- selection -------------------------------------------------------
    def rep(self, p, k_pool, page_table, first=0, count=None, dtype=None):
        dtype = dtype or p.dtype
        count = p.n if count is None else count
        k_pool = self._check(k_pool, dtype)
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        out = np.zeros((count, p.hkv, p.d), dtype=np.float64)
        s = self.shape(p, dtype)
        self.L.ora_rep(ctypes.byref(s), _ptr(k_pool), _ptr(pt), first, count, _ptr(out))
        return out

    def qmean(self, p, q, dtype=None):
        dtype = dtype or p.dtype
        q = self._check(q, dtype)
        out = np.zeros((p.hkv, p.d), dtype=np.float64)
        s = self.shape(p, dtype)
        self.L.ora_qmean(ctypes.byref(s), _ptr(q), _ptr(out))
        return out

    def scores(self, p, qbar, rep):
        qbar = np.ascontiguousarray(qbar, dtype=np.float64)
        rep = np.ascontiguousarray(rep, dtype=np.float64)
        assert rep.shape[0] >= p.n
        out = np.zeros((p.hkv, p.n), dtype=np.float64)
        s = self.shape(p)
        self.L.ora_scores(ctypes.byref(s), _ptr(qbar), _ptr(rep), _ptr(out))
        return out

    def select(self, p, scores):
        scores = np.ascontiguousarray(scores, dtype=np.float64)
        keff = max(0, min(p.k, p.n))
        out = np.zeros((p.hkv, max(keff, 1)), dtype=np.int32)
        s = self.shape(p)
        self.L.ora_select(ctypes.byref(s), _ptr(scores), _ptr(out))
        return out[:, :keff].copy()

    def selection(self, p, q, k_pool, page_table, dtype=None):
        """rep -> chunk-mean query -> scores -> top-K.  Returns (sel, scores)."""
        rep = self.rep(p, k_pool, page_table, 0, p.n, dtype)
        sc = self.scores(p, self.qmean(p, q, dtype), rep)
        return self.select(p, sc), sc

    # --- attention -------------------------------------------------------
    def all_rows(self, p):
        return np.arange(p.c * p.hq, dtype=np.int64)

    def fwd(self, p, q, k_pool, v_pool, page_table, sel, rows=None, dtype=None):
        dtype = dtype or p.dtype
        rows = self.all_rows(p) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        q, k_pool, v_pool = (self._check(a, dtype) for a in (q, k_pool, v_pool))
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        o = np.zeros((len(rows), p.d), dtype=np.float64)
        lse = np.zeros(len(rows), dtype=np.float64)
        s = self.shape(p, dtype)
        self.L.ora_fwd(ctypes.byref(s), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(pt), _ptr(sel),
                       len(rows), _ptr(rows), _ptr(o), _ptr(lse))
        return o, lse

    def bwd(self, p, q, k_pool, v_pool, page_table, sel, dout, rows=None, dkdv=True, dtype=None):
        """Returns dq [nrows][d], dk, dv [hkv][nkeys][d] (None if dkdv is False)."""
        dtype = dtype or p.dtype
        rows = self.all_rows(p) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        q, k_pool, v_pool, dout = (self._check(a, dtype) for a in (q, k_pool, v_pool, dout))
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        s = self.shape(p, dtype)
        nkeys = self.L.ora_nkeys(ctypes.byref(s))
        dq = np.zeros((len(rows), p.d), dtype=np.float64)
        dk = np.zeros((p.hkv, nkeys, p.d), dtype=np.float64) if dkdv else None
        dv = np.zeros((p.hkv, nkeys, p.d), dtype=np.float64) if dkdv else None
        self.L.ora_bwd(ctypes.byref(s), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(pt), _ptr(sel),
                       _ptr(dout), len(rows), _ptr(rows), _ptr(dq), _ptr(dk), _ptr(dv))
        return dq, dk, dv

    def key_slots(self, p, page_table, sel):
        """Pool (slot, row) of every key jj of J(h), as two int64 arrays [hkv][nkeys]."""
        keff = max(0, min(p.k, p.n))
        pk = keff * p.ps
        nkeys = pk + p.c
        sel = np.asarray(sel, dtype=np.int64).reshape(p.hkv, keff)
        pt = np.asarray(page_table, dtype=np.int64)
        jj = np.arange(nkeys)
        slot = np.zeros((p.hkv, nkeys), dtype=np.int64)
        row = np.zeros((p.hkv, nkeys), dtype=np.int64)
        for h in range(p.hkv):
            pages = np.empty(nkeys, dtype=np.int64)
            pages[:pk] = sel[h][jj[:pk] // p.ps]
            pages[pk:] = p.n + (jj[pk:] - pk) // p.ps
            slot[h] = pt[pages]
            row[h, :pk] = jj[:pk] % p.ps
            row[h, pk:] = (jj[pk:] - pk) % p.ps
        return slot, row

    # --- a whole sequence, chunk by chunk ------------------------------------
    def sequence(self, s, x, sels=None):
        """Chunk-recurrent attention of one layer over a whole sequence (the
        OOMB page, technical summary, section 2: chunk-recurrent training with
        page-level sparse attention over a paged KV cache).

        Forward, chunks in order: chunk i (a chunk step whose prior pages are the
        initial context and chunks 0 .. i-1) scores those pages by their
        representative vectors, takes its top-K, and attends.  Backward, chunks
        in reverse order: each chunk reuses its selection and adds its dK/dV
        into the pools shared by the whole sequence.  `s` is a synth.Sequence;
        `sels`, if given, replaces the chunks' own selections.

        Returns a dict: per chunk lists sel, scores, o [c*hq][d], lse [c*hq],
        dq [c*hq][d]; pool-shaped dk, dv [slots][hkv][ps][d] (the sums).
        """
        last = s.step(s.chunks - 1)
        pt = np.ascontiguousarray(x["page_table"], dtype=np.int32)
        # a page's representative vector depends only on its keys: those of all
        # pages at once, for the chunks to read their prior pages from
        rep = self.rep(last, x["k_pool"], pt, 0, s.pages)
        out = {"sel": [], "scores": [], "o": [], "lse": [], "dq": [None] * s.chunks}
        for i in range(s.chunks):
            p = s.step(i)
            q = np.ascontiguousarray(x["q"][i])
            sc = self.scores(p, self.qmean(p, q), rep[:p.n]) if p.n > 0 else np.zeros((p.hkv, 0))
            sel = self.select(p, sc) if sels is None else np.asarray(sels[i], dtype=np.int32).reshape(p.hkv, p.keff)
            o, lse = self.fwd(p, q, x["k_pool"], x["v_pool"], pt, sel)
            out["sel"].append(sel)
            out["scores"].append(sc)
            out["o"].append(o)
            out["lse"].append(lse)
        dk = np.zeros((last.slots, s.hkv, s.ps, s.d), dtype=np.float64)
        dv = np.zeros_like(dk)
        for i in reversed(range(s.chunks)):
            p = s.step(i)
            dq, dki, dvi = self.bwd(p, np.ascontiguousarray(x["q"][i]), x["k_pool"], x["v_pool"], pt, out["sel"][i],
                                    np.ascontiguousarray(x["do"][i]))
            slot, row = self.key_slots(p, pt, out["sel"][i])
            for h in range(p.hkv):
                np.add.at(dk, (slot[h], h, row[h]), dki[h])
                np.add.at(dv, (slot[h], h, row[h]), dvi[h])
            out["dq"][i] = dq
        out["dk"], out["dv"] = dk, dv
        return out
