"""Chunk-recurrent attention of one layer over a whole sequence, on the device.

The OOMB page's training scheme (technical summary, section 2: chunk-recurrent
training over a paged KV cache with page-level sparse attention) processes a
long sequence in chunks of C tokens.  In the forward pass chunk i picks, per
kv-head, the top-K pages among all earlier pages (an optional initial context,
then chunks 0 .. i-1), attends to them and causally to itself, and its own
pages then get their representative vectors so that later chunks can score
them.  The backward pass visits the chunks in reverse order; each reuses its
forward page selection, O and log-sum-exp, and adds its dK/dV contributions in
place into the gradient pools that all chunks share.

Layout: the sequence's K/V live in pools of page slots reached through one page
table; logical page m of the sequence is slot page_table[m], the initial
context takes logical pages 0 .. n0-1 and chunk i takes pages
n0 + i*C/ps .. n0 + (i+1)*C/ps - 1.  Q, O and dO are [chunks][C][Hq][D].

Marshalling only: every step runs in the library's kernels.
"""
from __future__ import annotations

import torch

from . import (make_desc, oomb_attn_bwd, oomb_attn_fwd, oomb_bwd_workspace_bytes, oomb_rep_update,
               oomb_select_topk, oomb_select_workspace_bytes)
from .step import TORCH_DTYPE


class ChunkedSequence:
    def __init__(self, n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, n_chunks, top_k,
                 n_initial_pages=0, n_slots=None, dtype="bf16", softmax_scale=0.0, device="cuda",
                 keep_activations=True):
        if chunk_len % page_size:
            raise ValueError("chunk_len must be a multiple of page_size")
        self.hq, self.hkv, self.d, self.ps, self.c = n_q_heads, n_kv_heads, head_dim, page_size, chunk_len
        self.n_chunks, self.top_k, self.n0, self.dtype = n_chunks, top_k, n_initial_pages, dtype
        self.keep_activations = keep_activations
        self.chunk_pages = chunk_len // page_size
        self.total_pages = n_initial_pages + n_chunks * self.chunk_pages
        self.n_slots = self.total_pages if n_slots is None else n_slots
        # chunk i: n_initial_pages + i * chunk_pages prior pages
        self.descs = [make_desc(n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, self.prior_pages(i), top_k,
                                self.n_slots, rep_capacity=self.total_pages, dtype=dtype,
                                softmax_scale=softmax_scale)
                      for i in range(n_chunks)]
        f32 = dict(dtype=torch.float32, device=device)
        self.rep = torch.zeros((self.total_pages, n_kv_heads, head_dim), **f32)
        self.sel = [torch.zeros((n_kv_heads, max(self.keff(i), 1)), dtype=torch.int32, device=device)
                    for i in range(n_chunks)]
        n_act = n_chunks if keep_activations else 1
        self.o = torch.empty((n_act, chunk_len, n_q_heads, head_dim), dtype=TORCH_DTYPE[dtype], device=device)
        self.lse = torch.empty((n_act, n_q_heads, chunk_len), **f32)
        self.dq = torch.empty((n_chunks, chunk_len, n_q_heads, head_dim), **f32)
        ws_sel = max(oomb_select_workspace_bytes(d) for d in self.descs)
        ws_bwd = max(oomb_bwd_workspace_bytes(d) for d in self.descs)
        self.ws_select = torch.empty(max(ws_sel, 256), dtype=torch.uint8, device=device)
        self.ws_bwd = torch.empty(max(ws_bwd, 256), dtype=torch.uint8, device=device)

    def prior_pages(self, i):
        return self.n0 + i * self.chunk_pages

    def keff(self, i):
        return max(0, min(self.top_k, self.prior_pages(i)))

    def _act(self, i):
        return i if self.keep_activations else 0

    def forward(self, q, k_pool, v_pool, page_table, stream=None, on_chunk=None):
        """Chunks in order: select among the earlier pages, attend, then give the
        chunk's pages their representative vectors.  on_chunk(i, O, LSE), if
        given, is called after chunk i's forward is enqueued (with one activation
        buffer, that chunk's O and LSE are overwritten by the next chunk).
        Returns (O, LSE)."""
        if self.n0 > 0:
            oomb_rep_update(self.descs[0], k_pool, page_table, 0, self.n0, self.rep, stream=stream)
        for i, desc in enumerate(self.descs):
            a = self._act(i)
            oomb_select_topk(desc, q[i], self.rep, self.sel[i], None, self.ws_select, stream=stream)
            oomb_attn_fwd(desc, q[i], k_pool, v_pool, page_table, self.sel[i], self.o[a], self.lse[a],
                          stream=stream)
            if on_chunk is not None:
                on_chunk(i, self.o[a], self.lse[a])
            oomb_rep_update(desc, k_pool, page_table, self.prior_pages(i), self.chunk_pages, self.rep,
                            stream=stream)
        return self.o, self.lse

    def backward(self, q, k_pool, v_pool, page_table, dO, dk_pool, dv_pool, stream=None):
        """Chunks in reverse order with their forward selections; dK/dV are added
        into the pools in place.  Without kept activations each chunk's forward
        is re-run first, with its saved selection.  Returns dQ."""
        for i in reversed(range(self.n_chunks)):
            a = self._act(i)
            if not self.keep_activations:
                oomb_attn_fwd(self.descs[i], q[i], k_pool, v_pool, page_table, self.sel[i], self.o[a],
                              self.lse[a], stream=stream)
            oomb_attn_bwd(self.descs[i], q[i], k_pool, v_pool, page_table, self.sel[i], self.o[a], self.lse[a],
                          dO[i], self.dq[i], dk_pool, dv_pool, self.ws_bwd, stream=stream)
        return self.dq
