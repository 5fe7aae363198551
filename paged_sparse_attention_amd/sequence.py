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
                 keep_activations=True, overlap_recompute=True):
        if chunk_len % page_size:
            raise ValueError("chunk_len must be a multiple of page_size")
        self.hq, self.hkv, self.d, self.ps, self.c = n_q_heads, n_kv_heads, head_dim, page_size, chunk_len
        self.n_chunks, self.top_k, self.n0, self.dtype = n_chunks, top_k, n_initial_pages, dtype
        self.keep_activations = keep_activations
        # re-run forwards overlap the backward of the chunk after them (two activation buffers)
        self.overlap = overlap_recompute and not keep_activations and n_chunks > 1
        self._side = None
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
        n_act = n_chunks if keep_activations else (2 if self.overlap else 1)
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
        if self.keep_activations:
            return i
        return i % 2 if self.overlap else 0

    def forward(self, q, k_pool, v_pool, page_table, stream=None, on_chunk=None):
        """Chunks in order: select among the earlier pages, attend, then give the
        chunk's pages their representative vectors.  on_chunk(i, O, LSE), if
        given, is called after chunk i's forward is enqueued (without kept
        activations, that chunk's O and LSE are overwritten by a later chunk).
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
        is re-run first, with its saved selection.  Returns dQ.

        With re-run forwards and overlap_recompute, chunk i-1's forward runs on
        a second stream while chunk i's backward runs on `stream`: the two are
        independent (the forward reads the K/V pools, the backward writes only
        dQ and the gradient pools), and the workgroups of one fill the compute
        units that the other's last round leaves idle.  The activation buffers
        alternate, and events order each forward after the backward that last
        read its buffer and before the backward that reads it.  The same
        kernels run on the same inputs, so the results are bitwise those of
        the serial order."""
        if self.overlap:
            return self._backward_overlapped(q, k_pool, v_pool, page_table, dO, dk_pool, dv_pool, stream)
        for i in reversed(range(self.n_chunks)):
            a = self._act(i)
            if not self.keep_activations:
                oomb_attn_fwd(self.descs[i], q[i], k_pool, v_pool, page_table, self.sel[i], self.o[a],
                              self.lse[a], stream=stream)
            oomb_attn_bwd(self.descs[i], q[i], k_pool, v_pool, page_table, self.sel[i], self.o[a], self.lse[a],
                          dO[i], self.dq[i], dk_pool, dv_pool, self.ws_bwd, stream=stream)
        return self.dq

    def _backward_overlapped(self, q, k_pool, v_pool, page_table, dO, dk_pool, dv_pool, stream):
        main = stream if stream is not None else torch.cuda.current_stream()
        if not isinstance(main, torch.cuda.Stream):
            main = torch.cuda.ExternalStream(int(main))
        if self._side is None:
            self._side = torch.cuda.Stream(device=main.device)
        side = self._side
        n = self.n_chunks
        fwd_done = [torch.cuda.Event() for _ in range(n)]
        bwd_done = [torch.cuda.Event() for _ in range(n)]

        def fwd(i):
            a = self._act(i)
            oomb_attn_fwd(self.descs[i], q[i], k_pool, v_pool, page_table, self.sel[i], self.o[a], self.lse[a],
                          stream=side)
            fwd_done[i].record(side)

        side.wait_stream(main)
        fwd(n - 1)
        for i in reversed(range(n)):
            if i > 0:
                if i + 1 < n:
                    side.wait_event(bwd_done[i + 1])   # chunk i+1's backward read the buffer of chunk i-1
                fwd(i - 1)
            main.wait_event(fwd_done[i])
            a = self._act(i)
            oomb_attn_bwd(self.descs[i], q[i], k_pool, v_pool, page_table, self.sel[i], self.o[a], self.lse[a],
                          dO[i], self.dq[i], dk_pool, dv_pool, self.ws_bwd, stream=main)
            bwd_done[i].record(main)
        return self.dq
