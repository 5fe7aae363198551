"""One chunk step of paged top-K chunk attention on the device.

ChunkStep owns the per-step outputs and workspaces (torch tensors, allocated
once) and calls the four entry points of liboomb.so in the order of the OOMB
page's method (technical summary, section 2): refresh the representative
vectors of the chunk's new pages, pick the top-K prior pages per kv-head,
attend forward, then run the backward with the same pages, accumulating dK/dV
in place into the caller's paged gradient pools.  Marshalling only.
"""
from __future__ import annotations

import torch

from . import (make_desc, oomb_attn_bwd, oomb_attn_fwd, oomb_bwd_workspace_bytes, oomb_rep_update,
               oomb_select_topk, oomb_select_workspace_bytes)

TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


class ChunkStep:
    def __init__(self, n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, n_prior_pages, top_k, n_slots,
                 dtype="bf16", softmax_scale=0.0, device="cuda"):
        self.desc = make_desc(n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, n_prior_pages, top_k,
                              n_slots, dtype=dtype, softmax_scale=softmax_scale)
        self.hq, self.hkv, self.d, self.ps, self.c = n_q_heads, n_kv_heads, head_dim, page_size, chunk_len
        self.n, self.keff = n_prior_pages, max(0, min(top_k, n_prior_pages))
        self.chunk_pages = chunk_len // page_size
        f32 = dict(dtype=torch.float32, device=device)
        self.rep = torch.zeros((n_prior_pages + self.chunk_pages, n_kv_heads, head_dim), **f32)
        self.sel = torch.zeros((n_kv_heads, max(self.keff, 1)), dtype=torch.int32, device=device)
        self.scores = torch.zeros((n_kv_heads, max(n_prior_pages, 1)), **f32)
        self.o = torch.empty((chunk_len, n_q_heads, head_dim), dtype=TORCH_DTYPE[dtype], device=device)
        self.lse = torch.empty((n_q_heads, chunk_len), **f32)
        self.dq = torch.empty((chunk_len, n_q_heads, head_dim), **f32)
        self.ws_select = torch.empty(max(oomb_select_workspace_bytes(self.desc), 256), dtype=torch.uint8,
                                     device=device)
        self.ws_bwd = torch.empty(max(oomb_bwd_workspace_bytes(self.desc), 256), dtype=torch.uint8, device=device)

    def rep_update(self, k_pool, page_table, first_page, n_pages, stream=None):
        oomb_rep_update(self.desc, k_pool, page_table, first_page, n_pages, self.rep, stream=stream)

    def select(self, q, stream=None, keep_scores=True):
        oomb_select_topk(self.desc, q, self.rep, self.sel, self.scores if keep_scores else None, self.ws_select,
                         stream=stream)

    def fwd(self, q, k_pool, v_pool, page_table, stream=None):
        oomb_attn_fwd(self.desc, q, k_pool, v_pool, page_table, self.sel, self.o, self.lse, stream=stream)

    def bwd(self, q, k_pool, v_pool, page_table, dO, dk_pool, dv_pool, stream=None):
        oomb_attn_bwd(self.desc, q, k_pool, v_pool, page_table, self.sel, self.o, self.lse, dO, self.dq, dk_pool,
                      dv_pool, self.ws_bwd, stream=stream)

    def step(self, q, k_pool, v_pool, page_table, dO, dk_pool, dv_pool, stream=None):
        """The chunk's pages get their representative vectors, then select, forward, backward."""
        self.rep_update(k_pool, page_table, self.n, self.chunk_pages, stream=stream)
        self.select(q, stream=stream, keep_scores=False)
        self.fwd(q, k_pool, v_pool, page_table, stream=stream)
        self.bwd(q, k_pool, v_pool, page_table, dO, dk_pool, dv_pool, stream=stream)
