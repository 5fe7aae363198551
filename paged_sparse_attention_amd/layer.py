"""A decoder layer around the paged attention path, trained chunk by chunk.

The OOMB page (technical summary, section 2) trains long sequences chunk by
chunk: each chunk's keys and values go into the paged KV cache, the chunk
attends to the top-K earlier pages and causally to itself, and the backward
pass walks the chunks in reverse, re-running each chunk's forward so that the
activations held at any time are those of one chunk, while the gradients of
the cached keys and values are added in place into paged gradient buffers
outside the autograd graph.  This module puts that attention inside a
Qwen2-style decoder block (RMSNorm, QKV projections with bias, rotary
positions, output projection, RMSNorm, SwiGLU MLP, two residual adds) with
random weights of a given shape; there are no trained weights or data here.

Device work: the projections are library GEMMs on bf16 tensors (fp32
accumulation) and the residual adds are torch operations; the RMSNorms, rotary
positions and the SwiGLU product are liboomb's fused kernels (forward and
backward), and every step of the attention runs in liboomb's kernels: rep
update, top-K selection, fused forward, fused backward with dK/dV added into
the pools.  Weights are kept as fp32 masters and cast to bf16 once per sweep;
each chunk's weight gradients are added into fp32 sums.

Per chunk i (positions i*C .. i*C + C - 1):
  forward   h = rms(x) * ln1; q, k, v = h W + b; rotary(q, k); k, v -> pages
            of chunk i; select among pages of chunks < i; o = attention;
            x1 = x + o Wo; h2 = rms(x1) * ln2; y = x1 + (silu(h2 Wg) * h2 Wu) Wd
  backward  (chunks in reverse) the forward again under autograd with the
            saved selection; the attention's backward adds dK/dV into the
            pools and hands back dQ and the chunk's own (now complete) rows of
            the pools as the gradients of its q, k, v.
The residual stream y, the gradients dx and the weight gradients are fp32.
"""
from __future__ import annotations

import torch

from . import (make_desc, oomb_attn_bwd, oomb_attn_fwd, oomb_bwd_workspace_bytes, oomb_rep_update,
               oomb_rmsnorm_bwd, oomb_rmsnorm_fwd, oomb_rmsnorm_gain_grad, oomb_rotary, oomb_select_topk,
               oomb_select_workspace_bytes, oomb_swiglu_bwd, oomb_swiglu_fwd)

WEIGHTS = ("ln1", "wq", "bq", "wk", "bk", "wv", "bv", "wo", "ln2", "wg", "wu", "wd")


class _RMSNorm(torch.autograd.Function):
    """h = x * rstd * gain (bf16) of fp32 rows x; the library's fused kernels."""

    @staticmethod
    def forward(ctx, x, gain, eps):
        x = x.contiguous()
        h = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
        rstd = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
        oomb_rmsnorm_fwd(x, gain, eps, h, rstd)
        ctx.save_for_backward(x, gain, rstd)
        return h

    @staticmethod
    def backward(ctx, dh):
        x, gain, rstd = ctx.saved_tensors
        dh = dh.to(torch.bfloat16).contiguous()
        dx = torch.empty_like(x)
        oomb_rmsnorm_bwd(x, gain, rstd, dh, None, dx)
        partial = torch.empty((max(1, min(64, x.shape[0])), x.shape[1]), dtype=torch.float32, device=x.device)
        oomb_rmsnorm_gain_grad(x, rstd, dh, partial)
        return dx, partial.sum(dim=0), None


class _SwiGLU(torch.autograd.Function):
    """silu(gate) * up, bf16; the library's fused kernels."""

    @staticmethod
    def forward(ctx, gate, up):
        gate, up = gate.contiguous(), up.contiguous()
        out = torch.empty_like(gate)
        oomb_swiglu_fwd(gate, up, out)
        ctx.save_for_backward(gate, up)
        return out

    @staticmethod
    def backward(ctx, dout):
        gate, up = ctx.saved_tensors
        dg, du = torch.empty_like(gate), torch.empty_like(up)
        oomb_swiglu_bwd(gate, up, dout.to(torch.bfloat16).contiguous(), dg, du)
        return dg, du


class _PagedAttention(torch.autograd.Function):
    """o = paged top-K chunk attention of chunk i with its saved selection, on
    the rotary-positioned q.  q and k come in before their rotary positions
    (bf16); the pools already hold the chunk's positioned keys and values
    (written in the forward sweep), so k and v are inputs only so that
    autograd routes their gradients: the backward reads them out of the
    gradient pools and turns dq and dk back through the rotation."""

    @staticmethod
    def forward(ctx, q_pre, k_pre, v, layer, i):
        q = layer._rotate(q_pre, i)
        o, lse = layer._attend(i, q)
        ctx.save_for_backward(q, o, lse)
        ctx.layer, ctx.i = layer, i
        return o

    @staticmethod
    def backward(ctx, do):
        q, o, lse = ctx.saved_tensors
        layer, i = ctx.layer, ctx.i
        dq, dk, dv = layer._attend_backward(i, q, o, lse, do.to(torch.bfloat16).contiguous())
        return layer._rotate(dq, i, inverse=True), layer._rotate(dk, i, inverse=True), dv.to(torch.bfloat16), \
            None, None


class ChunkedDecoderLayer:
    def __init__(self, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, page_size, chunk_len, n_chunks,
                 top_k, weights, page_table=None, rope_theta=1.0e6, eps=1.0e-6, device="cuda"):
        """weights: name -> tensor (any float dtype) of the shapes in synth.layer_tensors;
        page_table: int32 [pages] logical page -> pool slot (identity if None)."""
        if chunk_len % page_size:
            raise ValueError("chunk_len must be a multiple of page_size")
        self.h, self.hq, self.hkv, self.d = hidden, n_q_heads, n_kv_heads, head_dim
        self.inter, self.ps, self.c, self.n_chunks, self.top_k = intermediate, page_size, chunk_len, n_chunks, top_k
        self.eps = eps
        self.cp = chunk_len // page_size
        self.pages = n_chunks * self.cp
        self.master = {n: weights[n].to(device=device, dtype=torch.float32).clone() for n in WEIGHTS}
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.pt = (torch.arange(self.pages, **i32) if page_table is None
                   else page_table.to(device=device, dtype=torch.int32))
        self.descs = [make_desc(n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, i * self.cp, top_k,
                                self.pages, rep_capacity=self.pages, dtype="bf16") for i in range(n_chunks)]
        pool = (self.pages, n_kv_heads, page_size, head_dim)
        self.k_pool = torch.zeros(pool, dtype=torch.bfloat16, device=device)
        self.v_pool = torch.zeros(pool, dtype=torch.bfloat16, device=device)
        self.dk_pool = torch.zeros(pool, **f32)
        self.dv_pool = torch.zeros(pool, **f32)
        self.rep = torch.zeros((self.pages, n_kv_heads, head_dim), **f32)
        self.sel = [torch.zeros((n_kv_heads, max(min(top_k, i * self.cp), 1)), **i32) for i in range(n_chunks)]
        self.o = torch.empty((chunk_len, n_q_heads, head_dim), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((n_q_heads, chunk_len), **f32)
        self.dq = torch.empty((chunk_len, n_q_heads, head_dim), **f32)
        self.ws_select = torch.empty(max(max(oomb_select_workspace_bytes(d) for d in self.descs), 256),
                                     dtype=torch.uint8, device=device)
        self.ws_bwd = torch.empty(max(max(oomb_bwd_workspace_bytes(d) for d in self.descs), 256),
                                  dtype=torch.uint8, device=device)
        half = head_dim // 2
        inv = rope_theta ** (-torch.arange(half, dtype=torch.float64) * 2.0 / head_dim)
        ang = torch.arange(n_chunks * chunk_len, dtype=torch.float64)[:, None] * inv[None, :]
        self.cos = torch.cos(ang).to(device=device, dtype=torch.float32)
        self.sin = torch.sin(ang).to(device=device, dtype=torch.float32)

    # -- pieces of one chunk ------------------------------------------------
    def _slots(self, i):
        return self.pt[i * self.cp:(i + 1) * self.cp].long()

    def _rotate(self, x, i, inverse=False):
        """bf16 copy of x [C][heads][D] (fp32 or bf16) turned to the positions of chunk i."""
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
        oomb_rotary(x.contiguous(), out, self.cos, self.sin, i * self.c, inverse)
        return out

    def _qkv(self, x, i, w):
        """bf16 q [C][Hq][D] and k, v [C][Hkv][D], before the rotary positions; x fp32."""
        c, hq, hkv, d = self.c, self.hq, self.hkv, self.d
        h = _RMSNorm.apply(x, w["ln1"], self.eps)
        q = (h @ w["wq"] + w["bq"]).view(c, hq, d)
        k = (h @ w["wk"] + w["bk"]).view(c, hkv, d)
        v = (h @ w["wv"] + w["bv"]).view(c, hkv, d)
        return q, k, v

    def _mlp_block(self, x, o, w):
        x1 = x + (o.reshape(self.c, self.hq * self.d) @ w["wo"]).float()
        h2 = _RMSNorm.apply(x1, w["ln2"], self.eps)
        m = _SwiGLU.apply(h2 @ w["wg"], h2 @ w["wu"]) @ w["wd"]
        return x1 + m.float()

    def _weights(self):
        return {n: t.to(torch.bfloat16) for n, t in self.master.items()}

    def _attend(self, i, q):
        oomb_attn_fwd(self.descs[i], q, self.k_pool, self.v_pool, self.pt, self.sel[i], self.o, self.lse)
        return self.o.clone(), self.lse.clone()

    def _attend_backward(self, i, q, o, lse, do):
        oomb_attn_bwd(self.descs[i], q, self.k_pool, self.v_pool, self.pt, self.sel[i], o, lse, do, self.dq,
                      self.dk_pool, self.dv_pool, self.ws_bwd)
        # the chunk's own pages now hold every contribution: later chunks added
        # theirs before this one (reverse order), and this chunk's own just now
        s = self._slots(i)
        to_tokens = lambda pool: pool[s].permute(0, 2, 1, 3).reshape(self.c, self.hkv, self.d)
        return self.dq.clone(), to_tokens(self.dk_pool), to_tokens(self.dv_pool)

    # -- the two sweeps -----------------------------------------------------
    @torch.no_grad()
    def forward(self, x, queries=None):
        """x: bf16 [chunks*C][hidden].  Returns y fp32 [chunks*C][hidden]; keeps
        the pools, the representative vectors and every chunk's selection.
        queries: a list that, when given, receives each chunk's post-rotary
        bf16 queries (the ones the selection scored), for inspection."""
        w = self._weights()
        y = torch.empty((self.n_chunks * self.c, self.h), dtype=torch.float32, device=x.device)
        for i in range(self.n_chunks):
            xi = x[i * self.c:(i + 1) * self.c].float()
            q_pre, k_pre, v = self._qkv(xi, i, w)
            q, k = self._rotate(q_pre, i), self._rotate(k_pre, i)
            s = self._slots(i)
            self.k_pool[s] = k.view(self.cp, self.ps, self.hkv, self.d).permute(0, 2, 1, 3)
            self.v_pool[s] = v.view(self.cp, self.ps, self.hkv, self.d).permute(0, 2, 1, 3)
            desc = self.descs[i]
            if queries is not None:
                queries.append(q.clone())
            oomb_select_topk(desc, q, self.rep, self.sel[i], None, self.ws_select)
            o, _ = self._attend(i, q)
            oomb_rep_update(desc, self.k_pool, self.pt, i * self.cp, self.cp, self.rep)
            y[i * self.c:(i + 1) * self.c] = self._mlp_block(xi, o, w)
        return y

    def backward(self, x, dy):
        """Chunks in reverse with their saved selections.  Returns dx fp32; the
        weight gradients are left in grads (fp32, the masters' shapes).  The
        bf16 weights are cast once for the sweep and are the autograd leaves;
        each chunk's weight gradients (bf16, as the GEMMs give them) are added
        into fp32 sums and cleared."""
        self.dk_pool.zero_()
        self.dv_pool.zero_()
        w = {n: t.to(torch.bfloat16).requires_grad_(True) for n, t in self.master.items()}
        self.grads = {n: torch.zeros_like(t) for n, t in self.master.items()}
        dx = torch.empty((self.n_chunks * self.c, self.h), dtype=torch.float32, device=x.device)
        for i in reversed(range(self.n_chunks)):
            xi = x[i * self.c:(i + 1) * self.c].detach().float().requires_grad_(True)
            with torch.enable_grad():
                q_pre, k_pre, v = self._qkv(xi, i, w)
                o = _PagedAttention.apply(q_pre, k_pre, v, self, i)
                y = self._mlp_block(xi, o, w)
                torch.autograd.backward(y, dy[i * self.c:(i + 1) * self.c])
            dx[i * self.c:(i + 1) * self.c] = xi.grad
            for n, t in w.items():
                self.grads[n].add_(t.grad)
                t.grad = None
        return dx
