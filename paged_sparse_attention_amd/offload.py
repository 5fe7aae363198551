"""Chunk-recurrent attention of one layer with the KV cache and its gradients in
CPU memory.

The OOMB page's KV-cache stack (technical summary, section 2) adds to paged
memory and page-level sparse attention an asynchronous CPU offload: the KV
cache and its gradients, which grow with the context, are kept in CPU memory
and moved between CPU and GPU asynchronously, overlapped with computation, so
that the added training time stays small (the page reports under 5%).

This driver runs the same sequence as ChunkedSequence (sequence.py) with the
K/V pools and the dK/dV pools in pinned host memory.  The GPU holds only, per
chunk in flight, a staging pool with the blocks that chunk touches (its
selected (kv-head, page) blocks and its own pages; layout in include/oomb.h),
plus the representative-vector table, the selections and one chunk's
activations.  Three streams carry the work:

  compute  chunk pages into staging, rep update, selection, attention
  h2d      oomb_stage_gather: selected blocks (and, in the backward, the
           chunk's own pages) from the host pools into a staging buffer
  d2h      oomb_stage_offload_chunk after a chunk's forward (its keys and
           values to the host pools) and oomb_stage_flush_grads after its
           backward (the device adds the staged gradients into the host dK/dV
           pools over the link and clears the staging); with
           host_accumulate=True instead oomb_stage_grads_out (the staged
           gradients to a pinned host buffer, staging cleared), which a host
           worker thread adds into the pools with oomb_host_accumulate_grads
           while the device runs the next chunk.  Both give the same bits; the
           device flush measured faster at the Qwen2.5-7B shape (the link
           traffic slows the concurrent attention kernels whichever way it
           flows, and the host route adds the host's memory traffic)

Staging is double-buffered, so the copies for one chunk run while the
neighbouring chunk computes:
  forward   chunk i+1's selection is made before chunk i's attention (it needs
            only chunk i's representative vectors), so its gather overlaps
            chunk i's attention; the pages of chunk i it selects are copied
            from chunk i's staging buffer, so the gather need not wait for
            chunk i's offload.  This needs every chunk's queries up front,
            as in this single-layer driver; in a full model the next chunk's
            queries come from the layer below.
  backward  chunk i-1's gather and chunk i+1's gradient flush overlap chunk i's
            backward; flushes run in chunk order on one stream, so the host
            gradients receive each chunk's contribution in turn.

The attention calls are the library's ordinary entry points on the staging pool
with the staged descriptor, so every kv-head visits the same keys in the same
order as on device-resident pools: selections, O, LSE and dQ are bitwise those
of ChunkedSequence; dK/dV differ only in fp32 rounding (each chunk's
contribution is summed in staging and then added to the host pool, instead of
being added to the pool directly).

Marshalling and stream ordering only: every step runs in the library's kernels.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import torch

from . import (OOMB_STAGE_CHUNK, OOMB_STAGE_SELECTED, make_desc, oomb_attn_bwd, oomb_attn_fwd,
               oomb_bwd_workspace_bytes, oomb_host_accumulate_grads, oomb_host_view, oomb_rep_update,
               oomb_select_topk, oomb_select_workspace_bytes, oomb_stage_desc, oomb_stage_flush_grads,
               oomb_stage_gather, oomb_stage_grads_out, oomb_stage_offload_chunk, oomb_stage_tables)
from .step import TORCH_DTYPE


class OffloadedSequence:
    def __init__(self, n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, n_chunks, top_k,
                 n_initial_pages=0, n_slots=None, dtype="bf16", softmax_scale=0.0, device="cuda",
                 keep_activations=False, n_buffers=2, copy_cus=0, host_accumulate=False, host_threads=12):
        if chunk_len % page_size:
            raise ValueError("chunk_len must be a multiple of page_size")
        if n_buffers < 2:
            raise ValueError("n_buffers must be at least 2")
        self.hq, self.hkv, self.d, self.ps, self.c = n_q_heads, n_kv_heads, head_dim, page_size, chunk_len
        self.n_chunks, self.top_k, self.n0, self.dtype = n_chunks, top_k, n_initial_pages, dtype
        self.keep_activations, self.nbuf = keep_activations, n_buffers
        self.host_accumulate, self.host_threads = host_accumulate, host_threads
        self.chunk_pages = chunk_len // page_size
        self.total_pages = n_initial_pages + n_chunks * self.chunk_pages
        self.n_slots = self.total_pages if n_slots is None else n_slots
        self.descs = [make_desc(n_q_heads, n_kv_heads, head_dim, page_size, chunk_len, self.prior_pages(i), top_k,
                                self.n_slots, rep_capacity=self.total_pages, dtype=dtype,
                                softmax_scale=softmax_scale)
                      for i in range(n_chunks)]
        self.staged = [oomb_stage_desc(d) for d in self.descs]
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        # staged selection and identity page table, one pair per distinct K_eff
        self._tables = {}
        for i, sd in enumerate(self.staged):
            ke = self.keff(i)
            if ke not in self._tables:
                sel_s = torch.zeros(max(self.hkv * ke, 1), **i32)
                pt_s = torch.zeros(sd.n_slots, **i32)
                oomb_stage_tables(self.descs[i], sel_s, pt_s)
                self._tables[ke] = (sel_s, pt_s)
        # rep update of chunk i's pages reads them from staging: logical page
        # N_i + j -> staging slot Hkv*K_eff_i + j.  The chunks' page ranges are
        # disjoint, so one table of every page holds all of them (O(pages) of
        # device memory, not one table per chunk).
        self._pt_rep = torch.zeros(self.total_pages, **i32)
        for i in range(n_chunks):
            nsel = self.hkv * self.keff(i)
            self._pt_rep[self.prior_pages(i):self.prior_pages(i) + self.chunk_pages] = torch.arange(
                nsel, nsel + self.chunk_pages, **i32)
        n_stage = max(sd.n_slots for sd in self.staged)
        blk = (n_stage, n_kv_heads, page_size, head_dim)
        self.stage_k = [torch.empty(blk, dtype=TORCH_DTYPE[dtype], device=device) for _ in range(n_buffers)]
        self.stage_v = [torch.empty(blk, dtype=TORCH_DTYPE[dtype], device=device) for _ in range(n_buffers)]
        # gradient staging starts at zero; every flush leaves what it read at zero
        self.stage_dk = [torch.zeros(blk, **f32) for _ in range(n_buffers)]
        self.stage_dv = [torch.zeros(blk, **f32) for _ in range(n_buffers)]
        self.rep = torch.zeros((self.total_pages, n_kv_heads, head_dim), **f32)
        self.sel = [torch.zeros((n_kv_heads, max(self.keff(i), 1)), **i32) for i in range(n_chunks)]
        n_act = n_chunks if keep_activations else 1
        self.o = torch.empty((n_act, chunk_len, n_q_heads, head_dim), dtype=TORCH_DTYPE[dtype], device=device)
        self.lse = torch.empty((n_act, n_q_heads, chunk_len), **f32)
        self.dq = torch.empty((n_chunks, chunk_len, n_q_heads, head_dim), **f32)
        ws_sel = max(oomb_select_workspace_bytes(d) for d in self.descs)
        ws_bwd = max(oomb_bwd_workspace_bytes(d) for d in self.staged)
        self.ws_select = torch.empty(max(ws_sel, 256), dtype=torch.uint8, device=device)
        self.ws_bwd = torch.empty(max(ws_bwd, 256), dtype=torch.uint8, device=device)
        # host side of the gradient offload: two compact delta buffers that
        # the device writes in turn, and host copies of the page table and of
        # the selections (made on the compute stream during the forward)
        n_blocks = max(self.hkv * self.keff(i) + self.chunk_pages * self.hkv for i in range(n_chunks))
        if host_accumulate:
            self.delta_dk = [torch.empty((n_blocks, page_size, head_dim), dtype=torch.float32).pin_memory()
                             for _ in range(2)]
            self.delta_dv = [torch.empty_like(t).pin_memory() for t in self.delta_dk]
        self.sel_host = [torch.zeros(tuple(t.shape), dtype=torch.int32).pin_memory() for t in self.sel]
        self.pt_host = torch.zeros(self.total_pages, dtype=torch.int32).pin_memory()
        self._make_streams(device, copy_cus)

    def prior_pages(self, i):
        return self.n0 + i * self.chunk_pages

    def keff(self, i):
        return max(0, min(self.top_k, self.prior_pages(i)))

    def _act(self, i):
        return i if self.keep_activations else 0

    def _staged_call_args(self, i, b):
        sel_s, pt_s = self._tables[self.keff(i)]
        return self.staged[i], sel_s, pt_s, self.stage_k[b], self.stage_v[b]

    @staticmethod
    def _views(*host):
        return [oomb_host_view(h) for h in host]

    def forward(self, q, k_new, v_new, host_k, host_v, page_table, on_chunk=None):
        """q [chunks][C][Hq][D] and the chunks' own keys/values k_new, v_new
        [chunks][C/ps][Hkv][ps][D] on the device; host_k, host_v: pinned host
        pools [n_slots][Hkv][ps][D] holding the initial context (the chunks'
        pages are written into them here); page_table: int32 [total pages] on
        the device, logical page -> host slot.  on_chunk(i, O, LSE) as in
        ChunkedSequence.  Ordered after, and before, the caller's current
        stream; returns (O, LSE).  The host pools must stay allocated until
        that work has completed."""
        hk, hv = self._views(host_k, host_v)
        caller = torch.cuda.current_stream()
        comp = self._enter(caller)
        ev = lambda: torch.cuda.Event()
        fwd_done = [None] * self.n_chunks
        offloaded = [None] * self.n_chunks
        gathered = [None] * self.n_chunks

        def gather_selected(i, ready):
            """Selected blocks of chunk i into its staging buffer: pages of
            chunk i-1 from that chunk's staging buffer (still on the device),
            earlier pages from the host pools."""
            b = i % self.nbuf
            with torch.cuda.stream(self.h2d):
                self.h2d.wait_event(ready)  # chunk i's selection made, chunk i-1's pages staged
                if i >= 2:
                    self.h2d.wait_event(offloaded[i - 2])  # chunks before i-1 are in the host pools
                if i >= self.nbuf:  # buffer b's previous chunk has run and been offloaded
                    self.h2d.wait_event(fwd_done[i - self.nbuf])
                    self.h2d.wait_event(offloaded[i - self.nbuf])
                if self.keff(i) > 0:
                    recent = self.prior_pages(i - 1) if i >= 1 else self.prior_pages(i)
                    if recent > 0:
                        oomb_stage_gather(self.descs[i], hk, hv, page_table, self.sel[i], OOMB_STAGE_SELECTED,
                                          self.stage_k[b], self.stage_v[b], first_page=0, n_pages=recent,
                                          stream=self.h2d)
                    if i >= 1:
                        pb = (i - 1) % self.nbuf
                        oomb_stage_gather(self.descs[i], self.stage_k[pb], self.stage_v[pb], self._pt_rep,
                                          self.sel[i], OOMB_STAGE_SELECTED, self.stage_k[b], self.stage_v[b],
                                          src_slots=self.staged[i - 1].n_slots, first_page=recent,
                                          n_pages=self.chunk_pages, stream=self.h2d)
                gathered[i] = ev()
                gathered[i].record(self.h2d)

        with torch.cuda.stream(comp):
            self.pt_host.copy_(page_table[:self.total_pages], non_blocking=True)
            if self.n0 > 0:  # representative vectors of the initial context, read through the host view
                oomb_rep_update(self.descs[0], hk, page_table, 0, self.n0, self.rep, stream=comp)
            if self.keff(0) > 0:
                oomb_select_topk(self.descs[0], q[0], self.rep, self.sel[0], None, self.ws_select, stream=comp)
                self.sel_host[0].copy_(self.sel[0], non_blocking=True)
            ready = ev()
            ready.record(comp)
            gather_selected(0, ready)
            for i in range(self.n_chunks):
                b, a = i % self.nbuf, self._act(i)
                sd, sel_s, pt_s, sk, sv = self._staged_call_args(i, b)
                nsel = self.hkv * self.keff(i)
                if i >= self.nbuf:
                    comp.wait_event(offloaded[i - self.nbuf])  # buffer b's chunk pages are in the host pools
                sk[nsel:nsel + self.chunk_pages].copy_(k_new[i])
                sv[nsel:nsel + self.chunk_pages].copy_(v_new[i])
                oomb_rep_update(self.descs[i], sk, self._pt_rep, self.prior_pages(i), self.chunk_pages,
                                self.rep, stream=comp)
                if i + 1 < self.n_chunks and self.keff(i + 1) > 0:
                    oomb_select_topk(self.descs[i + 1], q[i + 1], self.rep, self.sel[i + 1], None, self.ws_select,
                                     stream=comp)
                    self.sel_host[i + 1].copy_(self.sel[i + 1], non_blocking=True)
                ready = ev()
                ready.record(comp)
                # chunk i's pages to the host and chunk i+1's blocks to the device,
                # both overlapping chunk i's attention
                with torch.cuda.stream(self.d2h):
                    self.d2h.wait_event(ready)
                    oomb_stage_offload_chunk(self.descs[i], sk, sv, page_table, hk, hv, stream=self.d2h)
                    offloaded[i] = ev()
                    offloaded[i].record(self.d2h)
                if i + 1 < self.n_chunks:
                    gather_selected(i + 1, ready)
                comp.wait_event(gathered[i])
                oomb_attn_fwd(sd, q[i], sk, sv, pt_s, sel_s, self.o[a], self.lse[a], stream=comp)
                fwd_done[i] = ev()
                fwd_done[i].record(comp)
                if on_chunk is not None:
                    on_chunk(i, self.o[a], self.lse[a])
            comp.wait_event(offloaded[-1])
        self._leave(comp, caller)
        return self.o, self.lse

    def backward(self, q, dO, host_k, host_v, host_dk, host_dv, page_table):
        """Chunks in reverse order with their forward selections; host_dk and
        host_dv (pinned fp32 pools) receive the gradients in place.  The forward
        must have run with the same page table (it wrote the chunks' pages into
        host_k / host_v); without kept activations each chunk's forward is
        re-run on its staged blocks.  Ordered after, and before, the caller's
        current stream.  With host accumulation the host gradients are final
        when this returns; otherwise once that stream's work completes.
        Returns dQ."""
        hk, hv, hdk, hdv = self._views(host_k, host_v, host_dk, host_dv)
        caller = torch.cuda.current_stream()
        comp = self._enter(caller)
        ev = lambda: torch.cuda.Event()
        start = ev()
        start.record(comp)  # after the forward, including its last offload
        last = self.n_chunks - 1
        bwd_done = [None] * self.n_chunks
        cleared = [None] * self.n_chunks   # chunk's gradient staging read out and zeroed
        gathered = [None] * self.n_chunks
        if self.host_accumulate:
            dviews = [self._views(self.delta_dk[j], self.delta_dv[j]) for j in range(2)]

        def gather(i):
            b = i % self.nbuf
            with torch.cuda.stream(self.h2d):
                self.h2d.wait_event(start)
                if i + self.nbuf <= last:  # buffer b's previous chunk has run
                    self.h2d.wait_event(bwd_done[i + self.nbuf])
                oomb_stage_gather(self.descs[i], hk, hv, page_table, self.sel[i],
                                  OOMB_STAGE_SELECTED | OOMB_STAGE_CHUNK, self.stage_k[b], self.stage_v[b],
                                  stream=self.h2d)
                gathered[i] = ev()
                gathered[i].record(self.h2d)

        def accumulate(i):
            # on the worker thread: once chunk i's gradient blocks have reached
            # host memory, add them into the host pools (the GIL is released
            # during the add, so the main thread keeps enqueuing)
            cleared[i].synchronize()
            j = i % 2
            oomb_host_accumulate_grads(self.descs[i], self.delta_dk[j], self.delta_dv[j], self.pt_host,
                                       self.sel_host[i], host_dk, host_dv, self.host_threads)

        adds = {}
        worker = ThreadPoolExecutor(max_workers=1) if self.host_accumulate else None

        try:
            with torch.cuda.stream(comp):
                gather(last)
                for i in reversed(range(self.n_chunks)):
                    b, a = i % self.nbuf, self._act(i)
                    sd, sel_s, pt_s, sk, sv = self._staged_call_args(i, b)
                    comp.wait_event(gathered[i])
                    if i + self.nbuf <= last:
                        comp.wait_event(cleared[i + self.nbuf])  # gradient staging b is back at zero
                    if not self.keep_activations:
                        oomb_attn_fwd(sd, q[i], sk, sv, pt_s, sel_s, self.o[a], self.lse[a], stream=comp)
                    oomb_attn_bwd(sd, q[i], sk, sv, pt_s, sel_s, self.o[a], self.lse[a], dO[i], self.dq[i],
                                  self.stage_dk[b], self.stage_dv[b], self.ws_bwd, stream=comp)
                    bwd_done[i] = ev()
                    bwd_done[i].record(comp)
                    if i > 0:
                        gather(i - 1)
                    if self.host_accumulate and i + 2 in adds:
                        adds.pop(i + 2).result()  # delta buffer i % 2 has been added on the host
                    with torch.cuda.stream(self.d2h):  # in chunk order on one stream
                        self.d2h.wait_event(bwd_done[i])
                        if self.host_accumulate:
                            oomb_stage_grads_out(self.descs[i], self.stage_dk[b], self.stage_dv[b], *dviews[i % 2],
                                                 stream=self.d2h)
                        else:
                            oomb_stage_flush_grads(self.descs[i], self.stage_dk[b], self.stage_dv[b], page_table,
                                                   self.sel[i], hdk, hdv, stream=self.d2h)
                        cleared[i] = ev()
                        cleared[i].record(self.d2h)
                    if self.host_accumulate:
                        adds[i] = worker.submit(accumulate, i)  # runs while the device computes chunk i-1
                if self.host_accumulate:
                    for i in sorted(adds, reverse=True):
                        adds.pop(i).result()
                comp.wait_event(cleared[0])
        finally:
            if worker is not None:
                worker.shutdown(wait=True)
        self._leave(comp, caller)
        return self.dq

    # ---- streams

    def _enter(self, caller):
        """The stream the attention runs on, ordered after the caller's work."""
        if self.comp is None:
            return caller
        e = torch.cuda.Event()
        e.record(caller)
        self.comp.wait_event(e)
        return self.comp

    def _leave(self, comp, caller):
        if comp is not caller:
            e = torch.cuda.Event()
            e.record(comp)
            caller.wait_event(e)

    def _make_streams(self, device, copy_cus):
        """Copy streams, and with copy_cus > 0 a compute stream, partitioned by
        compute-unit masks: the copy kernels get copy_cus compute units of their
        own (one per XCD when copy_cus is 8), the attention the rest.  Measured
        at the Qwen2.5-7B shape, the partition costs the attention more than it
        saves the copies (the forward kernel loses 15% with 8 units fewer), so
        the default is none.  All streams keep the default priority."""
        self.comp = None
        if copy_cus <= 0:
            self.h2d = torch.cuda.Stream(device=device)
            self.d2h = torch.cuda.Stream(device=device)
            return
        self.comp, self.h2d, self.d2h = _masked_streams(torch.device(device), copy_cus)


# Compute-unit-masked streams, made once per (device, copy_cus) and kept for
# the life of the process: torch records events on the streams that pinned
# host tensors were copied on when it frees them, so such a stream must
# outlive every tensor that may have touched it.
_MASKED = {}


def _masked_streams(device, copy_cus):
    import ctypes
    from . import hip_runtimes_loaded
    idx = device.index if device.index is not None else torch.cuda.current_device()
    key = (idx, copy_cus)
    if key in _MASKED:
        return _MASKED[key]
    n_cu = torch.cuda.get_device_properties(idx).multi_processor_count
    if copy_cus >= n_cu:
        raise ValueError("copy_cus must leave compute units for the attention")
    words = (n_cu + 31) // 32
    # CU k*(n_cu/copy_cus) + k: spread over the chip whether the mask bits run
    # XCD-major or XCD-interleaved
    step = n_cu // copy_cus
    picks = {(k * step + k) % n_cu for k in range(copy_cus)}
    copy_mask, comp_mask = [0] * words, [0] * words
    for c in range(n_cu):
        m = copy_mask if c in picks else comp_mask
        m[c // 32] |= 1 << (c % 32)
    rt = ctypes.CDLL(hip_runtimes_loaded()[0])

    def create(mask):
        st = ctypes.c_void_p()
        arr = (ctypes.c_uint32 * words)(*mask)
        rc = rt.hipExtStreamCreateWithCUMask(ctypes.byref(st), ctypes.c_uint32(words), arr)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with hipError {rc}")
        return torch.cuda.ExternalStream(st.value, device=idx)

    with torch.cuda.device(idx):
        _MASKED[key] = (create(comp_mask), create(copy_mask), create(copy_mask))
    return _MASKED[key]
