"""A full+sparse hybrid stack of SparseX layers on the GPU (SparseX paper
§3.4: layers before a threshold t use full attention; at the boundary one
Sparse-Q estimation with the K/V of the last full layer picks S; every later
layer recomputes only I_nr U S and reuses the realigned cache elsewhere).

Host bookkeeping only: buffers, block tables, uploads and the call order.
Each layer has its own inputs, weights and page pools; the layer input of
every layer is given (synthetic), so no residual/normalisation glue runs
between layers.
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib as L
from .layer import PAGE, DeviceLayout, PagePool, make_dims, rope_table, storage_dtype, workspace


class HybridStackRun:
    """One request batch through `n_layers` layers with threshold `t`.

    layout: list per request of pieces [("reuse", seg_id) | ("new", L)];
    seg_len / seg_p_src: per segment id, its length and the RoPE position of
    its cached copy; ratios: per request (num, den); overflow_tokens: the
    block of reused tokens on each side of a new run that joins the
    Sparse-Q set (§3.3; 0 = off).
    inputs(l) must return (x [n_tok, hidden], w_qkv, x_cache [sum seg len,
    hidden] in segment-id order) as device tensors of the storage type.
    """

    def __init__(self, dims, n_layers: int, threshold: int, layout, seg_len, seg_p_src, ratios,
                 inputs, device="cuda", page_seed: int = 7, overflow_tokens: int = 0,
                 keep_probe_cache: bool = False):
        self.dims, self.cdims = dims, make_dims(dims)
        # threshold 0: keep a device copy of layer 0's K pool as the in-layer
        # probe read it (before the selected rows are recomputed)
        self.keep_probe_cache = keep_probe_cache
        self.probe_k = None
        self.n_layers, self.t = n_layers, threshold
        self.device = device
        self.dt = storage_dtype(dims.dtype)
        n_req = len(layout)
        self.n_req = n_req
        reqs, runs = [], []
        for r, pieces in enumerate(layout):
            pl, start, rr = [], 0, []
            for kind, v in pieces:
                n = seg_len[v] if kind == "reuse" else int(v)
                pl.append((kind == "reuse", n))
                if kind == "reuse":
                    rr.append((start, v))
                start += n
            reqs.append((pl, ratios[r]))
            runs.append(rr)
        self.plan = L.sx_plan_layout(reqs, overflow_tokens=overflow_tokens)
        self.seq_start_h = self.plan["seq_start"]
        self.n_tok = int(self.seq_start_h[-1])
        lens = np.diff(self.seq_start_h)
        req_pages = [(int(n) + PAGE - 1) // PAGE for n in lens]
        seg_ids = sorted(seg_len)
        seg_pages = [(seg_len[s] + PAGE - 1) // PAGE for s in seg_ids]
        rng = np.random.default_rng(page_seed)
        # one request pool and one source pool per layer, same block tables
        n_req_pages = sum(req_pages)
        perm = rng.permutation(n_req_pages).astype(np.int32)
        self.max_pages = max(req_pages)
        bt = np.full((n_req, self.max_pages), -1, np.int32)
        o = 0
        for r, n in enumerate(req_pages):
            bt[r, :n] = perm[o:o + n]
            o += n
        n_src_pages = sum(seg_pages)
        sperm = rng.permutation(n_src_pages).astype(np.int32)
        self.seg_page_off, o = {}, 0
        for s, n in zip(seg_ids, seg_pages):
            self.seg_page_off[s] = o
            o += n
        self.seg_page_ids = sperm
        self.block_table = bt
        max_pos = max(self.n_tok, max(seg_p_src[s] + seg_len[s] for s in seg_ids)) + 1
        self.rope = rope_table(dims.theta, dims.head_dim, max_pos + 16, device)
        self.lay = DeviceLayout(self.seq_start_h, bt, self.rope, device)
        # cache-building layout: each segment alone at its original position
        cseq = np.concatenate([[0], np.cumsum([seg_len[s] for s in seg_ids])]).astype(np.int32)
        cbt = np.full((len(seg_ids), max(seg_pages)), -1, np.int32)
        for i, s in enumerate(seg_ids):
            cbt[i, :seg_pages[i]] = sperm[self.seg_page_off[s]:self.seg_page_off[s] + seg_pages[i]]
        self.cache_lay = DeviceLayout(cseq, cbt, self.rope, device,
                                      pos_offset=np.array([seg_p_src[s] for s in seg_ids], np.int32))
        self.n_cache_tok = int(cseq[-1])
        # realign jobs (identical for every layer: same tables, per-layer pools)
        segs = []
        for r, rr in enumerate(runs):
            for dst, sid in rr:
                segs.append(dict(req=r, dst_start=dst, len=seg_len[sid], p_src=seg_p_src[sid],
                                 src_slot0=0, src_pages_off=self.seg_page_off[sid]))
        self.jobs_h = L.sx_plan_realign(segs, sperm, bt)
        self.jobs = torch.from_numpy(self.jobs_h).to(device)
        # per-layer state
        self.inputs = inputs
        self.req_pools = [PagePool.alloc(n_req_pages, dims, device, fill_guard=False)
                          for _ in range(n_layers)]
        self.src_pools = [None if l < threshold else
                          PagePool.alloc(n_src_pages, dims, device, fill_guard=False)
                          for l in range(n_layers)]
        # metadata on the device
        p = self.plan
        self.tok_class = torch.from_numpy(p["tok_class"]).to(device)
        self.sq_rows = torch.from_numpy(p["sq_rows"]).to(device)
        self.sq_start = torch.from_numpy(p["sq_start"]).to(device)
        self.n_sq = int(p["sq_start"][-1])
        self.k_h = p["k"]
        self.k_sel = torch.from_numpy(self.k_h).to(device)
        self.n_sel = int(self.k_h.sum())
        self.n_act = self.n_sq + self.n_sel
        self.act_start_h = (p["sq_start"] + np.concatenate([[0], np.cumsum(self.k_h)])).astype(np.int32)
        self.act_start = torch.from_numpy(self.act_start_h).to(device)
        self.all_rows = torch.arange(self.n_tok, dtype=torch.int32, device=device)
        self.cache_rows = torch.arange(self.n_cache_tok, dtype=torch.int32, device=device)
        hq, d = dims.n_q_heads, dims.head_dim
        self.q_full = torch.empty((self.n_tok, hq, d), dtype=self.dt, device=device)
        self.o_full = torch.empty((self.n_tok, hq * d), dtype=self.dt, device=device)
        self.lse_full = torch.empty((self.n_tok, hq), dtype=torch.float32, device=device)
        # two Q buffers of the active rows: with layers pipelined, layer l+1's
        # recompute writes one while layer l's attention reads the other
        self.q_act_buf = [torch.empty((max(self.n_act, 1), hq, d), dtype=self.dt, device=device)
                          for _ in range(2)]
        self.q_act = self.q_act_buf[0]
        self.o_act = [torch.empty((max(self.n_act, 1), hq * d), dtype=self.dt, device=device)
                      for _ in range(n_layers)]
        self.sel_rows = torch.empty(max(self.n_sel, 1), dtype=torch.int32, device=device)
        self.act_rows = torch.empty(max(self.n_act, 1), dtype=torch.int32, device=device)
        self.scores = torch.empty(self.n_tok, dtype=torch.float32, device=device)
        self.ws_sel = workspace(L.SX_OP_SELECT, self.cdims, self.n_tok, self.n_sq, n_req, device)
        self.ws_attn = workspace(L.SX_OP_SPARSE_ATTN, self.cdims, self.n_tok, max(self.n_act, 1), n_req, device)
        self.ws_full = workspace(L.SX_OP_FULL_ATTN, self.cdims, self.n_tok, self.n_tok, n_req, device)
        self.o_full_layers = []

    def build_caches(self):
        """Segment caches of every sparse layer: each segment computed alone
        at its original positions (K/V only)."""
        for l in range(self.t, self.n_layers):
            _, w, xc = self.inputs(l)
            L.sx_recompute_kv(self.cdims, self.cache_lay.struct, xc, self.cache_rows, self.n_cache_tok, w,
                              self.src_pools[l].struct(), None)

    # ---- the hot path ---------------------------------------------------------
    def full_layer(self, l: int, timer=None):
        x, w, _ = self.inputs(l)
        pages = self.req_pools[l].struct()
        with _phase(timer, "full_recompute"):
            L.sx_recompute_kv(self.cdims, self.lay.struct, x, self.all_rows, self.n_tok, w, pages, self.q_full)
        with _phase(timer, "full_attn"):
            L.sx_full_attn(self.cdims, self.lay.struct, self.q_full, pages, self.o_full,
                           self.lse_full if l == self.t - 1 else None, self.ws_full)

    def select(self, l: int, timer=None):
        """Boundary: Sparse-Q rows of layer l (its Q, fresh K and LSE)."""
        with _phase(timer, "select"):
            L.sx_select_topk(self.cdims, self.lay.struct, self.q_full, self.sq_rows, self.sq_rows,
                             self.sq_start, self.n_sq, self.lse_full, self.req_pools[l].struct(),
                             self.tok_class, self.k_sel, self.sel_rows, self.act_rows, self.scores,
                             self.ws_sel)

    def select_in_layer(self, l: int, timer=None):
        """Threshold 0: Sparse-Q rows recomputed in layer l and probed over its
        realigned cache (LSE computed inside the selection)."""
        x, w, _ = self.inputs(l)
        pages = self.req_pools[l].struct()
        with _phase(timer, "realign"):
            L.sx_rope_realign(self.cdims, self.lay.struct, self.src_pools[l].struct(), pages, self.jobs,
                              len(self.jobs_h))
        with _phase(timer, "select_recompute"):
            L.sx_recompute_kv(self.cdims, self.lay.struct, x, self.sq_rows, self.n_sq, w, pages, self.q_full)
        with _phase(timer, "select"):
            L.sx_select_topk(self.cdims, self.lay.struct, self.q_full, None, self.sq_rows, self.sq_start,
                             self.n_sq, None, pages, self.tok_class, self.k_sel, self.sel_rows,
                             self.act_rows, self.scores, self.ws_sel)
        if self.keep_probe_cache:
            self.probe_k = self.req_pools[l].k.clone()

    def sparse_prep(self, l: int, timer=None, realign: bool = True, next_realign: bool = False):
        """Layer l's cache and queries: realign its reused runs (unless done
        already), recompute A.  next_realign: layer l+1's realign rides along
        in the same launch (sx_recompute_kv_realign; the two write different
        pools, and layer l+1's realign only has to finish before its own
        recomputation)."""
        x, w, _ = self.inputs(l)
        pages = self.req_pools[l].struct()
        if realign:
            with _phase(timer, "realign"):
                L.sx_rope_realign(self.cdims, self.lay.struct, self.src_pools[l].struct(), pages, self.jobs,
                                  len(self.jobs_h))
        if next_realign:
            with _phase(timer, "recompute_realign"):
                L.sx_recompute_kv_realign(self.cdims, self.lay.struct, x, self.act_rows, self.n_act, w, pages,
                                          self.q_act_buf[l % 2], self.src_pools[l + 1].struct(),
                                          self.req_pools[l + 1].struct(), self.jobs, len(self.jobs_h))
            return
        with _phase(timer, "recompute"):
            L.sx_recompute_kv(self.cdims, self.lay.struct, x, self.act_rows, self.n_act, w, pages,
                              self.q_act_buf[l % 2])

    def attn_plan(self, timer=None):
        """The active set is fixed once the selection is made (§3.4): the
        attention's work list over it is built once for every sparse layer."""
        with _phase(timer, "attn_plan"):
            L.sx_sparse_attn_plan(self.cdims, self.lay.struct, self.act_rows, self.act_start, self.n_act,
                                  self.ws_attn)

    def sparse_attn(self, l: int, timer=None):
        with _phase(timer, "sparse_attn"):
            L.sx_sparse_attn_run(self.cdims, self.lay.struct, self.q_act_buf[l % 2], self.act_rows,
                                 self.n_act, self.req_pools[l].struct(), self.o_act[l], None,
                                 self.ws_attn)

    def sparse_layer(self, l: int, timer=None, realign: bool = True, next_realign: bool = False):
        self.sparse_prep(l, timer, realign, next_realign)
        self.sparse_attn(l, timer)

    def sparse_layers_pipelined(self, first: int, timer=None, first_realigned: bool = False):
        """Sparse layers first..n-1 on two streams: layer l+1's realign and
        recompute (side stream) run while layer l's attention (launch
        stream) does; events order each attention after its own layer's
        preparation and each preparation after the attention that last read
        its Q buffer.  The launch stream ends after the last attention."""
        import torch
        main = torch.cuda.current_stream()
        if not hasattr(self, "side_stream"):
            self.side_stream = torch.cuda.Stream()   # default priority
        side = self.side_stream
        start = torch.cuda.Event()
        start.record(main)
        side.wait_event(start)
        prep_done, attn_done = {}, {}

        def prep(l):
            if l - 2 >= first:
                side.wait_event(attn_done[l - 2])
            with torch.cuda.stream(side):
                self.sparse_prep(l, timer, realign=not (first_realigned and l == first))
                ev = torch.cuda.Event()
                ev.record(side)
            prep_done[l] = ev

        prep(first)
        for l in range(first, self.n_layers):
            if l + 1 < self.n_layers:
                prep(l + 1)
            main.wait_event(prep_done[l])
            self.sparse_attn(l, timer)
            ev = torch.cuda.Event()
            ev.record(main)
            attn_done[l] = ev
        # the side stream's last work is done before the last attention began

    def decode_attention(self, l: int, q, o, lse=None):
        """Decode attention of each request's last token over layer l's mixed
        cache (sx_decode_attn); q [n_req, Hq, d], o [n_req, Hq*d]."""
        if not hasattr(self, "ws_dec"):
            self.ws_dec = workspace(L.SX_OP_DECODE, self.cdims, self.n_tok, 0, self.n_req, self.device)
        L.sx_decode_attn(self.cdims, self.lay.struct, q, self.req_pools[l].struct(), o, lse, self.ws_dec)

    def forward(self, timer=None, keep_full_outputs: bool = False, pipelined: bool = False,
                marks=None):
        """One prefill pass of the batch through every layer (pipelined: the
        sparse layers on two streams, see sparse_layers_pipelined).  marks
        (a dict, optional) receives events on the launch stream: "sparse"
        just before the selection, "end" after the last layer."""
        import torch

        def mark(name):
            if marks is not None:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record()
                marks[name] = ev

        self._forward(timer, keep_full_outputs, pipelined, mark)
        mark("end")

    def _forward(self, timer, keep_full_outputs, pipelined, mark):
        for l in range(self.t):
            self.full_layer(l, timer)
            if keep_full_outputs:
                self.o_full_layers.append(self.o_full.clone())
        if self.t >= self.n_layers:   # every layer full: nothing to select for
            return
        mark("sparse")
        if self.t > 0:
            self.select(self.t - 1, timer)
            self.attn_plan(timer)
            if pipelined:
                self.sparse_layers_pipelined(self.t, timer)
            else:
                self.sparse_layers(self.t, timer)
        else:
            self.select_in_layer(0, timer)
            self.attn_plan(timer)
            if pipelined:
                self.sparse_layers_pipelined(0, timer, first_realigned=True)
            else:
                self.sparse_layers(0, timer, first_realigned=True)

    def sparse_layers(self, first: int, timer=None, first_realigned: bool = False):
        """Sparse layers first..n-1 on one stream: each layer's recompute
        launch also carries the next layer's realign (which then needs no
        launch of its own); only layer `first` is realigned alone."""
        for l in range(first, self.n_layers):
            self.sparse_layer(l, timer, realign=(l == first and not first_realigned),
                              next_realign=(l + 1 < self.n_layers))


class _NoPhase:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


class _Phase:
    def __init__(self, timer, name):
        self.timer, self.name = timer, name

    def __enter__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *a):
        self.b.record()
        self.timer.setdefault(self.name, []).append((self.a, self.b))
        return False


def _phase(timer, name):
    return _NoPhase() if timer is None else _Phase(timer, name)


def phase_ms(timer) -> dict:
    """Total milliseconds per phase name (call after synchronising)."""
    return {k: sum(a.elapsed_time(b) for a, b in v) for k, v in timer.items()}


def phase_counts(timer) -> dict:
    return {k: len(v) for k, v in timer.items()}
