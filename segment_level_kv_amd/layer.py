"""One SparseX prefill layer on the GPU, driven through the libsx C ABI.

This module is host bookkeeping around the five device entry points: it
allocates page pools and buffers with torch, builds block tables and
uploads the scheduler metadata, and calls libsx in the order the method runs
(SparseX paper §3.1-§3.4; the flow of §4.5).  All arithmetic of the layer
runs in libsx's kernels; the token classes, budgets and realign jobs come
from libsx's host planners.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L

PAGE = 16
GUARD_BITS_BF16 = 0x7FA5          # a NaN pattern: any stray write to a guard page is visible
GUARD_F32 = float("nan")


def storage_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def make_dims(d) -> L.Dims:
    return L.Dims(d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, PAGE,
                  L.SX_BF16 if d.dtype == "bf16" else L.SX_F32)


@dataclass
class PagePool:
    """One layer's K and V pools: K [n_pages][Hkv][16][d], V [n_pages][Hkv][d][16]."""
    k: torch.Tensor
    v: torch.Tensor

    @classmethod
    def alloc(cls, n_pages: int, dims, device, fill_guard: bool = True):
        dt = storage_dtype(dims.dtype)
        k = torch.empty((n_pages, dims.n_kv_heads, PAGE, dims.head_dim), dtype=dt, device=device)
        v = torch.empty((n_pages, dims.n_kv_heads, dims.head_dim, PAGE), dtype=dt, device=device)
        if fill_guard:
            if dims.dtype == "bf16":
                k.view(torch.int16).fill_(GUARD_BITS_BF16)
                v.view(torch.int16).fill_(GUARD_BITS_BF16)
            else:
                k.fill_(GUARD_F32)
                v.fill_(GUARD_F32)
        return cls(k, v)

    @property
    def n_pages(self) -> int:
        return self.k.shape[0]

    def struct(self) -> L.Pages:
        return L.Pages(self.k.data_ptr(), self.v.data_ptr(), self.n_pages)


class DeviceLayout:
    """Device copies of a batch's request layout (seq_start, block table,
    per-request RoPE offset) and the RoPE table."""

    def __init__(self, seq_start: np.ndarray, block_table: np.ndarray, rope_tab: torch.Tensor,
                 device, pos_offset=None):
        self.seq_start_h = np.ascontiguousarray(seq_start, dtype=np.int32)
        self.block_table_h = np.ascontiguousarray(block_table, dtype=np.int32)
        self.seq_start = torch.from_numpy(self.seq_start_h).to(device)
        self.block_table = torch.from_numpy(self.block_table_h).to(device)
        self.pos_offset_h = None if pos_offset is None else np.ascontiguousarray(pos_offset, np.int32)
        self.pos_offset = None if pos_offset is None else torch.from_numpy(self.pos_offset_h).to(device)
        self.rope_tab = rope_tab
        self.struct = L.Layout(len(seq_start) - 1, int(seq_start[-1]), self.block_table_h.shape[1],
                               rope_tab.shape[0], self.seq_start.data_ptr(),
                               self.block_table.data_ptr(),
                               None if self.pos_offset is None else self.pos_offset.data_ptr(),
                               rope_tab.data_ptr())


def rope_table(theta: float, head_dim: int, n_pos: int, device) -> torch.Tensor:
    return torch.from_numpy(L.sx_rope_table(theta, head_dim, n_pos)).to(device)


def workspace(op: int, dims: L.Dims, n_tok: int, n_rows: int, n_req: int, device) -> torch.Tensor:
    nbytes = L.sx_workspace_bytes(op, dims, n_tok, n_rows, n_req)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def gather_logical(pool: PagePool, block_row: np.ndarray, n_tok: int):
    """Read a request's cache back as logical [T, Hkv, d] K and V (host)."""
    pages = torch.as_tensor(np.asarray(block_row[:(n_tok + PAGE - 1) // PAGE], dtype=np.int64),
                            device=pool.k.device)
    k = pool.k.index_select(0, pages).permute(0, 2, 1, 3).reshape(-1, pool.k.shape[1], pool.k.shape[3])
    v = pool.v.index_select(0, pages).permute(0, 3, 1, 2).reshape(-1, pool.v.shape[1], pool.v.shape[2])
    return k[:n_tok].float().cpu().double().numpy(), v[:n_tok].float().cpu().double().numpy()


class SparseXLayerRun:
    """Runs one SparseX layer for a seeded synthetic case (see synth.py).

    Steps (selection inside the layer, i.e. threshold at this layer):
      build caches    -- each reused segment's K/V at its original positions
                         (sx_recompute_kv with a per-request RoPE offset)
      realign         -- sx_rope_realign into the request's own pages
      Sparse-Q rows   -- sx_recompute_kv(I_nr) -> K/V pages, Q_sq
      probe + top-k   -- sx_select_topk -> S and A = I_nr U S
      recompute A     -- sx_recompute_kv(A) -> K/V pages (S overwritten), Q_A
      attention       -- sx_sparse_attn(A) -> O
    """

    def __init__(self, case, device="cuda", ratios=None, extra_guard_pages: int = 8,
                 overflow_tokens: int = 0, keep_probe_cache: bool = False):
        import torch as _t
        from . import synth
        self.case = case
        self.device = device
        # keep a device copy of the K pool as the selection read it (after the
        # realignment and the Sparse-Q rows, before the selected rows are
        # recomputed), for inspection
        self.keep_probe_cache = keep_probe_cache
        self.probe_k = None
        d = case.dims
        self.dims = d
        self.cdims = make_dims(d)
        self.dt = storage_dtype(d.dtype)
        n_req = len(case.requests)
        ratios = ratios or [rq.ratio for rq in case.requests]
        reqs = [([(kind == "reuse", n) for kind, n in case.piece_lengths(r)], ratios[r])
                for r in range(n_req)]
        self.plan = L.sx_plan_layout(reqs, overflow_tokens=overflow_tokens)
        seq_start = self.plan["seq_start"]
        self.n_tok = int(seq_start[-1])
        lens = np.diff(seq_start)
        # pages: requests' pages, then segment caches, then unused guard pages,
        # all drawn from one shuffled pool
        req_pages = [(int(n) + PAGE - 1) // PAGE for n in lens]
        seg_ids = sorted(case.segments)
        seg_pages = [(case.segments[s].length + PAGE - 1) // PAGE for s in seg_ids]
        n_pages = sum(req_pages) + sum(seg_pages) + extra_guard_pages
        perm = synth.page_permutation(case.page_perm_seed, n_pages)
        self.max_pages = max(req_pages)
        bt = np.full((n_req, self.max_pages), -1, dtype=np.int32)
        o = 0
        for r, n in enumerate(req_pages):
            bt[r, :n] = perm[o:o + n]
            o += n
        self.block_table = bt
        self.seg_page_off = {}
        seg_page_ids = []
        for s, n in zip(seg_ids, seg_pages):
            self.seg_page_off[s] = len(seg_page_ids)
            seg_page_ids.extend(perm[o:o + n].tolist())
            o += n
        self.seg_page_ids = np.array(seg_page_ids, dtype=np.int32)
        self.guard_pages = perm[o:].copy()
        self.pool = PagePool.alloc(n_pages, d, device)
        max_pos = max(self.n_tok, max(case.segments[s].p_src + case.segments[s].length
                                      for s in seg_ids)) + 1
        self.rope = rope_table(d.theta, d.head_dim, max_pos + 16, device)
        self.lay = DeviceLayout(seq_start, bt, self.rope, device)
        x = np.concatenate([case.request_x(r) for r in range(n_req)], axis=0)
        self.x = torch.from_numpy(x).to(self.dt).to(device)
        self.w = torch.from_numpy(case.w_qkv()).to(self.dt).to(device)

    # -- cache building ----------------------------------------------------------
    def build_caches(self):
        """K/V of every segment, computed alone at its original positions."""
        case, d = self.case, self.dims
        seg_ids = sorted(case.segments)
        lens = [case.segments[s].length for s in seg_ids]
        seq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        maxp = max((n + PAGE - 1) // PAGE for n in lens)
        bt = np.full((len(seg_ids), maxp), -1, dtype=np.int32)
        for i, s in enumerate(seg_ids):
            n = (lens[i] + PAGE - 1) // PAGE
            off = self.seg_page_off[s]
            bt[i, :n] = self.seg_page_ids[off:off + n]
        pos0 = np.array([case.segments[s].p_src for s in seg_ids], dtype=np.int32)
        lay = DeviceLayout(seq, bt, self.rope, self.device, pos_offset=pos0)
        xc = np.concatenate([case.segments[s].x_cache for s in seg_ids], axis=0)
        xc = torch.from_numpy(xc).to(self.dt).to(self.device)
        rows = torch.arange(int(seq[-1]), dtype=torch.int32, device=self.device)
        L.sx_recompute_kv(self.cdims, lay.struct, xc, rows, int(seq[-1]), self.w, self.pool.struct(),
                          None)
        self._cache_keepalive = (lay, xc, rows)

    # -- the layer -----------------------------------------------------------------
    def realign(self):
        case = self.case
        segs = []
        for r in range(len(case.requests)):
            for dst, sid in case.reuse_runs(r):
                sg = case.segments[sid]
                segs.append(dict(req=r, dst_start=dst, len=sg.length, p_src=sg.p_src,
                                 src_slot0=0, src_pages_off=self.seg_page_off[sid]))
        jobs = L.sx_plan_realign(segs, self.seg_page_ids, self.block_table)
        self.jobs_h = jobs
        self.jobs = torch.from_numpy(jobs).to(self.device)
        pages = self.pool.struct()
        L.sx_rope_realign(self.cdims, self.lay.struct, pages, pages, self.jobs, len(jobs))

    def run(self, build_caches: bool = True):
        dev, d, cd = self.device, self.dims, self.cdims
        if build_caches:
            self.build_caches()
        self.realign()
        plan = self.plan
        n_req = len(self.case.requests)
        pages = self.pool.struct()
        sq_rows = torch.from_numpy(plan["sq_rows"]).to(dev)
        sq_start = torch.from_numpy(plan["sq_start"]).to(dev)
        n_sq = int(plan["sq_start"][-1])
        tok_class = torch.from_numpy(plan["tok_class"]).to(dev)
        k = plan["k"]
        k_sel = torch.from_numpy(k).to(dev)
        self.q_sq = torch.empty((n_sq, d.n_q_heads, d.head_dim), dtype=self.dt, device=dev)
        L.sx_recompute_kv(cd, self.lay.struct, self.x, sq_rows, n_sq, self.w, pages, self.q_sq)
        n_sel = int(k.sum())
        n_act = n_sq + n_sel
        self.sel_rows = torch.empty(max(n_sel, 1), dtype=torch.int32, device=dev)
        self.act_rows = torch.empty(max(n_act, 1), dtype=torch.int32, device=dev)
        self.scores = torch.empty(self.n_tok, dtype=torch.float32, device=dev)
        ws = workspace(L.SX_OP_SELECT, cd, self.n_tok, n_sq, n_req, dev)
        L.sx_select_topk(cd, self.lay.struct, self.q_sq, None, sq_rows, sq_start, n_sq, None, pages,
                         tok_class, k_sel, self.sel_rows, self.act_rows, self.scores, ws)
        if self.keep_probe_cache:
            self.probe_k = self.pool.k.clone()
        act_start_h = (plan["sq_start"] + np.concatenate([[0], np.cumsum(k)])).astype(np.int32)
        self.act_start = torch.from_numpy(act_start_h).to(dev)
        self.q_act = torch.empty((n_act, d.n_q_heads, d.head_dim), dtype=self.dt, device=dev)
        L.sx_recompute_kv(cd, self.lay.struct, self.x, self.act_rows, n_act, self.w, pages, self.q_act)
        self.o = torch.empty((n_act, d.n_q_heads * d.head_dim), dtype=self.dt, device=dev)
        self.lse = torch.empty((n_act, d.n_q_heads), dtype=torch.float32, device=dev)
        ws2 = workspace(L.SX_OP_SPARSE_ATTN, cd, self.n_tok, n_act, n_req, dev)
        L.sx_sparse_attn(cd, self.lay.struct, self.q_act, self.act_rows, self.act_start, n_act, pages,
                         self.o, self.lse, ws2)
        self._keepalive = (sq_rows, sq_start, tok_class, k_sel, ws, ws2)
        return self

    # -- readback helpers ------------------------------------------------------------
    def request_cache(self, r: int):
        T = int(self.plan["seq_start"][r + 1] - self.plan["seq_start"][r])
        return gather_logical(self.pool, self.block_table[r], T)

    def probe_keys(self, r: int):
        """Request r's keys as the selection read them ([T, Hkv, d], host);
        needs keep_probe_cache."""
        T = int(self.plan["seq_start"][r + 1] - self.plan["seq_start"][r])
        k, _ = gather_logical(PagePool(self.probe_k, self.pool.v), self.block_table[r], T)
        return k

    def sq_queries(self, r: int):
        """Request r's Sparse-Q query rows as stored ([n_sq_r, Hq, d], host)."""
        a, b = int(self.plan["sq_start"][r]), int(self.plan["sq_start"][r + 1])
        return self.q_sq[a:b].float().cpu().double().numpy()
