"""ctypes binding of libsx (include/sx.h).

Argument marshalling only: every function here converts Python / torch
arguments into the C ABI's plain pointers and sizes and calls the function of
the same name in libsx.so.  Nothing is computed here.  If the library is not
built this module raises on first use; there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsx.so")

SX_OK, SX_EINVAL, SX_EUNSUPPORTED, SX_EWORKSPACE, SX_EDEVICE, SX_ENOMEM = 0, -1, -2, -3, -4, -5
SX_F32, SX_BF16 = 0, 1
SX_OP_REALIGN, SX_OP_RECOMPUTE, SX_OP_SELECT, SX_OP_TOPK, SX_OP_SPARSE_ATTN, SX_OP_FULL_ATTN, SX_OP_DECODE = range(7)

EXPORTED = [
    "sx_rope_table", "sx_plan_layout", "sx_plan_realign", "sx_realign_jobs_bound",
    "sx_workspace_bytes", "sx_rope_realign", "sx_recompute_kv", "sx_recompute_kv_realign", "sx_select_topk",
    "sx_topk",
    "sx_sparse_attn", "sx_sparse_attn_plan", "sx_sparse_attn_run", "sx_full_attn", "sx_decode_attn", "sx_decode_attn_noalloc", "sx_mfma_peak_probe", "sx_last_error",
    "sx_virtual_hash", "sx_index_create", "sx_index_destroy", "sx_index_alloc", "sx_index_release",
    "sx_index_insert", "sx_index_lookup", "sx_index_remove", "sx_index_stats", "sx_plan_segments",
]


class SxError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class Dims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("page_size", C.c_int32), ("dtype", C.c_int32)]


class Pages(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n_pages", C.c_int32)]


class Layout(C.Structure):
    _fields_ = [("n_req", C.c_int32), ("n_tok", C.c_int32), ("max_pages", C.c_int32),
                ("rope_len", C.c_int32), ("seq_start", C.c_void_p), ("block_table", C.c_void_p),
                ("pos_offset", C.c_void_p), ("rope_tab", C.c_void_p)]


class RealignJob(C.Structure):
    _fields_ = [("src_page", C.c_int32), ("dst_page", C.c_int32), ("src_slot", C.c_int32),
                ("dst_slot", C.c_int32), ("n_tok", C.c_int32), ("delta", C.c_int32)]


class Segment(C.Structure):
    _fields_ = [("req", C.c_int32), ("dst_start", C.c_int32), ("len", C.c_int32),
                ("p_src", C.c_int32), ("src_slot0", C.c_int32), ("src_pages_off", C.c_int32)]


_lib = None


def lib():
    """The loaded libsx.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m segment_level_kv_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I, Z, D, U = C.c_void_p, C.c_int32, C.c_size_t, C.c_double, C.c_uint64
        sig = {
            "sx_rope_table": (I, [D, I, I, P]),
            "sx_plan_layout": (I, [I, P, P, P, P, P, I, I, I, P, P, P, P, P, P]),
            "sx_plan_realign": (I, [P, I, P, I, P, I, I, I, P, P, I, P]),
            "sx_realign_jobs_bound": (I, [P, I, I]),
            "sx_workspace_bytes": (Z, [I, P, I, I, I]),
            "sx_rope_realign": (I, [P, P, P, P, P, I, P]),
            "sx_recompute_kv": (I, [P, P, P, P, I, P, P, P, P]),
            "sx_recompute_kv_realign": (I, [P, P, P, P, I, P, P, P, P, P, P, I, P]),
            "sx_select_topk": (I, [P, P, P, P, P, P, I, P, P, P, P, P, P, P, P, Z, P]),
            "sx_topk": (I, [P, P, P, I, I, P, P, P, Z, P]),
            "sx_sparse_attn": (I, [P, P, P, P, P, I, P, P, P, P, Z, P]),
            "sx_sparse_attn_plan": (I, [P, P, P, P, I, P, Z, P]),
            "sx_sparse_attn_run": (I, [P, P, P, P, I, P, P, P, P, Z, P]),
            "sx_full_attn": (I, [P, P, P, P, P, P, P, Z, P]),
            "sx_decode_attn": (I, [P, P, P, P, P, P, P, Z, P]),
            "sx_decode_attn_noalloc": (I, [P, P, P, P, P, P, P]),
            "sx_mfma_peak_probe": (I, [I, I, I, P, P]),
            "sx_last_error": (C.c_char_p, []),
            "sx_virtual_hash": (I, [P, I, U, P]),
            "sx_index_create": (I, [I, I, I, I, P]),
            "sx_index_destroy": (None, [P]),
            "sx_index_alloc": (I, [P, I, P]),
            "sx_index_release": (I, [P, P, I]),
            "sx_index_insert": (I, [P, P, I, U, P, I, I]),
            "sx_index_lookup": (I, [P, P, I, U, P, P]),
            "sx_index_remove": (I, [P, P, I]),
            "sx_index_stats": (I, [P, P]),
            "sx_plan_segments": (I, [I, I, P, P, I, I, I, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().sx_last_error().decode()


def _check(st: int, fn: str):
    if st != SX_OK:
        raise SxError(st, fn, last_error())


def _ptr(t):
    """Device/host address of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _ref(s):
    return None if s is None else C.addressof(s)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# host planners
# ---------------------------------------------------------------------------

def sx_rope_table(theta: float, head_dim: int, n_pos: int) -> np.ndarray:
    tab = np.empty((n_pos, head_dim // 2, 2), dtype=np.float32)
    _check(lib().sx_rope_table(float(theta), head_dim, n_pos, _ptr(tab)), "sx_rope_table")
    return tab


def sx_plan_layout(requests, fallback_tokens: int = 64, overflow_tokens: int = 0):
    """requests: list of (pieces, (num, den)); pieces = [(is_reuse, length)].

    Returns dict of numpy arrays: seq_start, tok_class, sq_rows, sq_start,
    n_cand, k."""
    n_req = len(requests)
    piece_start = [0]
    reuse, lens, num, den = [], [], [], []
    for pieces, (a, b) in requests:
        for is_reuse, L in pieces:
            reuse.append(1 if is_reuse else 0)
            lens.append(int(L))
        piece_start.append(len(lens))
        num.append(int(a))
        den.append(int(b))
    n_cap = max(1, sum(lens))
    a32 = lambda v: np.ascontiguousarray(np.array(v, dtype=np.int32).reshape(-1))
    ps, ru, ln, nu, de = a32(piece_start), a32(reuse or [0]), a32(lens or [0]), a32(num), a32(den)
    seq_start = np.zeros(n_req + 1, np.int32)
    tok_class = np.zeros(n_cap, np.uint8)
    sq_rows = np.zeros(n_cap, np.int32)
    sq_start = np.zeros(n_req + 1, np.int32)
    n_cand = np.zeros(n_req, np.int32)
    k = np.zeros(n_req, np.int32)
    _check(lib().sx_plan_layout(n_req, _ptr(ps), _ptr(ru), _ptr(ln), _ptr(nu), _ptr(de),
                                fallback_tokens, overflow_tokens, n_cap, _ptr(seq_start),
                                _ptr(tok_class),
                                _ptr(sq_rows), _ptr(sq_start), _ptr(n_cand), _ptr(k)),
           "sx_plan_layout")
    n_tok = int(seq_start[-1])
    return dict(seq_start=seq_start, tok_class=tok_class[:n_tok], sq_rows=sq_rows[:sq_start[-1]],
                sq_start=sq_start, n_cand=n_cand, k=k)


def _i32(v):
    return np.ascontiguousarray(np.asarray(v, dtype=np.int32).reshape(-1))


def sx_virtual_hash(tokens, extra_key: int) -> int:
    t = _i32(tokens)
    out = np.zeros(1, np.uint64)
    _check(lib().sx_virtual_hash(_ptr(t), len(t), int(extra_key), _ptr(out)), "sx_virtual_hash")
    return int(out[0])


class SegmentIndex:
    """Owner of one sx_index (the block pool and its virtual-block index)."""

    def __init__(self, n_blocks: int, block_size: int = 16, evict_num: int = 9,
                 evict_den: int = 10):
        h = C.c_void_p()
        _check(lib().sx_index_create(n_blocks, block_size, evict_num, evict_den, C.byref(h)),
               "sx_index_create")
        self._h = h
        self.block_size = block_size

    def close(self):
        if self._h:
            lib().sx_index_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int) -> list:
        ids = np.zeros(max(n, 1), np.int32)
        _check(lib().sx_index_alloc(self._h, n, _ptr(ids)), "sx_index_alloc")
        return ids[:n].tolist()

    def release(self, ids):
        a = _i32(ids)
        _check(lib().sx_index_release(self._h, _ptr(a), len(a)), "sx_index_release")

    def insert(self, tokens, extra_key: int, ids, p_src: int, frozen: bool):
        t, a = _i32(tokens), _i32(ids)
        _check(lib().sx_index_insert(self._h, _ptr(t), len(t), int(extra_key), _ptr(a), p_src,
                                     1 if frozen else 0), "sx_index_insert")

    def lookup(self, tokens, extra_key: int):
        t = _i32(tokens)
        nb = len(t) // self.block_size
        blk, pos = np.zeros(max(nb, 1), np.int32), np.zeros(max(nb, 1), np.int32)
        _check(lib().sx_index_lookup(self._h, _ptr(t), len(t), int(extra_key), _ptr(blk),
                                     _ptr(pos)), "sx_index_lookup")
        return blk[:nb].tolist(), pos[:nb].tolist()

    def remove(self, ids):
        a = _i32(ids)
        _check(lib().sx_index_remove(self._h, _ptr(a), len(a)), "sx_index_remove")

    def stats(self):
        st = np.zeros(4, np.int32)
        _check(lib().sx_index_stats(self._h, _ptr(st)), "sx_index_stats")
        return tuple(int(x) for x in st)


def sx_plan_segments(req: int, dst_start: int, blocks, pos, n_tok: int, block_size: int = 16,
                     ids_off: int = 0):
    """Returns (segments as dicts, src_ids list, pieces [(is_reuse, L)])."""
    b, p = _i32(blocks), _i32(pos)
    cap = n_tok // block_size + 1
    segs = (Segment * cap)()
    ids = np.zeros(cap, np.int32)
    reuse, lens = np.zeros(cap, np.int32), np.zeros(cap, np.int32)
    ns, ni, npc = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib().sx_plan_segments(req, dst_start, _ptr(b) if len(b) else None,
                                  _ptr(p) if len(p) else None, n_tok, block_size, ids_off, segs,
                                  C.byref(ns), _ptr(ids), C.byref(ni), _ptr(reuse), _ptr(lens),
                                  C.byref(npc)), "sx_plan_segments")
    out = [dict(req=s.req, dst_start=s.dst_start, len=s.len, p_src=s.p_src, src_slot0=s.src_slot0,
                src_pages_off=s.src_pages_off) for s in segs[:ns.value]]
    return out, ids[:ni.value].tolist(), [(bool(reuse[i]), int(lens[i])) for i in range(npc.value)]


def sx_plan_realign(segments, src_page_ids: np.ndarray, block_table: np.ndarray,
                    pos_offset=None, page_size: int = 16) -> np.ndarray:
    """segments: list of dict(req, dst_start, len, p_src, src_slot0,
    src_pages_off).  Returns a structured int32 array [n_jobs, 6]."""
    n = len(segments)
    segs = (Segment * max(n, 1))()
    for i, s in enumerate(segments):
        segs[i] = Segment(s["req"], s["dst_start"], s["len"], s["p_src"], s.get("src_slot0", 0),
                          s["src_pages_off"])
    bound = lib().sx_realign_jobs_bound(segs, n, page_size)
    jobs = np.zeros((max(bound, 1), 6), dtype=np.int32)
    n_jobs = C.c_int32(0)
    src = np.ascontiguousarray(src_page_ids, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    po = None if pos_offset is None else np.ascontiguousarray(pos_offset, dtype=np.int32)
    _check(lib().sx_plan_realign(segs, n, _ptr(src), src.size, _ptr(bt), bt.shape[0], bt.shape[1],
                                 page_size, _ptr(po), _ptr(jobs), jobs.shape[0], C.byref(n_jobs)),
           "sx_plan_realign")
    return jobs[:n_jobs.value].copy()


def sx_workspace_bytes(op: int, dims: Dims, n_tok: int, n_rows: int, n_req: int) -> int:
    return int(lib().sx_workspace_bytes(op, _ref(dims), n_tok, n_rows, n_req))


# ---------------------------------------------------------------------------
# device entry points (torch tensors in, nothing returned)
# ---------------------------------------------------------------------------

def sx_rope_realign(dims: Dims, lay: Layout, src: Pages, dst: Pages, jobs, n_jobs: int,
                    stream=None):
    _check(lib().sx_rope_realign(_ref(dims), _ref(lay), _ref(src), _ref(dst), _ptr(jobs), n_jobs,
                                 _stream(stream)), "sx_rope_realign")


def sx_recompute_kv(dims: Dims, lay: Layout, x, rows, n_rows: int, w_qkv, kv: Pages, q_out,
                    stream=None):
    _check(lib().sx_recompute_kv(_ref(dims), _ref(lay), _ptr(x), _ptr(rows), n_rows, _ptr(w_qkv),
                                 _ref(kv), _ptr(q_out), _stream(stream)), "sx_recompute_kv")


def sx_recompute_kv_realign(dims: Dims, lay: Layout, x, rows, n_rows: int, w_qkv, kv: Pages, q_out,
                            rsrc: Pages, rdst: Pages, jobs, n_jobs: int, stream=None):
    _check(lib().sx_recompute_kv_realign(_ref(dims), _ref(lay), _ptr(x), _ptr(rows), n_rows, _ptr(w_qkv),
                                         _ref(kv), _ptr(q_out), _ref(rsrc), _ref(rdst), _ptr(jobs), n_jobs,
                                         _stream(stream)), "sx_recompute_kv_realign")


def sx_select_topk(dims: Dims, lay: Layout, q, q_index, sq_rows, sq_start, n_sq: int, lse,
                   kv: Pages, tok_class, k_sel, sel_rows, act_rows, scores, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sx_select_topk(_ref(dims), _ref(lay), _ptr(q), _ptr(q_index), _ptr(sq_rows),
                                _ptr(sq_start), n_sq, _ptr(lse), _ref(kv), _ptr(tok_class),
                                _ptr(k_sel), _ptr(sel_rows), _ptr(act_rows), _ptr(scores),
                                _ptr(ws), ws_bytes, _stream(stream)), "sx_select_topk")


def sx_topk(scores, tok_class, seq_start, n_req: int, n_tok: int, k_sel, sel_rows, ws,
            stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sx_topk(_ptr(scores), _ptr(tok_class), _ptr(seq_start), n_req, n_tok, _ptr(k_sel),
                         _ptr(sel_rows), _ptr(ws), ws_bytes, _stream(stream)), "sx_topk")


def sx_sparse_attn(dims: Dims, lay: Layout, q, rows, row_start, n_rows: int, kv: Pages, o, lse,
                   ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sx_sparse_attn(_ref(dims), _ref(lay), _ptr(q), _ptr(rows), _ptr(row_start),
                                n_rows, _ref(kv), _ptr(o), _ptr(lse), _ptr(ws), ws_bytes,
                                _stream(stream)), "sx_sparse_attn")


def sx_sparse_attn_plan(dims: Dims, lay: Layout, rows, row_start, n_rows: int, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sx_sparse_attn_plan(_ref(dims), _ref(lay), _ptr(rows), _ptr(row_start), n_rows,
                                     _ptr(ws), ws_bytes, _stream(stream)), "sx_sparse_attn_plan")


def sx_sparse_attn_run(dims: Dims, lay: Layout, q, rows, n_rows: int, kv: Pages, o, lse, ws,
                       stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sx_sparse_attn_run(_ref(dims), _ref(lay), _ptr(q), _ptr(rows), n_rows, _ref(kv),
                                    _ptr(o), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)),
           "sx_sparse_attn_run")


def sx_decode_attn(dims: Dims, lay: Layout, q, kv: Pages, o, lse, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sx_decode_attn(_ref(dims), _ref(lay), _ptr(q), _ref(kv), _ptr(o), _ptr(lse),
                                _ptr(ws), ws_bytes, _stream(stream)), "sx_decode_attn")


def sx_decode_attn_noalloc(dims: Dims, lay: Layout, q, kv: Pages, o, lse, stream=None):
    _check(lib().sx_decode_attn_noalloc(_ref(dims), _ref(lay), _ptr(q), _ref(kv), _ptr(o),
                                        _ptr(lse), _stream(stream)), "sx_decode_attn_noalloc")


def sx_mfma_peak_probe(n_workgroups: int, iters: int, out, stream=None, random_operands: bool = False):
    _check(lib().sx_mfma_peak_probe(int(n_workgroups), int(iters), 1 if random_operands else 0,
                                    _ptr(out), _stream(stream)),
           "sx_mfma_peak_probe")


def sx_full_attn(dims: Dims, lay: Layout, q, kv: Pages, o, lse, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sx_full_attn(_ref(dims), _ref(lay), _ptr(q), _ref(kv), _ptr(o), _ptr(lse),
                              _ptr(ws), ws_bytes, _stream(stream)), "sx_full_attn")
