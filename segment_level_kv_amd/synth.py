"""Seeded synthetic inputs for the SparseX prefill layer.

This module produces *inputs only*: weights, layer inputs, segment layouts,
original cache offsets, selection ratios and page shuffles.  It holds none of
the method's arithmetic (no RoPE, no projection, no attention, no selection),
so both the GPU path and the CPU oracle can consume what it makes without
sharing any computation.

Workload shapes follow the evaluation settings of "SparseX: Efficient
Segment-Level KV Cache Sharing for Interleaved LLM Serving" (arXiv
2606.01751): §5 builds each test as a cache-building request followed by an
evaluation request that recombines cached segments with new text; App. B
describes 16K contexts made of 4K segments, agent prompts and chat prompts
(instruction + reused history + question).  The datasets themselves (LOCOMO,
LongMemEval, RULER, MASLab) are not used: seeded Gaussian values with the
same shapes stand in for them.

Value recipe: X ~ N(0,1) per element, then RMSNorm (unit gain) per row;
W ~ N(0, 1/hidden).  Both are cast to the storage type (torch's
round-to-nearest-even float32 -> bfloat16 cast for bf16).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16


@dataclass(frozen=True)
class Dims:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    theta: float
    dtype: str            # "bf16" or "f32"
    page_size: int = PAGE_SIZE
    eps: float = 1e-5     # RMSNorm epsilon of the input recipe

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass
class Segment:
    """A reused segment: its layer input rows and where it was cached."""
    seg_id: int
    length: int
    p_src: int                 # original start position of the cached copy
    x: np.ndarray              # [L, hidden] storage values (float64)
    x_cache: np.ndarray        # [L, hidden] the rows the cache was built from


@dataclass
class Request:
    """pieces: ("reuse", seg_id) or ("new", index into new_x)."""
    pieces: list
    new_x: list                # list of [L, hidden] float64 arrays
    ratio: tuple               # (num, den)


@dataclass
class LayerCase:
    name: str
    dims: Dims
    wq: np.ndarray             # [Hq*d, hidden] float64 storage values
    wk: np.ndarray             # [Hkv*d, hidden]
    wv: np.ndarray
    segments: dict             # seg_id -> Segment
    requests: list             # list of Request
    page_perm_seed: int
    extra: dict = field(default_factory=dict)

    # ---- plain views (no method arithmetic) --------------------------------
    def piece_lengths(self, r: int):
        """[("reuse"|"new", L), ...] of request r."""
        out = []
        for kind, ref in self.requests[r].pieces:
            if kind == "reuse":
                out.append(("reuse", self.segments[ref].length))
            else:
                out.append(("new", self.requests[r].new_x[ref].shape[0]))
        return out

    def request_x(self, r: int) -> np.ndarray:
        """Layer input rows of request r in token order [T, hidden]."""
        rows = []
        for kind, ref in self.requests[r].pieces:
            if kind == "reuse":
                rows.append(self.segments[ref].x)
            else:
                rows.append(self.requests[r].new_x[ref])
        return np.concatenate(rows, axis=0)

    def reuse_runs(self, r: int):
        """[(dst_start, seg_id), ...] for the reused runs of request r."""
        out, start = [], 0
        for kind, ref in self.requests[r].pieces:
            L = self.segments[ref].length if kind == "reuse" else self.requests[r].new_x[ref].shape[0]
            if kind == "reuse":
                out.append((start, ref))
            start += L
        return out

    def n_tokens(self, r: int) -> int:
        return sum(L for _, L in self.piece_lengths(r))

    def w_qkv(self) -> np.ndarray:
        """Rows of W_q, then W_k, then W_v: [(Hq+2Hkv)*d, hidden]."""
        return np.concatenate([self.wq, self.wk, self.wv], axis=0)


# ---------------------------------------------------------------------------
# value helpers
# ---------------------------------------------------------------------------

def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float values to the storage type; returned as float64 values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).to(torch.float64).numpy()
    if dtype == "f32":
        return t.to(torch.float64).numpy()
    raise ValueError(dtype)


def torch_storage(a: np.ndarray, dtype: str):
    """Storage-typed CPU torch tensor holding exactly the values of `a`."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _rmsnormed_gaussian(rng: np.random.Generator, n: int, hidden: int, eps: float) -> np.ndarray:
    x = rng.standard_normal((n, hidden), dtype=np.float32).astype(np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)


def _weights(rng, dims: Dims):
    std = 1.0 / np.sqrt(dims.hidden)
    mk = lambda rows: to_storage(rng.standard_normal((rows, dims.hidden), dtype=np.float32) * std,
                                 dims.dtype)
    wq = mk(dims.n_q_heads * dims.head_dim)
    wk = mk(dims.n_kv_heads * dims.head_dim)
    wv = mk(dims.n_kv_heads * dims.head_dim)
    return wq, wk, wv


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


# ---------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------

TINY = Dims(hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64, theta=1e4, dtype="f32")
LLAMA8B = Dims(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, theta=5e5, dtype="bf16")
QWEN7B = Dims(hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, theta=1e6, dtype="bf16",
              eps=1e-6)


def make_case(name: str, dims: Dims, seg_lengths, layouts, ratios, seed: int,
              p_src_max=None, p_src_fixed=None, cache_noise: float = 0.0,
              x_cache_fn=None) -> LayerCase:
    """Generic builder.

    seg_lengths: list of segment lengths (seg_id = index).
    layouts: per request, list of ("reuse", seg_id) / ("new", L).
    ratios: per request (num, den).
    p_src_max: original offsets drawn uniformly in [0, p_src_max - L]
    (inclusive), unless p_src_fixed gives them.
    cache_noise > 0: the cache of a segment is built from
    RMSNorm(X + cache_noise * N(0,1)) instead of X (a stand-in for the
    context dependence of a deeper layer's input).
    """
    r_w, r_seg, r_off, r_new, r_noise, r_page = _streams(seed, 6)
    wq, wk, wv = _weights(r_w, dims)
    segments = {}
    for sid, L in enumerate(seg_lengths):
        x = to_storage(_rmsnormed_gaussian(r_seg, L, dims.hidden, dims.eps), dims.dtype)
        if p_src_fixed is not None:
            p = int(p_src_fixed[sid])
        else:
            p = int(r_off.integers(0, max(p_src_max - L, 0) + 1))
        if cache_noise > 0:
            noisy = x + cache_noise * r_noise.standard_normal(x.shape)
            xc = to_storage(noisy / np.sqrt(np.mean(noisy * noisy, axis=1, keepdims=True)
                                            + dims.eps), dims.dtype)
        else:
            xc = x
        segments[sid] = Segment(sid, L, p, x, xc)
    requests = []
    for lay, ratio in zip(layouts, ratios):
        pieces, new_x = [], []
        for kind, v in lay:
            if kind == "reuse":
                pieces.append(("reuse", int(v)))
            else:
                new_x.append(to_storage(_rmsnormed_gaussian(r_new, int(v), dims.hidden, dims.eps),
                                        dims.dtype))
                pieces.append(("new", len(new_x) - 1))
        requests.append(Request(pieces, new_x, tuple(ratio)))
    return LayerCase(name, dims, wq, wk, wv, segments, requests,
                     page_perm_seed=int(r_page.integers(0, 2**31 - 1)))


def tiny_case(seed: int = 1001, ratio=(25, 100), cache_noise: float = 0.0) -> LayerCase:
    """hidden 256, 4 q / 1 kv heads, d 64, fp32.  Two reused segments of 64
    tokens cached at random original offsets in [0, 512), then 16 new
    tokens.  Ratio 25%."""
    return make_case("tiny", TINY, [64, 64], [[("reuse", 0), ("reuse", 1), ("new", 16)]],
                     [ratio], seed, p_src_max=512, cache_noise=cache_noise)


def llama_layer_case(seed: int = 1002, ratio=(15, 100), n_seg: int = 8, seg_len: int = 512,
                     suffix: int = 256, cache_noise: float = 0.0, dims: Dims = LLAMA8B) -> LayerCase:
    """Llama-3-8B-shaped single layer in bf16: 8 reused segments of 512
    tokens, each cached alone at an offset in [0, 8192-512], plus a 256-token
    new suffix (4,352 tokens).  Ratio 15%."""
    lay = [("reuse", i) for i in range(n_seg)] + ([("new", suffix)] if suffix else [])
    return make_case("llama1l", dims, [seg_len] * n_seg, [lay], [ratio], seed,
                     p_src_max=8192, cache_noise=cache_noise)


def interleaved_case(seed: int = 1005, ratio=(20, 100), dims: Dims = LLAMA8B) -> LayerCase:
    """Two requests whose new runs sit between reused segments (the layout
    the overflow blocks of §3.3 are meant for), sharing segments 1 and 3:
      r0: new 40 | seg0 300 | new 24 | seg1 200 | seg2 20 | new 8 | seg3 150
      r1: seg3 150 | new 5 | seg1 200 | new 33
    r0 ends on a reused segment (tail fallback), r1 on new tokens."""
    lay0 = [("new", 40), ("reuse", 0), ("new", 24), ("reuse", 1), ("reuse", 2), ("new", 8),
            ("reuse", 3)]
    lay1 = [("reuse", 3), ("new", 5), ("reuse", 1), ("new", 33)]
    return make_case("interleaved", dims, [300, 200, 20, 150], [lay0, lay1], [ratio, ratio],
                     seed, p_src_max=4096)


def rag_layout(n_passages: int = 16, system: int = 512, passage: int = 1920, query: int = 256):
    """RAG mix: reused system segment + reused passages + new query.

    Returns (seg_lengths, layout, p_src): the system segment was cached
    alone at 0 and each passage in a [system | passage] request at `system`.
    """
    seg_lengths = [system] + [passage] * n_passages
    layout = [("reuse", i) for i in range(n_passages + 1)] + [("new", query)]
    p_src = [0] + [system] * n_passages
    return seg_lengths, layout, p_src


def rag32k_case(seed: int = 1003, ratio=(10, 100), n_passages: int = 16) -> LayerCase:
    """One layer of the RAG mix on Llama-3-8B shapes (31,488 tokens)."""
    seg_lengths, layout, p_src = rag_layout(n_passages)
    return make_case("rag32k", LLAMA8B, seg_lengths, [layout], [ratio], seed,
                     p_src_fixed=p_src)


def agent_layout(seed: int = 1004, n_pool: int = 64, n_req: int = 4, target: int = 65536,
                 lmin: int = 32, lmax: int = 2048):
    """Agent interleave: a pool of segments with log-uniform lengths in
    [lmin, lmax] rounded to a multiple of 16; each request concatenates
    freshly permuted passes over the pool until the next segment would pass
    `target` tokens.  No new tokens.  Ratios uniform in [5%, 30%] (in 1/1000
    steps).  Returns (seg_lengths, layouts, ratios)."""
    rng = np.random.default_rng(seed)
    raw = np.exp(rng.uniform(np.log(lmin), np.log(lmax), n_pool))
    lengths = [int(max(PAGE_SIZE, PAGE_SIZE * round(v / PAGE_SIZE))) for v in raw]
    layouts, ratios = [], []
    for _ in range(n_req):
        lay, total, done = [], 0, False
        while not done:
            for sid in rng.permutation(n_pool):
                if total + lengths[sid] > target:
                    done = True
                    break
                lay.append(("reuse", int(sid)))
                total += lengths[sid]
        layouts.append(lay)
        ratios.append((int(rng.integers(50, 301)), 1000))
    return lengths, layouts, ratios


def agent_case(seed: int = 1004, n_req: int = 4, target: int = 65536, n_pool: int = 64,
               lmax: int = 2048) -> LayerCase:
    lengths, layouts, ratios = agent_layout(seed, n_pool, n_req, target, lmax=lmax)
    return make_case("agent64k", LLAMA8B, lengths, layouts, ratios, seed + 17, p_src_max=8192)


def chat_layout(instruction: int = 120, history: int = 31000, question: int = 80,
                block: int = 16):
    """Multi-round chat prompt: a fixed instruction prefix, the reused
    conversation history and the question (Appendix B.1 prompt shape).

    The history was cached alone, from position 0, by an earlier request;
    only its whole blocks were cached (the final, incomplete block is not),
    so its last history % block tokens are recomputed with the new text.
    Returns (seg_lengths, layout, p_src)."""
    cached = (history // block) * block
    layout = [("new", instruction), ("reuse", 0)]
    if history > cached:
        layout.append(("new", history - cached))
    layout.append(("new", question))
    return [cached], layout, [0]


def qwen_layout(n_seg: int = 32, seg_len: int = 4000, suffix: int = 1024):
    seg_lengths = [seg_len] * n_seg
    layout = [("reuse", i) for i in range(n_seg)] + [("new", suffix)]
    return seg_lengths, layout


def qwen128k_case(seed: int = 1005, ratio=(10, 100)) -> LayerCase:
    """One sparse layer of the long-context mix on Qwen2.5-7B shapes: 32
    reused segments of 4,000 tokens, each cached alone at an offset in
    [0, 128K - 4000], then a 1,024-token new suffix (129,024 tokens)."""
    seg_lengths, layout = qwen_layout()
    return make_case("qwen128k", QWEN7B, seg_lengths, [layout], [ratio], seed,
                     p_src_max=128 * 1024)


def page_permutation(seed: int, n_pages: int) -> np.ndarray:
    """Seeded shuffle of physical page ids (so block tables are not
    contiguous)."""
    return np.random.default_rng(seed).permutation(n_pages).astype(np.int32)


def gaussian(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Plain seeded N(0, scale^2) float64 array (for kernel-level inputs)."""
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# device-side generation for large workloads (same recipe, torch generator)
# ---------------------------------------------------------------------------

def torch_rmsnormed_rows(gen, n: int, hidden: int, eps: float, dtype, device):
    """N(0,1) rows, RMSNorm with unit gain, cast to the storage type."""
    import torch
    x = torch.randn((n, hidden), generator=gen, device=device, dtype=torch.float32)
    x = x * torch.rsqrt(torch.mean(x * x, dim=1, keepdim=True) + eps)
    return x.to(dtype)


def torch_weights(gen, dims: Dims, dtype, device):
    """W_qkv rows (W_q, W_k, W_v) ~ N(0, 1/hidden) in the storage type."""
    import torch
    w = torch.randn((dims.qkv_rows, dims.hidden), generator=gen, device=device, dtype=torch.float32)
    return (w * (1.0 / np.sqrt(dims.hidden))).to(dtype)


class TorchStackInputs:
    """Per-layer (x, w_qkv, x_cache) generated once on the device."""

    def __init__(self, seed: int, dims: Dims, n_layers: int, n_tok: int, n_cache_tok: int,
                 threshold: int, device):
        import torch
        dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        self.layers = []
        for l in range(n_layers):
            x = torch_rmsnormed_rows(gen, n_tok, dims.hidden, dims.eps, dt, device)
            w = torch_weights(gen, dims, dt, device)
            xc = (torch_rmsnormed_rows(gen, n_cache_tok, dims.hidden, dims.eps, dt, device)
                  if l >= threshold else None)
            self.layers.append((x, w, xc))

    def __call__(self, l: int):
        return self.layers[l]
