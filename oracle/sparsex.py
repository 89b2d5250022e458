"""Plain float64 CPU oracle of one SparseX prefill layer (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module.  It shares no code with the GPU
path and imports nothing from it.

Source: "SparseX: Efficient Segment-Level KV Cache Sharing for Interleaved
LLM Serving" (arXiv 2606.01751).  Citations below name the section and which
display equation of that section they follow; the paper's equations carry no
numbers, so "§3.1 eq. b" means the second display equation of §3.1.

Where the paper leaves a step open, the reading used is stated in the
docstring of the function that takes it.  All arithmetic is float64; values
are rounded to the storage type ("bf16" or "f32") exactly where the layer
stores them.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "round_bf16",
    "round_store",
    "rope_inv_freq",
    "rope_rotate",
    "realign_segment",
    "plan_request",
    "project_rows",
    "causal_attention",
    "attention_mass_scores",
    "select_topk",
    "sparse_layer",
    "full_layer",
]

# ---------------------------------------------------------------------------
# Storage rounding
# ---------------------------------------------------------------------------

_BF16_DROP = 45                      # float64 keeps 52 fraction bits, bf16 keeps 7
_FP32_MIN_NORMAL = 2.0 ** -126       # bf16 shares float32's exponent range
_BF16_SUBNORMAL_STEP = 2.0 ** -133   # spacing of bf16 subnormals
_BF16_OVERFLOW = 2.0 ** 128


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Returned as float64 holding bf16-representable values.  The rounding is
    done once, directly from float64 (no intermediate float32 rounding).
    Normal range: round the 52-bit fraction to 7 bits on the raw bit
    pattern (a carry into the exponent is the correct result).  Below the
    float32 normal range: round to the bf16 subnormal grid.  Overflow goes
    to +-inf; NaN stays NaN.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(_BF16_DROP)) & np.uint64(1)
    half_minus_one = np.uint64((1 << (_BF16_DROP - 1)) - 1)
    mask = ~np.uint64((1 << _BF16_DROP) - 1)
    rounded = ((bits + half_minus_one + lsb) & mask).view(np.float64)
    small = np.abs(x) < _FP32_MIN_NORMAL
    if np.any(small):
        sub = np.round(x / _BF16_SUBNORMAL_STEP) * _BF16_SUBNORMAL_STEP
        rounded = np.where(small, sub, rounded)
    rounded = np.where(np.abs(rounded) >= _BF16_OVERFLOW, np.copysign(np.inf, x), rounded)
    rounded = np.where(np.isnan(x), x, rounded)
    return rounded


def round_store(x, dtype: str) -> np.ndarray:
    """Round to the storage type of the layer: "bf16" or "f32" (both RNE)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ---------------------------------------------------------------------------
# RoPE -- paper §3.1, eq. b (k_m = R_m k, q_m = R_m q) and eq. d (delta)
# ---------------------------------------------------------------------------

def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """Rotation frequencies omega_i = theta^(-2i/d), i < d/2 (float64).

    The paper gives only the rotation R_m (§3.1 eq. b).  Reading taken: the
    rotate-half convention, pairing element i with element i + d/2, with
    these frequencies, 0-based positions and no scaling.
    """
    i = np.arange(d // 2, dtype=np.float64)
    return theta ** (-2.0 * i / d)


def rope_rotate(x, pos, theta: float) -> np.ndarray:
    """Apply R_pos to the last axis of x (float64, no rounding).

    x: [..., d];  pos: integer array broadcastable to x.shape[:-1] (may be
    negative: R_{-a} is the inverse rotation).  For each pair
    (x_i, x_{i+d/2}) with angle a = pos * omega_i:
        x_i'       = x_i cos a - x_{i+d/2} sin a
        x_{i+d/2}' = x_i sin a + x_{i+d/2} cos a
    Angles are formed in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    pos = np.asarray(pos, dtype=np.float64)
    ang = pos[..., None] * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def realign_segment(k_cached, v_cached, p_src: int, p_dst: int, theta: float, dtype: str):
    """Delta-RoPE re-alignment of one reused segment (§3.1 eq. d; §4.4, §4.5).

    k_cached[j] holds R_{p_src+j} k_j (already rotated at its original
    position); the segment moves to start at p_dst.  Returns
        K'[j] = R_{p_dst - p_src} k_cached[j]   rounded to storage,
        V'[j] = v_cached[j]                      copied unchanged.
    Copy semantics (§4.4): the inputs are not modified.
    """
    k_cached = np.asarray(k_cached, dtype=np.float64)
    delta = np.full(k_cached.shape[:-1], p_dst - p_src)
    k_new = round_store(rope_rotate(k_cached, delta, theta), dtype)
    v_new = np.array(v_cached, dtype=np.float64, copy=True)
    return k_new, v_new


# ---------------------------------------------------------------------------
# Layout -- §3.2 (index sets; the fallback paragraph)
# ---------------------------------------------------------------------------

FALLBACK_TOKENS = 64


def plan_request(pieces, ratio, fallback_tokens: int = FALLBACK_TOKENS,
                 overflow_tokens: int = 0) -> dict:
    """Token classes and the selection budget of one request (§3.2, §3.3).

    pieces: ordered list of ("reuse", L) or ("new", L) runs; positions are
    0-based token indices in the request (T = sum of L).  Empty runs are
    ignored.  ratio: (num, den), the selection ratio as an exact fraction.

    I_reuse is the set of tokens of reused runs, I_nr its complement (§3.2,
    first display).  Fallback (§3.2, last paragraph), reading taken: it
    triggers iff the request's last token is reused; then the last
    min(fallback_tokens, L) tokens of the final reused run join I_nr (they
    get queries, fresh K/V and take part in scoring).  The selection
    candidates are the remaining reused tokens, R = |candidates|, and the
    budget is k = floor(num * R / den) in exact integer arithmetic (the
    ratio is read as a fraction of the reused tokens, so that ratio 100%
    recomputes every token).

    Overflow (§3.3, second paragraph), off when overflow_tokens is 0.
    Reading taken: a block is overflow_tokens tokens (the 16-token KV page
    of a block-aligned layout); for every maximal run of non-reused pieces,
    the last min(overflow_tokens, L) tokens of the reused piece right before
    it and the first min(overflow_tokens, L) tokens of the reused piece right
    after it join the Sparse-Q set, as the fallback tokens do: the paragraph
    widens the Sparse-Q index interval itself, so the widened rows get
    queries, fresh K/V, probe and attend.  They are thereby no selection
    candidates and the budget k counts only the remaining reused tokens.

    Returns dict(T, is_reuse[bool T], sq[int, ascending], cand[int,
    ascending], k, fallback[bool], overflow[int, ascending]: the tokens the
    overflow step marked, whether or not the fallback also took them).
    """
    pieces = [(kind, int(n)) for kind, n in pieces if int(n) > 0]
    for kind, _ in pieces:
        if kind not in ("reuse", "new"):
            raise ValueError(f"unknown piece kind {kind!r}")
    T = sum(n for _, n in pieces)
    is_reuse = np.zeros(T, dtype=bool)
    in_sq = np.zeros(T, dtype=bool)
    start = 0
    for kind, n in pieces:
        if kind == "reuse":
            is_reuse[start:start + n] = True
        else:
            in_sq[start:start + n] = True
        start += n
    fallback = False
    if pieces and pieces[-1][0] == "reuse":
        n_last = pieces[-1][1]
        m = min(fallback_tokens, n_last)
        in_sq[T - m:T] = True
        fallback = True
    if overflow_tokens < 0:
        raise ValueError("overflow_tokens must be >= 0")
    widened = np.zeros(T, dtype=bool)
    if overflow_tokens > 0:
        starts = np.cumsum([0] + [n for _, n in pieces])
        for p, (kind, n) in enumerate(pieces):
            if kind != "new":
                continue
            if p > 0 and pieces[p - 1][0] == "reuse":          # previous reuse segment
                m = min(overflow_tokens, pieces[p - 1][1])
                widened[starts[p] - m:starts[p]] = True
            if p + 1 < len(pieces) and pieces[p + 1][0] == "reuse":   # next reuse segment
                m = min(overflow_tokens, pieces[p + 1][1])
                widened[starts[p + 1]:starts[p + 1] + m] = True
        in_sq |= widened
    sq = np.flatnonzero(in_sq)
    cand = np.flatnonzero(is_reuse & ~in_sq)
    num, den = int(ratio[0]), int(ratio[1])
    if den <= 0 or num < 0 or num > den:
        raise ValueError("ratio must be a fraction in [0, 1]")
    k = (num * len(cand)) // den
    return dict(T=T, is_reuse=is_reuse, sq=sq, cand=cand, k=int(k), fallback=fallback,
                overflow=np.flatnonzero(widened))


# ---------------------------------------------------------------------------
# Projection -- §3.4 "Sparse-KV Recomputation" of the selected rows
# ---------------------------------------------------------------------------

def project_rows(x_rows, wq, wk, wv, pos, theta: float, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, dtype: str, want_q: bool = True):
    """Q/K/V of a set of rows at their positions (§3.1 eq. b; §3.4).

    x_rows [n, hidden] (storage values), wq [Hq*d, hidden], wk/wv
    [Hkv*d, hidden]; pos [n].  Reading taken: plain projections without bias
    (q = W_q x), RoPE at the row's position on q and k, none on v; each
    result rounded once to storage.  Returns q [n, Hq, d] (or None),
    k [n, Hkv, d], v [n, Hkv, d].
    """
    x = np.asarray(x_rows, dtype=np.float64)
    n = x.shape[0]
    pos = np.asarray(pos)
    k = (x @ np.asarray(wk, dtype=np.float64).T).reshape(n, n_kv_heads, head_dim)
    v = (x @ np.asarray(wv, dtype=np.float64).T).reshape(n, n_kv_heads, head_dim)
    k = round_store(rope_rotate(k, pos[:, None], theta), dtype)
    v = round_store(v, dtype)
    q = None
    if want_q:
        q = (x @ np.asarray(wq, dtype=np.float64).T).reshape(n, n_q_heads, head_dim)
        q = round_store(rope_rotate(q, pos[:, None], theta), dtype)
    return q, k, v


# ---------------------------------------------------------------------------
# Attention -- §3.2 (Sparse-Q rows attend to all available keys, causally)
# ---------------------------------------------------------------------------

def causal_attention(q, q_pos, K, V):
    """Causal GQA softmax attention of some query rows over a key range.

    q [n, Hq, d] at positions q_pos [n]; K, V [T, Hkv, d] indexed by
    position.  Query head h reads kv head h // (Hq/Hkv).  For every row i
    and head h:  l_j = q.k_j / sqrt(d) for 0 <= j <= q_pos[i],
    O = sum_j softmax(l)_j v_j,  LSE = log sum_j exp(l_j).
    No soft-cap, bias or window.  Returns O [n, Hq, d] and LSE [n, Hq] in
    float64, unrounded.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, hq, d = q.shape
    hkv = K.shape[1]
    g_sz = hq // hkv
    scale = 1.0 / math.sqrt(d)
    out = np.empty((n, hq, d))
    lse = np.empty((n, hq))
    for i in range(n):
        p = int(q_pos[i])
        for g in range(hkv):
            hs = slice(g * g_sz, (g + 1) * g_sz)
            logits = (q[i, hs] @ K[:p + 1, g].T) * scale          # [G, p+1]
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            z = e.sum(axis=1, keepdims=True)
            out[i, hs] = (e @ V[:p + 1, g]) / z
            lse[i, hs] = (m + np.log(z))[:, 0]
    return out, lse


def attention_mass_scores(q_sq, sq_pos, K, lse):
    """Sparse-Q attention mass received by every key (§3.2, display c; text
    after it: one global score aggregated across heads).

    s_j = sum_h sum_{i in Sparse-Q, pos_i >= j} exp(q_i^h . k_j / sqrt(d)
          - LSE_i^h)
    i.e. the causal softmax probability that Sparse-Q row i, head h, puts on
    key j, summed over all Sparse-Q rows and all query heads.  Readings
    taken: the softmax is the full causal one (normalised over every key
    j <= pos_i, reused or new); the aggregate is a plain sum.
    q_sq [n_sq, Hq, d]; K [T, Hkv, d]; lse [n_sq, Hq].  Returns s [T]
    (defined for every key; only reused keys are candidates).
    """
    q_sq = np.asarray(q_sq, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    n_sq, hq, d = q_sq.shape
    T, hkv, _ = K.shape
    g_sz = hq // hkv
    scale = 1.0 / math.sqrt(d)
    s = np.zeros(T)
    for i in range(n_sq):
        p = int(sq_pos[i])
        for g in range(hkv):
            hs = slice(g * g_sz, (g + 1) * g_sz)
            logits = (q_sq[i, hs] @ K[:p + 1, g].T) * scale      # [G, p+1]
            s[:p + 1] += np.exp(logits - lse[i, hs][:, None]).sum(axis=0)
    return s


def select_topk(scores, cand, k: int) -> np.ndarray:
    """Top-k of the candidates by score, per request (§3.3 first sentence;
    §3.4 "the selected top-k tokens").

    Order: score descending, then index ascending (the paper does not say
    how ties break; lower index wins).  -0.0 and +0.0 compare equal.
    Returns the k chosen indices in ascending order.
    """
    cand = np.asarray(cand, dtype=np.int64)
    if not 0 <= k <= len(cand):
        raise ValueError("k out of range")
    s = np.asarray(scores, dtype=np.float64)[cand]
    order = np.lexsort((cand, -s))        # primary: -score; secondary: index
    return np.sort(cand[order[:k]])


# ---------------------------------------------------------------------------
# One layer -- §3.2 (Sparse-Q), §3.4 (threshold, recomputation)
# ---------------------------------------------------------------------------

def _positions(T: int, pos0: int) -> np.ndarray:
    return np.arange(T, dtype=np.int64) + pos0


def sparse_layer(x, wq, wk, wv, plan: dict, segments, theta: float, n_q_heads: int,
                 n_kv_heads: int, head_dim: int, dtype: str, selected=None, lse_probe=None,
                 q_probe=None, k_probe=None, pos0: int = 0, out_rows=None) -> dict:
    """One SparseX prefill layer of one request.

    x [T, hidden]: layer input (storage values).  plan: from plan_request.
    segments: one tuple (dst_start, p_src, k_cached [L,Hkv,d],
    v_cached [L,Hkv,d]) per reused run, in order; k_cached is rotated at
    p_src + j.  pos0 shifts every RoPE position of the request.

    Steps, in the paper's order:
      1. realign every reused run into the request's cache (§3.1 eq. d);
      2. recompute q, k, v of the Sparse-Q rows I_nr (§3.2) and write k, v;
      3. if `selected` is None (selection inside this layer -- the threshold
         is layer 0, §3.4 last paragraph): Sparse-Q probe.  LSE of the
         Sparse-Q rows over the mixed cache, the attention mass scores, and
         the top-k of the candidates (select_topk).  Otherwise `selected` is
         the set S chosen at the boundary layer and is used as given;
      4. recompute the selected rows S and overwrite their k, v (§3.4);
      5. attention of the active rows A = I_nr U S (ascending) over the
         mixed cache (§3.2; §4.5 last paragraph).
    Readings taken: non-selected reused tokens get no query and no output;
    the k/v of S replace the realigned ones; the probe of step 3 uses the
    mixed cache of this layer.

    out_rows (for checks at full size): None computes O for every row of A;
    an int n computes it only for n rows of A spread evenly over it (first
    and last included); an array gives the rows (a subset of A).  O,
    O_exact and lse_A then hold those rows, listed in "O_rows".

    Returns dict with O [|A|, Hq*d] (rounded), O_exact (unrounded), A, S,
    scores (None if not probed), lse_sq, K, V (final mixed cache), q_A,
    O_rows.
    """
    T = plan["T"]
    pos = _positions(T, pos0)
    K = np.full((T, n_kv_heads, head_dim), np.nan)
    V = np.full((T, n_kv_heads, head_dim), np.nan)
    x = np.asarray(x, dtype=np.float64)
    # 1. realign
    for dst_start, p_src, k_c, v_c in segments:
        L = k_c.shape[0]
        kn, vn = realign_segment(k_c, v_c, p_src, pos0 + dst_start, theta, dtype)
        K[dst_start:dst_start + L] = kn
        V[dst_start:dst_start + L] = vn
    # 2. Sparse-Q rows
    sq = plan["sq"]
    q_sq, k_sq, v_sq = project_rows(x[sq], wq, wk, wv, pos[sq], theta, n_q_heads,
                                    n_kv_heads, head_dim, dtype)
    K[sq] = k_sq
    V[sq] = v_sq
    # 3. probe + select
    scores = None
    lse_sq = None
    if selected is None:
        _, lse_sq = causal_attention(q_sq, sq, K, V)
        scores = attention_mass_scores(q_sq, sq, K, lse_sq)
        S = select_topk(scores, plan["cand"], plan["k"])
    else:
        S = np.asarray(selected, dtype=np.int64)
    # 4. recompute S
    q_S, k_S, v_S = project_rows(x[S], wq, wk, wv, pos[S], theta, n_q_heads, n_kv_heads,
                                 head_dim, dtype)
    K[S] = k_S
    V[S] = v_S
    # 5. attention for A
    A = np.union1d(sq, S)
    q_A = np.empty((len(A), n_q_heads, head_dim))
    q_A[np.searchsorted(A, sq)] = q_sq
    q_A[np.searchsorted(A, S)] = q_S
    if out_rows is None:
        rows = A
    elif np.isscalar(out_rows):
        rows = A[np.unique(np.linspace(0, len(A) - 1, int(out_rows)).round().astype(np.int64))]
    else:
        rows = np.asarray(out_rows, dtype=np.int64)
        if not np.isin(rows, A).all():
            raise ValueError("out_rows must be active rows")
    O, lse_A = causal_attention(q_A[np.searchsorted(A, rows)], rows, K, V)
    O = O.reshape(len(rows), n_q_heads * head_dim)
    return dict(O=round_store(O, dtype), O_exact=O, A=A, S=S, scores=scores, lse_sq=lse_sq,
                lse_A=lse_A, K=K, V=V, q_A=q_A, q_sq=q_sq, O_rows=rows)


def full_layer(x, wq, wk, wv, theta: float, n_q_heads: int, n_kv_heads: int, head_dim: int,
               dtype: str, pos0: int = 0) -> dict:
    """Full causal prefill layer: every row recomputed and attending (the
    "full attention" layers before the threshold, §3.4; also the "full
    recompute" baseline of §5).  Returns O (rounded), O_exact, lse, K, V, q.
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    pos = _positions(T, pos0)
    q, k, v = project_rows(x, wq, wk, wv, pos, theta, n_q_heads, n_kv_heads, head_dim, dtype)
    O, lse = causal_attention(q, np.arange(T), k, v)
    O = O.reshape(T, n_q_heads * head_dim)
    return dict(O=round_store(O, dtype), O_exact=O, lse=lse, K=k, V=v, q=q)
