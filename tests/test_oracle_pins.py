"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks an oracle function against a closed form, an identity the
paper states, a library routine or a brute-force computation written here
in a different form, chosen so that a dropped term, a wrong sign or index,
or a transposed operand fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sparsex as ox

RNG = np.random.default_rng(7)


# ---------------------------------------------------------------- bf16 ------

def test_round_bf16_matches_torch_cast_on_float32_values():
    """For float32 inputs, round_bf16 must equal torch's RNE float32->bf16."""
    vals = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32),
        (RNG.standard_normal(2000) * 1e30).astype(np.float32),
        (RNG.standard_normal(2000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1.17549435e-38, 1e-40, -1e-40],
                 dtype=np.float32),
    ])
    # values exactly half-way between two bf16 numbers: ties must go to even
    base = torch.randn(4000).to(torch.bfloat16).to(torch.float32).numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([vals, ties])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(vals.astype(np.float64))
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_round_bf16_direct_from_float64_no_double_rounding():
    """1 + 2^-8 + 2^-40 is just above the midpoint between 1 and 1+2^-7: it
    must round up, although a float32 detour would round it to the midpoint
    first and then to even (down)."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # tie -> even
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6  # tie -> even
    assert np.isinf(oracle.round_bf16(np.array([3.4e38 * 1.01]))[0])


def test_round_store_f32_is_numpy_cast():
    x = RNG.standard_normal(1000)
    assert np.array_equal(oracle.round_store(x, "f32"), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- RoPE ------

def _complex_rope(x, pos, theta):
    """Independent form: pair (x_i, x_{i+d/2}) as z = x_i + i x_{i+d/2},
    rotated by e^{i pos omega_i}."""
    d = x.shape[-1]
    h = d // 2
    om = np.array([theta ** (-(2.0 * i) / d) for i in range(h)])
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.asarray(pos, float)[..., None] * om)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_frequencies_closed_form():
    om = oracle.rope_inv_freq(128, 5e5)
    assert om[0] == 1.0
    assert math.isclose(om[1], 5e5 ** (-2 / 128), rel_tol=1e-15)
    assert math.isclose(om[63], 5e5 ** (-126 / 128), rel_tol=1e-15)


def test_rope_matches_complex_rotation():
    x = RNG.standard_normal((50, 3, 64))
    pos = RNG.integers(-5000, 140000, size=(50, 3))
    got = oracle.rope_rotate(x, pos, 1e6)
    ref = _complex_rope(x, pos, 1e6)
    assert np.max(np.abs(got - ref)) < 1e-11


def test_rope_first_pair_explicit_matrix():
    """d = 2: one pair with omega = 1, R_m = [[cos m, -sin m], [sin m, cos m]]."""
    x = np.array([0.3, -1.7])
    for m in (0, 1, 7, -3, 12345):
        R = np.array([[math.cos(m), -math.sin(m)], [math.sin(m), math.cos(m)]])
        assert np.allclose(oracle.rope_rotate(x, m, 10000.0), R @ x, atol=1e-12)


def test_rope_delta_equals_direct_rotation():
    """Pin P1 (§3.1 eq. c/d): R_{p'-p} (R_p k) = R_{p'} k."""
    k = RNG.standard_normal((200, 8, 128))
    p = RNG.integers(0, 130000, size=(200, 1))
    pn = RNG.integers(0, 130000, size=(200, 1))
    via_delta = oracle.rope_rotate(oracle.rope_rotate(k, p, 5e5), pn - p, 5e5)
    direct = oracle.rope_rotate(k, pn, 5e5)
    rel = np.max(np.abs(via_delta - direct)) / np.max(np.abs(direct))
    assert rel < 1e-10   # angles up to 1.3e5 rad carry ~1e-11 absolute error in float64


def test_rope_zero_delta_is_exact_copy_and_group_laws():
    """Pins P2/P3: R_0 = I exactly; R_a R_b = R_{a+b}; R_{-a} R_a = I;
    pair norms preserved."""
    k = RNG.standard_normal((64, 2, 64))
    assert np.array_equal(oracle.rope_rotate(k, 0, 1e4), k)
    a, b = 977, -4321
    ab = oracle.rope_rotate(oracle.rope_rotate(k, b, 1e4), a, 1e4)
    assert np.allclose(ab, oracle.rope_rotate(k, a + b, 1e4), atol=1e-11)
    back = oracle.rope_rotate(oracle.rope_rotate(k, a, 1e4), -a, 1e4)
    assert np.allclose(back, k, atol=1e-12)
    r = oracle.rope_rotate(k, 31337, 1e4)
    h = 32
    assert np.allclose(r[..., :h] ** 2 + r[..., h:] ** 2, k[..., :h] ** 2 + k[..., h:] ** 2)


def test_rope_relative_identity():
    """§3.1 eq. c: <R_m q, R_n k> = q^T R_{n-m} k."""
    q = RNG.standard_normal(128)
    k = RNG.standard_normal(128)
    for m, n in [(0, 5), (100, 3), (70000, 70123), (5, 5)]:
        lhs = oracle.rope_rotate(q, m, 5e5) @ oracle.rope_rotate(k, n, 5e5)
        rhs = q @ oracle.rope_rotate(k, n - m, 5e5)
        assert math.isclose(lhs, rhs, rel_tol=1e-9, abs_tol=1e-9)


def test_realign_segment_copy_semantics_and_values():
    kc = oracle.round_bf16(RNG.standard_normal((40, 2, 64)))
    vc = oracle.round_bf16(RNG.standard_normal((40, 2, 64)))
    kc0, vc0 = kc.copy(), vc.copy()
    kn, vn = oracle.realign_segment(kc, vc, 300, 16, 1e4, "bf16")
    assert np.array_equal(kc, kc0) and np.array_equal(vc, vc0)   # sources untouched
    assert np.array_equal(vn, vc)                                 # V copied
    assert np.array_equal(kn, oracle.round_bf16(_complex_rope(kc, np.full((40, 2), -284), 1e4)))
    same, _ = oracle.realign_segment(kc, vc, 77, 77, 1e4, "bf16")
    assert np.array_equal(same, kc)                               # delta 0: bit-exact


# -------------------------------------------------------------- layout ------

def test_plan_request_hand_cases():
    p = oracle.plan_request([("reuse", 64), ("reuse", 64), ("new", 16)], (25, 100))
    assert p["T"] == 144 and not p["fallback"]
    assert np.array_equal(p["sq"], np.arange(128, 144))
    assert np.array_equal(p["cand"], np.arange(128))
    assert p["k"] == 32
    # tail is reused: last 64 tokens of the final segment join the Sparse-Q set
    p = oracle.plan_request([("new", 10), ("reuse", 100)], (1, 2))
    assert p["fallback"]
    assert np.array_equal(p["sq"], np.concatenate([np.arange(10), np.arange(46, 110)]))
    assert np.array_equal(p["cand"], np.arange(10, 46))
    assert p["k"] == 18
    # short final segment: all of it moves
    p = oracle.plan_request([("reuse", 50), ("reuse", 20)], (100, 100))
    assert np.array_equal(p["sq"], np.arange(50, 70))
    assert p["k"] == 50 and len(p["cand"]) == 50
    # exact decimal flooring: 15% of 4096 = 614.4 -> 614
    p = oracle.plan_request([("reuse", 4096), ("new", 256)], (15, 100))
    assert p["k"] == 614
    # empty pieces are ignored; a trailing empty "new" does not hide a reused tail
    p = oracle.plan_request([("reuse", 32), ("new", 0)], (0, 1))
    assert p["fallback"] and len(p["cand"]) == 0 and p["k"] == 0


def test_plan_request_brute_force_random():
    rng = np.random.default_rng(3)
    for _ in range(200):
        pieces = [(("reuse", "new")[rng.integers(2)], int(rng.integers(0, 90)))
                  for _ in range(rng.integers(1, 7))]
        num = int(rng.integers(0, 101))
        p = oracle.plan_request(pieces, (num, 100))
        # brute force, token by token
        toks = []
        for kind, n in pieces:
            toks += [kind] * n
        T = len(toks)
        last_reuse_run = []
        if T and toks[-1] == "reuse":
            j = T - 1
            while j >= 0 and toks[j] == "reuse":
                j -= 1
            # the final reused *piece* (not run): walk pieces backwards
            kept = [pc for pc in pieces if pc[1] > 0]
            n_last = kept[-1][1]
            last_reuse_run = list(range(T - min(64, n_last), T))
        sq = sorted(set(i for i in range(T) if toks[i] == "new") | set(last_reuse_run))
        cand = [i for i in range(T) if toks[i] == "reuse" and i not in set(last_reuse_run)]
        assert p["T"] == T
        assert list(p["sq"]) == sq
        assert list(p["cand"]) == cand
        assert p["k"] == (num * len(cand)) // 100


def test_plan_request_overflow_hand_cases():
    """§3.3 second paragraph: one block of the reused neighbours on each side
    of every non-reused interval joins the Sparse-Q set."""
    pieces = [("reuse", 100), ("new", 20), ("reuse", 50), ("new", 10)]
    p = oracle.plan_request(pieces, (1, 2), overflow_tokens=16)
    assert not p["fallback"]
    assert np.array_equal(p["overflow"], np.r_[84:100, 120:136, 154:170])
    assert np.array_equal(p["sq"], np.r_[84:136, 154:180])
    assert np.array_equal(p["cand"], np.r_[0:84, 136:154])
    assert p["k"] == 51
    # off by default: the same request without overflow
    q = oracle.plan_request(pieces, (1, 2))
    assert len(q["overflow"]) == 0 and np.array_equal(q["sq"], np.r_[100:120, 170:180])
    # a reused piece shorter than two blocks between two new runs is taken whole
    p = oracle.plan_request([("new", 5), ("reuse", 20), ("new", 5)], (1, 1), overflow_tokens=16)
    assert np.array_equal(p["overflow"], np.r_[5:25]) and len(p["cand"]) == 0 and p["k"] == 0
    # shorter than one block
    p = oracle.plan_request([("reuse", 7), ("new", 3)], (1, 1), overflow_tokens=16)
    assert np.array_equal(p["sq"], np.r_[0:10]) and p["k"] == 0
    # overflow and the tail fallback overlap-free here; both join the Sparse-Q set
    p = oracle.plan_request([("new", 10), ("reuse", 100)], (1, 2), overflow_tokens=16)
    assert p["fallback"]
    assert np.array_equal(p["overflow"], np.r_[10:26])
    assert np.array_equal(p["sq"], np.r_[0:26, 46:110])
    assert np.array_equal(p["cand"], np.r_[26:46]) and p["k"] == 10
    # adjacent reused pieces: only the piece touching the new run gives a block
    p = oracle.plan_request([("reuse", 40), ("reuse", 8), ("new", 4), ("reuse", 30)], (0, 1),
                            overflow_tokens=16)
    assert np.array_equal(p["overflow"], np.r_[40:48, 52:68])
    # adjacent new pieces form one interval: no block between them
    p = oracle.plan_request([("reuse", 40), ("new", 4), ("new", 6), ("reuse", 40), ("new", 1)],
                            (0, 1), overflow_tokens=16)
    assert np.array_equal(p["overflow"], np.r_[24:40, 50:66, 74:90])
    with pytest.raises(ValueError):
        oracle.plan_request(pieces, (1, 2), overflow_tokens=-1)


def test_plan_request_overflow_brute_force_random():
    """Dual formulation, token by token: a reused token is widened iff its
    own piece borders a new piece on that side within one block."""
    rng = np.random.default_rng(11)
    for _ in range(300):
        pieces = [(("reuse", "new")[rng.integers(2)], int(rng.integers(0, 60)))
                  for _ in range(rng.integers(1, 8))]
        B = int(rng.integers(1, 33))
        num = int(rng.integers(0, 101))
        p = oracle.plan_request(pieces, (num, 100), overflow_tokens=B)
        kept = [pc for pc in pieces if pc[1] > 0]
        toks, widened = [], set()
        for i, (kind, n) in enumerate(kept):
            t0 = len(toks)
            toks += [kind] * n
            if kind != "reuse":
                continue
            if i + 1 < len(kept) and kept[i + 1][0] == "new":
                widened |= set(range(t0 + n - min(B, n), t0 + n))
            if i > 0 and kept[i - 1][0] == "new":
                widened |= set(range(t0, t0 + min(B, n)))
        T = len(toks)
        tail = set()
        if kept and kept[-1][0] == "reuse":
            tail = set(range(T - min(64, kept[-1][1]), T))
        sq = sorted(set(i for i in range(T) if toks[i] == "new") | tail | widened)
        cand = [i for i in range(T) if toks[i] == "reuse" and i not in tail | widened]
        assert list(p["overflow"]) == sorted(widened)
        assert list(p["sq"]) == sq
        assert list(p["cand"]) == cand
        assert p["k"] == (num * len(cand)) // 100


# ------------------------------------------------------------ attention -----

def _attn_triple_loop(q, q_pos, K, V):
    """Pure-Python loops, written independently of the oracle."""
    n, hq, d = q.shape
    G = hq // K.shape[1]
    out = np.zeros((n, hq, d))
    lse = np.zeros((n, hq))
    for i in range(n):
        for h in range(hq):
            g = h // G
            ls = []
            for j in range(int(q_pos[i]) + 1):
                ls.append(sum(q[i, h, t] * K[j, g, t] for t in range(d)) / math.sqrt(d))
            mx = max(ls)
            w = [math.exp(v - mx) for v in ls]
            z = sum(w)
            lse[i, h] = mx + math.log(z)
            for t in range(d):
                out[i, h, t] = sum(w[j] * V[j, g, t] for j in range(len(w))) / z
    return out, lse


def test_causal_attention_vs_triple_loop():
    T, hq, hkv, d = 20, 4, 2, 8
    K = RNG.standard_normal((T, hkv, d))
    V = RNG.standard_normal((T, hkv, d))
    rows = np.array([0, 3, 4, 11, 19])
    q = RNG.standard_normal((len(rows), hq, d)) * 2
    o, l = oracle.causal_attention(q, rows, K, V)
    o2, l2 = _attn_triple_loop(q, rows, K, V)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(l, l2, atol=1e-12)


def test_causal_attention_closed_forms():
    """Pins P8/P9: q = 0 gives the mean of v_0..v_i; constant V gives that
    constant; the first token attends only to itself."""
    T, hq, hkv, d = 33, 6, 3, 16
    K = RNG.standard_normal((T, hkv, d))
    V = RNG.standard_normal((T, hkv, d))
    rows = np.arange(T)
    o, lse = oracle.causal_attention(np.zeros((T, hq, d)), rows, K, V)
    for i in (0, 5, 32):
        for h in range(hq):
            assert np.allclose(o[i, h], V[:i + 1, h // 2].mean(axis=0), atol=1e-13)
            assert math.isclose(lse[i, h], math.log(i + 1), abs_tol=1e-13)
    Vc = np.full((T, hkv, d), 0.625)
    q = RNG.standard_normal((T, hq, d))
    o, _ = oracle.causal_attention(q, rows, K, Vc)
    assert np.allclose(o, 0.625, atol=1e-14)
    assert np.allclose(o[0], np.repeat(Vc[0], 2, axis=0))


def test_attention_uses_gqa_group_of_query_head():
    """Query head h must read kv head h // G (contiguous groups): perturbing
    kv head 1 may only change query heads G..2G-1."""
    T, hq, hkv, d = 10, 4, 2, 4
    K = RNG.standard_normal((T, hkv, d))
    V = RNG.standard_normal((T, hkv, d))
    q = RNG.standard_normal((T, hq, d))
    o1, _ = oracle.causal_attention(q, np.arange(T), K, V)
    V2 = V.copy()
    V2[:, 1] += 1.0
    o2, _ = oracle.causal_attention(q, np.arange(T), K, V2)
    assert np.allclose(o1[:, :2], o2[:, :2]) and np.allclose(o2[:, 2:], o1[:, 2:] + 1.0)


def _scores_brute(q_sq, sq_pos, K, lse):
    n, hq, d = q_sq.shape
    T = K.shape[0]
    G = hq // K.shape[1]
    s = [0.0] * T
    for j in range(T):
        for i in range(n):
            if sq_pos[i] < j:
                continue
            for h in range(hq):
                lg = sum(q_sq[i, h, t] * K[j, h // G, t] for t in range(d)) / math.sqrt(d)
                s[j] += math.exp(lg - lse[i, h])
    return np.array(s)


def test_attention_mass_scores_brute_force_and_mass_conservation():
    T, hq, hkv, d = 24, 4, 2, 8
    K = RNG.standard_normal((T, hkv, d))
    V = RNG.standard_normal((T, hkv, d))
    sq = np.array([5, 6, 17, 23])
    q = RNG.standard_normal((len(sq), hq, d)) * 1.5
    _, lse = oracle.causal_attention(q, sq, K, V)
    s = oracle.attention_mass_scores(q, sq, K, lse)
    assert np.allclose(s, _scores_brute(q, sq, K, lse), atol=1e-12)
    # every softmax row sums to one: total mass = (#Sparse-Q rows) x Hq
    assert math.isclose(s.sum(), len(sq) * hq, rel_tol=1e-12)
    assert np.all(s[24:] == 0) and np.all(s >= 0)


def test_attention_mass_scores_closed_form_zero_queries():
    """Pin P8: q = 0 => s_j = Hq * sum_{i in Sparse-Q, i >= j} 1/(i+1)."""
    T, hq, hkv, d = 40, 8, 2, 16
    K = RNG.standard_normal((T, hkv, d))
    sq = np.array([9, 10, 30, 39])
    q = np.zeros((len(sq), hq, d))
    _, lse = oracle.causal_attention(q, sq, K, K)
    s = oracle.attention_mass_scores(q, sq, K, lse)
    ref = np.array([hq * sum(1.0 / (i + 1) for i in sq if i >= j) for j in range(T)])
    assert np.allclose(s, ref, rtol=1e-13)


# --------------------------------------------------------------- top-k ------

def test_select_topk_vs_stable_sort():
    """Pin P10: first k of a stable sort by descending score (brute force),
    including adversarial ties and signed zeros."""
    rng = np.random.default_rng(11)
    cases = [rng.standard_normal(300), np.ones(300), np.where(rng.random(300) < 0.5, 2.0, 1.0),
             np.where(rng.random(300) < 0.5, 0.0, -0.0), np.round(rng.random(300) * 4) / 4]
    for s in cases:
        cand = np.sort(rng.choice(300, size=200, replace=False))
        for k in (0, 1, 7, 100, 200):
            got = oracle.select_topk(s, cand, k)
            items = sorted(cand.tolist(), key=lambda j: (-float(s[j]) + 0.0, j))  # -0.0 == 0.0
            assert list(got) == sorted(items[:k])


# -------------------------------------------------------- projection --------

def test_project_rows_against_loops():
    hidden, hq, hkv, d = 12, 2, 1, 4
    x = RNG.standard_normal((3, hidden))
    wq = RNG.standard_normal((hq * d, hidden))
    wk = RNG.standard_normal((hkv * d, hidden))
    wv = RNG.standard_normal((hkv * d, hidden))
    pos = np.array([0, 5, 900])
    q, k, v = oracle.project_rows(x, wq, wk, wv, pos, 1e4, hq, hkv, d, "f32")
    for r in range(3):
        qq = np.array([sum(x[r, c] * wq[o, c] for c in range(hidden)) for o in range(hq * d)])
        kk = np.array([sum(x[r, c] * wk[o, c] for c in range(hidden)) for o in range(hkv * d)])
        vv = np.array([sum(x[r, c] * wv[o, c] for c in range(hidden)) for o in range(hkv * d)])
        assert np.allclose(q[r], _complex_rope(qq.reshape(hq, d), np.full(hq, pos[r]), 1e4), atol=1e-6)
        assert np.allclose(k[r], _complex_rope(kk.reshape(hkv, d), np.full(hkv, pos[r]), 1e4), atol=1e-6)
        assert np.allclose(v[r], vv.reshape(hkv, d), atol=1e-6)
    assert np.array_equal(v, v.astype(np.float32).astype(np.float64))   # stored as fp32
