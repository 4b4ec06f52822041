"""Pins for the fp64 CPU oracle (no GPU).

Each oracle function is checked against something other than itself:
hand-derived values (tests/golden), an explicit-mask brute force, a closed
form, a library routine (torch SDPA in fp64, numpy matmul, math.exp) or an
invariant of the mathematics.  Planted mistakes in the oracle's arithmetic
(a dropped term, a wrong sign or index, a transposed operand) fail at least
one of these.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _lists(hkv, lists_v, lists_o):
    cap_v = max(1, max(len(x) for x in lists_v))
    cap_s = max(1, max(len(x) for x in lists_o))
    vidx = np.full((hkv, cap_v), -1, np.int32)
    soff = np.full((hkv, cap_s), -1, np.int32)
    for g in range(hkv):
        vidx[g, :len(lists_v[g])] = sorted(lists_v[g])
        soff[g, :len(lists_o[g])] = sorted(lists_o[g])
    vcnt = np.array([len(x) for x in lists_v], np.int32)
    scnt = np.array([len(x) for x in lists_o], np.int32)
    return vidx, vcnt, soff, scnt


def _rand_sets(rng, n, pv, ps, force_zero=None):
    cols = [int(c) for c in np.nonzero(rng.random(n) < pv)[0]]
    offs = [int(o) for o in np.nonzero(rng.random(n) < ps)[0]]
    if force_zero is False and 0 in offs:
        offs.remove(0)
    return cols, offs


# ----------------------------------------------------------------- golden, by hand

def test_hand_worked_attention():
    gold = json.load(open(os.path.join(GOLD, "hand_attention.json")))
    n, d = 4, 2
    w = np.array([1.0, 2.0, 3.0, 4.0])
    q = np.zeros((1, n, d))
    q[0, :, 0] = 1.0
    k = np.zeros((1, n, d))
    k[0, :, 0] = np.log(w)
    v = np.stack([np.arange(n, dtype=np.float64), np.ones(n)], axis=1)[None]
    for case in gold["cases"]:
        vidx, vcnt, soff, scnt = _lists(1, [case["columns"]], [case["offsets"]])
        for i in range(n):
            assert list(oracle.row_set(vidx, vcnt, soff, scnt, 0, i)) == case["sets"][i]
        out, lse = oracle.attn(q, k, v, vidx, vcnt, soff, scnt, scale=1.0)
        np.testing.assert_allclose(out[0], np.array(case["out"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(np.exp(lse[0]), np.array(case["lse_exp"]), rtol=1e-14, atol=0)


def test_hand_worked_selection():
    gold = json.load(open(os.path.join(GOLD, "hand_select.json")))
    for case in gold["cases"]:
        kind = oracle.VERTICAL if case["kind"] == "vertical" else oracle.SLASH
        logit = np.array([case["logit"]], np.float32)
        idx, cnt, U, T = oracle.select(logit, kind, case["mass"], case["cap"], return_ut=True)
        assert int(U[0]) == case["U"] and int(T[0]) == case["T"], case
        assert int(cnt[0]) == case["count"], case
        assert list(idx[0, :cnt[0]]) == case["idx"], case
        assert (idx[0, cnt[0]:] == -1).all()


# ----------------------------------------------------------------- the pattern

def test_row_sets_match_explicit_mask():
    rng = np.random.default_rng(7)
    for trial in range(60):
        n = int(rng.integers(1, 65))
        cols, offs = _rand_sets(rng, n, rng.random() * 0.4, rng.random() * 0.4,
                                force_zero=bool(trial % 2))
        vidx, vcnt, soff, scnt = _lists(1, [cols], [offs])
        mask = brute.explicit_mask(n, cols, offs)
        for i in range(n):
            got = oracle.row_set(vidx, vcnt, soff, scnt, 0, i)
            assert list(got) == list(np.nonzero(mask[i])[0]), (trial, i)


def test_pair_count_closed_form():
    """sum_i |S_i| = sum_{c in V}(n-c) + sum_{o in O}(n-o) - #{(c,o): c+o <= n-1}."""
    rng = np.random.default_rng(11)
    for n, pv, ps in [(1, 1.0, 1.0), (50, 0.3, 0.2), (700, 0.05, 0.1), (3000, 0.01, 0.06), (4096, 1.0, 0.0)]:
        cols, offs = _rand_sets(rng, n, pv, ps)
        vidx, vcnt, soff, scnt = _lists(1, [cols], [offs])
        c = np.array(cols, np.int64)
        o = np.array(offs, np.int64)
        both = int((c[:, None] + o[None, :] <= n - 1).sum()) if len(c) and len(o) else 0
        closed = int((n - c).sum() + (n - o).sum()) - both
        assert oracle.pair_count(vidx, vcnt, soff, scnt, 0, n) == closed


# ----------------------------------------------------------------- attention

@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_attention_matches_bruteforce(dtype):
    import workloads
    rng = np.random.default_rng(3)
    for trial in range(12):
        n = int(rng.integers(1, 65))
        d = int(rng.choice([1, 4, 16, 64]))
        hkv = int(rng.integers(1, 3))
        group = int(rng.integers(1, 4))
        hq = hkv * group
        q = rng.standard_normal((hq, n, d)) * 2
        k = rng.standard_normal((hkv, n, d)) * 2
        v = rng.standard_normal((hkv, n, d))
        if dtype == "f32":
            q, k, v = (x.astype(np.float32) for x in (q, k, v))
        elif dtype == "bf16":
            q, k, v = (workloads.to_bf16_bits(x) for x in (q, k, v))
        sets = [_rand_sets(rng, n, 0.25, 0.25, force_zero=bool(trial % 2)) for _ in range(hkv)]
        vidx, vcnt, soff, scnt = _lists(hkv, [s[0] for s in sets], [s[1] for s in sets])
        scale = 1.0 / math.sqrt(d)
        out, lse = oracle.attn(q, k, v, vidx, vcnt, soff, scnt, scale=scale)
        as64 = (lambda x: workloads.bf16_bits_to_f32(x).astype(np.float64)) if dtype == "bf16" \
            else (lambda x: x.astype(np.float64))
        Q, K, Vv = as64(q), as64(k), as64(v)
        for h in range(hq):
            g = h // group
            mask = brute.explicit_mask(n, *sets[g])
            bo, bl = brute.masked_attention(Q[h], K[g], Vv[g], mask, scale)
            np.testing.assert_allclose(out[h], bo, rtol=0, atol=1e-12)
            fin = np.isfinite(bl)
            assert (np.isfinite(lse[h]) == fin).all()
            np.testing.assert_allclose(lse[h][fin], bl[fin], rtol=0, atol=1e-12)


def _sdpa(q, k, v, group, mask=None, causal=False):
    Q = torch.from_numpy(q)
    K = torch.from_numpy(k).repeat_interleave(group, dim=0)
    V = torch.from_numpy(v).repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(
        Q[None], K[None], V[None], attn_mask=None if mask is None else torch.from_numpy(mask),
        is_causal=causal)[0].numpy()


@pytest.mark.parametrize("which", ["all_columns", "all_offsets", "both"])
def test_dense_equivalence_sdpa(which):
    """Every column (or every offset 0..n-1) selected equals dense causal attention."""
    rng = np.random.default_rng(5)
    hkv, group, n, d = 2, 3, 96, 32
    q = rng.standard_normal((hkv * group, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    allc = list(range(n))
    cols = allc if which in ("all_columns", "both") else [5, 17]
    offs = allc if which in ("all_offsets", "both") else [0, 3]
    vidx, vcnt, soff, scnt = _lists(hkv, [cols] * hkv, [offs] * hkv)
    out, lse = oracle.attn(q, k, v, vidx, vcnt, soff, scnt)
    ref = _sdpa(q, k, v, group, causal=True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # lse against the dense log-sum-exp
    s = np.einsum("hid,hjd->hij", q, np.repeat(k, group, 0)) / math.sqrt(d)
    s[:, np.triu(np.ones((n, n), bool), 1)] = -np.inf
    ref_lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_sliding_window_is_band_sdpa():
    """Offsets {0..w-1} alone give sliding-window attention."""
    rng = np.random.default_rng(9)
    n, d, w = 80, 16, 7
    q = rng.standard_normal((1, n, d))
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((1, n, d))
    vidx, vcnt, soff, scnt = _lists(1, [[]], [list(range(w))])
    out, _ = oracle.attn(q, k, v, vidx, vcnt, soff, scnt)
    i = np.arange(n)
    band = (i[None, :] <= i[:, None]) & (i[:, None] - i[None, :] < w)
    ref = _sdpa(q, k, v, 1, mask=band)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(13)
    n, d = 40, 8
    q = rng.standard_normal((1, n, d))
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((1, n, d))
    s_diag = (q[0] * k[0]).sum(-1) / math.sqrt(d)
    # O = {0}, V = {}: each row sees only itself
    out, lse = oracle.attn(q, k, v, *_lists(1, [[]], [[0]]))
    np.testing.assert_allclose(out[0], v[0], atol=1e-13)
    np.testing.assert_allclose(lse[0], s_diag, atol=1e-13)
    # V = {0}, O = {}: each row sees only column 0
    out, lse = oracle.attn(q, k, v, *_lists(1, [[0]], [[]]))
    np.testing.assert_allclose(out[0], np.broadcast_to(v[0, 0], (n, d)), atol=1e-13)
    np.testing.assert_allclose(lse[0], (q[0] @ k[0, 0]) / math.sqrt(d), atol=1e-13)
    # nothing visible for rows below the smallest column / offset: zero and -inf
    out, lse = oracle.attn(q, k, v, *_lists(1, [[10]], [[12]]))
    assert (out[0, :10] == 0).all() and np.isneginf(lse[0, :10]).all()
    assert np.isfinite(lse[0, 10:]).all()


def test_invariants_value_ones_and_zero_query():
    rng = np.random.default_rng(17)
    n, d = 128, 16
    cols, offs = _rand_sets(rng, n, 0.1, 0.1, force_zero=False)
    lists = _lists(1, [cols], [offs])
    mask = brute.explicit_mask(n, cols, offs)
    nonempty = mask.any(1)
    q = rng.standard_normal((1, n, d))
    k = rng.standard_normal((1, n, d))
    ones = np.ones((1, n, d))
    out, _ = oracle.attn(q, k, ones, *lists)
    np.testing.assert_allclose(out[0][nonempty], 1.0, atol=1e-13)
    # zero queries: uniform average over S_i and lse = log |S_i|
    v = rng.standard_normal((1, n, d))
    out, lse = oracle.attn(np.zeros_like(q), k, v, *lists)
    for i in np.nonzero(nonempty)[0]:
        js = np.nonzero(mask[i])[0]
        np.testing.assert_allclose(out[0, i], v[0, js].mean(0), atol=1e-13)
        assert abs(lse[0, i] - math.log(len(js))) < 1e-13


def test_probabilities_sum_to_one_via_identity_values():
    """With d = n and V = identity, out_i is the probability row P_i: it sums to
    1 and is supported exactly on S_i."""
    rng = np.random.default_rng(19)
    n = 48
    q = rng.standard_normal((1, n, n))
    k = rng.standard_normal((1, n, n))
    v = np.eye(n)[None]
    cols, offs = _rand_sets(rng, n, 0.15, 0.15, force_zero=False)
    out, _ = oracle.attn(q, k, v, *_lists(1, [cols], [offs]))
    mask = brute.explicit_mask(n, cols, offs)
    P = out[0]
    rows = mask.any(1)
    np.testing.assert_allclose(P[rows].sum(1), 1.0, atol=1e-13)
    assert ((P > 0) == mask).all()


def test_sampled_rows_equal_full():
    rng = np.random.default_rng(23)
    hkv, group, n, d = 2, 2, 200, 8
    q = rng.standard_normal((hkv * group, n, d)).astype(np.float32)
    k = rng.standard_normal((hkv, n, d)).astype(np.float32)
    v = rng.standard_normal((hkv, n, d)).astype(np.float32)
    sets = [_rand_sets(rng, n, 0.05, 0.05) for _ in range(hkv)]
    lists = _lists(hkv, [s[0] for s in sets], [s[1] for s in sets])
    out, lse = oracle.attn(q, k, v, *lists)
    rows = np.array([[3, 199], [0, 0], [1, 57], [2, 100]])
    o2, l2 = oracle.attn(q, k, v, *lists, rows=rows)
    np.testing.assert_array_equal(o2, out[rows[:, 0], rows[:, 1]])
    np.testing.assert_array_equal(l2, lse[rows[:, 0], rows[:, 1]])


# ----------------------------------------------------------------- the indexer

def test_indexer_matches_numpy_and_invariants():
    import workloads
    rng = np.random.default_rng(29)
    hkv, n, d, hidden = 3, 50, 16, 24
    k = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    v = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    w1, w2 = workloads.indexer_weights(rng, 2 * d, hidden)
    vl, sl = oracle.index(k, v, w1, w2)
    K = workloads.bf16_bits_to_f32(k).astype(np.float64)
    V = workloads.bf16_bits_to_f32(v).astype(np.float64)
    W1 = workloads.bf16_bits_to_f32(w1).astype(np.float64)
    W2 = workloads.bf16_bits_to_f32(w2).astype(np.float64)
    x = np.concatenate([K, V], axis=-1)
    h = np.maximum(x @ W1.T, 0.0)
    ref = h @ W2.T
    np.testing.assert_allclose(vl, ref[..., 0], atol=1e-12)
    np.testing.assert_allclose(sl, ref[..., 1], atol=1e-12)
    # zero input -> zero logits; doubling W2 doubles; positive scaling of x scales
    z = np.zeros_like(K)
    vz, sz = oracle.index(z, z, W1, W2)
    assert (vz == 0).all() and (sz == 0).all()
    v2, s2 = oracle.index(K, V, W1, 2 * W2)
    np.testing.assert_allclose(v2, 2 * vl, atol=1e-12)
    np.testing.assert_allclose(s2, 2 * sl, atol=1e-12)
    v3, s3 = oracle.index(3 * K, 3 * V, W1, W2)
    np.testing.assert_allclose(v3, 3 * vl, atol=1e-11)
    # K and V enter the first layer through different weight columns
    vs, _ = oracle.index(V, K, W1, W2)
    ref_sw = np.maximum(np.concatenate([V, K], -1) @ W1.T, 0) @ W2.T
    np.testing.assert_allclose(vs, ref_sw[..., 0], atol=1e-12)


# ----------------------------------------------------------------- selection

def test_exp_spec_against_math_exp():
    xs = np.concatenate([np.linspace(-32.0, 0.0, 200001, dtype=np.float32),
                         -np.abs(np.random.default_rng(1).standard_normal(20000).astype(np.float32)),
                         np.array([0.0, -0.0, -1e-30, -32.0, -math.log(2)], np.float32)])
    got = oracle.exp_spec(xs).astype(np.float64)
    ref = np.exp(xs.astype(np.float64))
    rel = np.abs(got - ref) / ref
    assert rel.max() < 2.0 ** -21, rel.max()
    assert oracle.exp_spec(np.float32(0.0)) == 1.0
    assert int(oracle.mass_u(np.float32(0.0))) == 2 ** 32
    assert int(oracle.mass_u(np.float32(-32.5))) == 0
    # quantised mass tracks exp(x) * 2^32 to within rounding plus the exp error
    u = oracle.mass_u(xs[:5000]).astype(np.float64)
    ref_u = np.exp(xs[:5000].astype(np.float64)) * 2.0 ** 32
    assert (np.abs(u - ref_u) <= 0.5 + ref_u * 2.0 ** -21).all()


def test_selection_is_minimal_by_exhaustive_search():
    rng = np.random.default_rng(31)
    for trial in range(80):
        n = int(rng.integers(1, 11))
        # few distinct values so that ties are common
        logit = rng.choice(np.array([0.0, -0.5, -1.0, -3.0, -40.0], np.float32), size=n)
        mass = float(rng.choice([1e-9, 0.3, 0.5, 0.77, 0.95, 1.0]))
        kind = int(rng.integers(0, 2))
        idx, cnt, U, T = oracle.select(logit[None], kind, mass, n, return_ut=True)
        score = logit if kind == oracle.VERTICAL else logit[::-1]
        u = oracle.mass_u(score - score.max())
        assert int(U[0]) == int(u.sum())
        assert int(T[0]) == math.ceil(mass * float(int(U[0])))
        K = int(cnt[0])
        assert K == brute.min_subset_size(u, int(T[0]))
        chosen = idx[0, :K]
        assert (np.diff(chosen) > 0).all()
        assert sum(int(u[c]) for c in chosen) >= int(T[0])
        # every unchosen candidate is ranked after every chosen one
        for c in set(range(n)) - set(chosen.tolist()):
            for s in chosen:
                assert (score[c] < score[s]) or (score[c] == score[s] and c > s)


def test_selection_caps_and_ties():
    n = 1000
    logit = np.zeros((1, n), np.float32)
    idx, cnt = oracle.select(logit, oracle.VERTICAL, 0.95, 100)
    assert cnt[0] == 100 and list(idx[0]) == list(range(100))
    idx, cnt = oracle.select(logit, oracle.SLASH, 0.5, n)
    assert cnt[0] == 500 and list(idx[0, :500]) == list(range(500))
    # a tiny mass selects exactly the arg-max (lowest index among equal maxima)
    rng = np.random.default_rng(37)
    lg = rng.standard_normal((4, n)).astype(np.float32)
    lg[2, [17, 400]] = 10.0
    idx, cnt = oracle.select(lg, oracle.VERTICAL, 1e-12, n)
    assert (cnt == 1).all()
    assert list(idx[:, 0]) == [int(np.argmax(lg[h])) for h in range(4)]
    assert idx[2, 0] == 17
    # -0.0 and +0.0 tie
    z = np.array([[-0.0, 0.0, -0.0]], np.float32)
    idx, cnt = oracle.select(z, oracle.VERTICAL, 0.5, 3)
    assert list(idx[0, :cnt[0]]) == [0, 1]


def test_selection_zipf_closed_form():
    """Logits -s ln(rank): softmax is the Zipf pmf, so the budget is the
    smallest K with H_{K,s} >= mass * H_{n,s}, and the chosen positions are
    those of ranks 1..K (then capped)."""
    import workloads
    rng = np.random.default_rng(41)
    n, s = 20000, 1.1
    lg = workloads.zipf_logits(rng, 2, n, s)
    ranks = np.rint(np.exp(-lg.astype(np.float64) / s)).astype(np.int64)
    w = np.arange(1, n + 1, dtype=np.float64) ** -s
    cum = np.cumsum(w)
    for mass in (0.5, 0.8, 0.95):
        K = int(np.searchsorted(cum, mass * cum[-1]) + 1)
        idx, cnt = oracle.select(lg, oracle.VERTICAL, mass, n)
        assert (cnt == K).all(), (mass, cnt, K)
        for h in range(2):
            assert set(idx[h, :K].tolist()) == set(np.nonzero(ranks[h] <= K)[0].tolist())
        cap = 64
        kc = min(K, cap)
        idx, cnt = oracle.select(lg, oracle.VERTICAL, mass, cap)
        assert (cnt == kc).all()
        for h in range(2):
            assert set(idx[h, :kc].tolist()) == set(np.nonzero(ranks[h] <= kc)[0].tolist())


def test_slash_reads_score_at_last_row():
    rng = np.random.default_rng(43)
    n = 300
    lg = rng.standard_normal((3, n)).astype(np.float32)
    iv, cv = oracle.select(lg[:, ::-1].copy(), oracle.VERTICAL, 0.6, n)
    is_, cs = oracle.select(lg, oracle.SLASH, 0.6, n)
    np.testing.assert_array_equal(cv, cs)
    np.testing.assert_array_equal(iv, is_)


# ------------------------------------------------- max-based threshold selection

def test_hand_worked_threshold_selection():
    gold = json.load(open(os.path.join(GOLD, "hand_select_threshold.json")))
    for case in gold["cases"]:
        kind = oracle.VERTICAL if case["kind"] == "vertical" else oracle.SLASH
        logit = np.array([case["logit"]], np.float32)
        idx, cnt, A = oracle.select_threshold(logit, kind, case["alpha"], case["cap"], return_a=True)
        assert A == case["A"], case
        assert int(cnt[0]) == case["count"], case
        assert list(idx[0, :cnt[0]]) == case["idx"], case
        assert (idx[0, cnt[0]:] == -1).all()


def test_threshold_zipf_closed_form():
    """Logits -s ln(rank): p_c / max p = rank^-s, so alpha keeps exactly the
    ranks r <= alpha^(-1/s); alpha sits halfway (in log) between two ranks."""
    import workloads
    rng = np.random.default_rng(51)
    n, s = 20000, 1.1
    lg = workloads.zipf_logits(rng, 2, n, s)
    ranks = np.rint(np.exp(-lg.astype(np.float64) / s)).astype(np.int64)
    for K in (1, 7, 37, 400):
        alpha = math.sqrt(K * (K + 1.0)) ** -s
        idx, cnt = oracle.select_threshold(lg, oracle.VERTICAL, alpha, n)
        assert (cnt == K).all(), (K, cnt)
        for h in range(2):
            assert set(idx[h, :K].tolist()) == set(np.nonzero(ranks[h] <= K)[0].tolist())
        kc = min(K, 5)
        idx, cnt = oracle.select_threshold(lg, oracle.VERTICAL, alpha, 5)
        assert (cnt == kc).all()
        for h in range(2):
            assert set(idx[h, :kc].tolist()) == set(np.nonzero(ranks[h] <= kc)[0].tolist())


def test_threshold_matches_real_arithmetic_bruteforce():
    """exp(s_c - max) >= alpha in float64, ordered by (score desc, index asc),
    capped; draws whose margin to the threshold is tiny are skipped."""
    rng = np.random.default_rng(53)
    checked = 0
    for trial in range(400):
        n = int(rng.integers(1, 30))
        lg = (rng.standard_normal(n) * 2).astype(np.float32)
        lg[rng.random(n) < 0.2] = lg[0]          # ties
        alpha = float(np.exp(rng.uniform(-6, 0)))
        cap = int(rng.integers(1, n + 1))
        kind = int(rng.integers(0, 2))
        score = lg if kind == 0 else lg[::-1]
        s = [0.0 if float(x) == 0.0 else float(x) for x in score]
        m = max(s)
        ratio = [math.exp(x - m) for x in s]
        if any(abs(r - alpha) <= 1e-5 * alpha for r in ratio):
            continue
        kept = sum(r >= alpha for r in ratio)
        order = sorted(range(n), key=lambda c: (-s[c], c))
        want = sorted(order[:min(kept, cap)])
        idx, cnt = oracle.select_threshold(lg[None, :], kind, alpha, cap)
        assert int(cnt[0]) == len(want) and list(idx[0, :cnt[0]]) == want, (lg, alpha, cap, kind)
        checked += 1
    assert checked > 300


def test_threshold_special_cases():
    lg = np.array([[3.0, -2.0, 3.0, 1.0, 3.0]], np.float32)
    idx, cnt = oracle.select_threshold(lg, oracle.VERTICAL, 1.0, 5)
    assert list(idx[0, :cnt[0]]) == [0, 2, 4]                  # the tied maxima only
    idx, cnt = oracle.select_threshold(lg, oracle.VERTICAL, 1e-12, 5)
    assert int(cnt[0]) == 5                                    # within ln(1e12) = 27.6 of the max
    far = np.array([[0.0, -40.0, -1.0]], np.float32)
    idx, cnt = oracle.select_threshold(far, oracle.VERTICAL, 1e-12, 3)
    assert list(idx[0, :cnt[0]]) == [0, 2]                      # 40 below the max: mass 0
    with pytest.raises(ValueError):
        oracle.select_threshold(lg, oracle.VERTICAL, 0.0, 5)
    with pytest.raises(ValueError):
        oracle.select_threshold(lg, oracle.VERTICAL, 1.5, 5)


# -------------------------------------------- vertical/slash ground-truth sums

def _explicit_aggregate(q, k, scale):
    """Whole P matrices in numpy (float64), then column and diagonal sums."""
    hq, n, _ = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    a_v = np.zeros((hkv, n))
    a_s = np.zeros((hkv, n))
    causal = np.tril(np.ones((n, n), dtype=bool))
    for h in range(hq):
        g = h // G
        s = scale * (q[h] @ k[g].T)
        s = np.where(causal, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        a_v[g] += p.sum(axis=0)
        for o in range(n):
            a_s[g, o] += np.diagonal(p, offset=-o).sum()
    return a_v, a_s


@pytest.mark.parametrize("hq,hkv,n,d", [(1, 1, 1, 8), (2, 1, 17, 16), (4, 2, 64, 32), (8, 2, 50, 64)])
def test_aggregate_matches_explicit_matrices(hq, hkv, n, d):
    rng = np.random.default_rng(hq * 100 + n)
    q = rng.standard_normal((hq, n, d))
    k = rng.standard_normal((hkv, n, d))
    scale = 1.0 / math.sqrt(d)
    a_v, a_s = oracle.aggregate(q, k, scale)
    e_v, e_s = _explicit_aggregate(q, k, scale)
    np.testing.assert_allclose(a_v, e_v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a_s, e_s, rtol=1e-12, atol=1e-12)


def test_aggregate_row_sums_and_uniform_closed_form():
    """Rows of P sum to 1, so each sum totals G*n; with Q = 0 every row is
    uniform over j <= i, so a_v[j] = a_s[j] = G * (H_n - H_j)."""
    rng = np.random.default_rng(61)
    hq, hkv, n, d = 8, 2, 300, 32
    q = rng.standard_normal((hq, n, d))
    k = rng.standard_normal((hkv, n, d))
    a_v, a_s = oracle.aggregate(q, k)
    np.testing.assert_allclose(a_v.sum(axis=1), 4 * n, rtol=1e-12)
    np.testing.assert_allclose(a_s.sum(axis=1), 4 * n, rtol=1e-12)
    a_v, a_s = oracle.aggregate(np.zeros_like(q), k)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    want = 4 * (H[n] - H[:n])
    for g in range(hkv):
        np.testing.assert_allclose(a_v[g], want, rtol=1e-12)
        np.testing.assert_allclose(a_s[g], want, rtol=1e-12)


def test_aggregate_diagonal_attention():
    """Keys equal to their queries times a large factor: each row attends to
    itself, so all mass sits on offset 0 and on the row's own column."""
    rng = np.random.default_rng(62)
    hq, hkv, n, d = 1, 1, 40, 64
    x = rng.standard_normal((1, n, d))
    x /= np.linalg.norm(x, axis=2, keepdims=True)
    a_v, a_s = oracle.aggregate(x * 30.0, x * 30.0, scale=1.0)
    assert a_s[0, 0] > n - 1e-3
    np.testing.assert_allclose(a_v[0], 1.0, atol=2e-3)


# ------------------------------------------- per-query-head sets, packed batches

def test_qh_sets_equal_shared_sets_when_identical_within_group():
    """Per-query-head sets that repeat the group's set give the shared result."""
    rng = np.random.default_rng(31)
    hkv, group, n, d = 2, 3, 120, 16
    q = rng.standard_normal((hkv * group, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    lv = [[0, 5, 77], [3, 9]]
    lo = [[0, 1, 30], [0, 2, 4, 100]]
    shared = _lists(hkv, lv, lo)
    per_q = _lists(hkv * group, [lv[h // group] for h in range(hkv * group)],
                   [lo[h // group] for h in range(hkv * group)])
    o1, l1 = oracle.attn(q, k, v, *shared)
    o2, l2 = oracle.attn_qh(q, k, v, *per_q)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_qh_all_offsets_is_dense_causal_sdpa():
    """Head 0 gets every offset, head 1 only the diagonal: SDPA per head."""
    rng = np.random.default_rng(32)
    n, d = 64, 8
    q = rng.standard_normal((2, n, d))
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((1, n, d))
    sets = _lists(2, [[], []], [list(range(n)), [0]])
    out, _ = oracle.attn_qh(q, k, v, *sets)
    np.testing.assert_allclose(out[0], _sdpa(q[:1], k, v, 1, causal=True)[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[1], np.repeat(v, 1, 0)[0], rtol=0, atol=1e-12)


def test_varlen_sequences_are_independent_and_match_single_calls():
    rng = np.random.default_rng(33)
    hkv, group, d = 2, 2, 16
    cu = [0, 70, 70, 200, 201]
    total = cu[-1]
    q = rng.standard_normal((hkv * group, total, d))
    k = rng.standard_normal((hkv, total, d))
    v = rng.standard_normal((hkv, total, d))
    per_seq = [_lists(hkv, [[0, 3], [1]], [[0, 1, 2], [0, 5]]) for _ in range(4)]
    stack = [np.stack([ps[i] for ps in per_seq]) for i in range(4)]
    out, lse = oracle.attn_varlen(q, k, v, cu, *stack)
    for s in range(4):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        o, l = oracle.attn(q[:, a:b], k[:, a:b], v[:, a:b], *per_seq[s])
        np.testing.assert_array_equal(out[:, a:b], o)
        np.testing.assert_array_equal(lse[:, a:b], l)
    # sampled rows equal the full computation's rows
    srows = np.array([[0, 0], [3, 69], [1, 70], [2, 150], [3, 200]], np.int32)
    so, sl = oracle.attn_varlen(q, k, v, cu, *stack, rows=srows)
    np.testing.assert_array_equal(so, out[srows[:, 0], srows[:, 1]])
    np.testing.assert_array_equal(sl, lse[srows[:, 0], srows[:, 1]])
    # changing the last sequence's keys leaves the others untouched
    k2 = k.copy()
    k2[:, 200:] += 1.0
    out2, _ = oracle.attn_varlen(q, k2, v, cu, *stack)
    np.testing.assert_array_equal(out2[:, :200], out[:, :200])
    # a single sequence with every offset is dense causal attention (SDPA)
    one = [np.stack([x]) for x in _lists(hkv, [[], []], [list(range(70))] * 2)]
    out3, _ = oracle.attn_varlen(q[:, :70], k[:, :70], v[:, :70], [0, 70], *one)
    np.testing.assert_allclose(out3, _sdpa(q[:, :70], k[:, :70], v[:, :70], group, causal=True),
                               rtol=0, atol=1e-12)
