"""Host-side logic of bench.py that the reported numbers rest on: the
closed-form pair count behind the algorithmic flops, the per-row set sizes
behind the CPU baseline's rate, and the code digest that decides whether a
recorded counter reading still applies."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _brute_pairs(cols, offs, n):
    """sum_i |S_i| with S_i = {j <= i : j in cols or i - j in offs}, by enumeration."""
    c = np.zeros(n, bool)
    c[cols] = True
    o = np.zeros(n, bool)
    o[offs] = True
    total = 0
    for i in range(n):
        j = np.arange(i + 1)
        total += int((c[j] | o[i - j]).sum())
    return total


def _lists(rng, hkv, n, dup=True):
    vl, ol = [], []
    for _ in range(hkv):
        cols = rng.choice(n, rng.integers(0, n // 3 + 1), replace=False)
        offs = rng.choice(n, rng.integers(0, n // 3 + 1), replace=False)
        if dup and len(cols):
            cols = np.concatenate([cols, cols[:2], [-1, n + 5]])  # duplicates and out-of-range entries
        vl.append(cols)
        ol.append(offs)
    cap_v = max(1, max(len(x) for x in vl))
    cap_s = max(1, max(len(x) for x in ol))
    vidx = np.full((hkv, cap_v), -1, np.int32)
    soff = np.full((hkv, cap_s), -1, np.int32)
    for g in range(hkv):
        vidx[g, :len(vl[g])] = vl[g]
        soff[g, :len(ol[g])] = ol[g]
    return vidx, np.array([len(x) for x in vl], np.int32), soff, np.array([len(x) for x in ol], np.int32)


def test_pair_counts_closed_form_matches_enumeration():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 64, 65, 300):
        vidx, vcnt, soff, scnt = _lists(rng, 3, n)
        got = bench.pair_counts(vidx, vcnt, soff, scnt, n)
        for g in range(3):
            c = vidx[g, :vcnt[g]]
            o = soff[g, :scnt[g]]
            want = _brute_pairs(np.unique(c[(c >= 0) & (c < n)]), np.unique(o[(o >= 0) & (o < n)]), n)
            assert got[g] == want, (n, g)


def test_pair_counts_special_cases():
    n = 100
    allx = np.arange(n, dtype=np.int32)[None]
    none = np.full((1, 1), -1, np.int32)
    causal = n * (n + 1) // 2
    cnt_all, cnt_none = np.array([n], np.int32), np.array([0], np.int32)
    assert bench.pair_counts(allx, cnt_all, none, cnt_none, n)[0] == causal
    assert bench.pair_counts(none, cnt_none, allx, cnt_all, n)[0] == causal
    assert bench.pair_counts(allx, cnt_all, allx, cnt_all, n)[0] == causal
    # offset 0 alone is the diagonal; column 0 alone is the first column
    zero = np.zeros((1, 1), np.int32)
    one = np.array([1], np.int32)
    assert bench.pair_counts(none, cnt_none, zero, one, n)[0] == n
    assert bench.pair_counts(zero, one, none, cnt_none, n)[0] == n
    assert bench.pair_counts(zero, one, zero, one, n)[0] == 2 * n - 1


def test_row_sizes_match_enumeration():
    rng = np.random.default_rng(4)
    n, hkv, group = 200, 2, 3
    vidx, vcnt, soff, scnt = _lists(rng, hkv, n, dup=False)
    rows = np.array([[h, i] for h in range(hkv * group) for i in (0, 1, 57, n - 1)])
    got = bench.row_sizes(vidx, vcnt, soff, scnt, rows, group)
    for (h, i), size in zip(rows, got):
        g = h // group
        c = set(vidx[g, :vcnt[g]].tolist())
        o = set(soff[g, :scnt[g]].tolist())
        assert size == sum(1 for j in range(i + 1) if j in c or (i - j) in o)


def test_code_digest_ignores_comments_only():
    a = "int f(int x) {\n  // add one\n  return x + 1; /* done */\n}\n"
    b = "int f(int x) {\n  // increment\n  return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert bench.source_digest(bench.ATTN_SOURCES) == bench.source_digest(bench.ATTN_SOURCES)
