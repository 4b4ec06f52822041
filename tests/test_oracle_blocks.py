"""Pins for the FlashPrefill block path of the CPU oracle (no GPU).

FlashPrefill (gist.science summary of arXiv 2603.06199, Spanish page,
section 2.A 'Estrategia de Aproximacion de Bloques' and 2.B 'Umbralizacion
Dinamica Basada en Maximos').  Each function is checked against hand-derived
values, closed forms, torch SDPA in fp64, the vertical-slash oracle (an
independent code path) or invariants of the definitions, so that a wrong
mean, a wrong probe row or count, a missing normaliser, a strict instead of
non-strict comparison or a threshold taken in the wrong precision fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
BS = oracle.BLOCK


# ----------------------------------------------------------------- block means

def test_block_means_arithmetic_keys():
    """k[g][j][t] = j + 10 t: a block's mean is its middle position (+10 t);
    the short last block averages only the keys it has."""
    hkv, n, d = 2, 3 * BS + 5, 3
    j = np.arange(n, dtype=np.float64)
    k = np.broadcast_to(j[None, :, None] + 10.0 * np.arange(d)[None, None, :], (hkv, n, d)).copy()
    kbar = oracle.block_means(k)
    assert kbar.shape == (hkv, 4, d)
    for J in range(3):
        np.testing.assert_allclose(kbar[:, J, 0], J * BS + (BS - 1) / 2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(kbar[:, 3, 0], (3 * BS + n - 1) / 2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(kbar[:, :, 2] - kbar[:, :, 0], 20.0, rtol=0, atol=1e-12)


def test_block_means_bf16_input():
    """bf16 bits decode to the same small integers."""
    n, d = 2 * BS, 2
    k = np.zeros((1, n, d), np.float32)
    k[0, :, 0] = np.arange(n) % 8          # integers exact in bf16
    bits = (k.view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_allclose(oracle.block_means(bits)[0, :, 0], 3.5, rtol=0, atol=0)


def test_am_gm_proxy_bound():
    """exp(scale q . kbar_J) is the geometric mean of exp(scale q . k_j) over
    the block, so it never exceeds their arithmetic mean, with equality when
    the block's keys are equal."""
    rng = np.random.default_rng(3)
    n, d = 4 * BS, 16
    k = rng.standard_normal((1, n, d))
    k[0, BS:2 * BS] = k[0, BS]               # block 1: equal keys
    kbar = oracle.block_means(k)[0]
    for q in rng.standard_normal((20, d)):
        gm = np.exp(kbar @ q * 0.3)
        am = np.exp((k[0] @ q * 0.3).reshape(4, BS)).mean(1)
        assert (gm <= am * (1 + 1e-12)).all()
        np.testing.assert_allclose(gm[1], am[1], rtol=1e-12)


# ----------------------------------------------------------------- block scores

def test_scores_hand_values():
    """d = 2, scale 1, one probe row per block with q = (1, 0); block means
    (0, 0), (ln 2, 0), (ln 3, 0) (keys +/- 0.25 around them in the second
    coordinate, so the mean and not any one key is used): query block 3 sees
    z = 0, ln 2, ln 3, so its scores are 1/6, 2/6, 3/6."""
    n, d = 4 * BS, 2
    k = np.zeros((1, n, d))
    for J, c in enumerate([0.0, math.log(2), math.log(3), 5.0]):
        k[0, J * BS:(J + 1) * BS, 0] = c
        k[0, J * BS:(J + 1) * BS, 1] = np.where(np.arange(BS) % 2 == 0, 0.25, -0.25)
    q = np.zeros((1, n, d))
    q[0, :, 0] = 1.0
    sc = oracle.block_scores(q, k, skel=1, scale=1.0)[0]
    np.testing.assert_allclose(sc[3, :3], [1 / 6, 2 / 6, 3 / 6], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sc[2, :2], [1 / 3, 2 / 3], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sc[1, :1], [1.0], rtol=0, atol=1e-14)
    assert (sc[np.triu_indices(4)] == 0).all()


@pytest.mark.parametrize("group,skel", [(1, 1), (4, 8), (2, 64)])
def test_scores_uniform_when_q_zero(group, skel):
    """Q = 0: every probe is uniform over its candidates, so score = 1/I."""
    rng = np.random.default_rng(4)
    hkv, n, d = 2, 6 * BS + 7, 8
    q = np.zeros((hkv * group, n, d))
    k = rng.standard_normal((hkv, n, d))
    sc = oracle.block_scores(q, k, skel=skel)
    nb = sc.shape[1]
    for I in range(nb):
        np.testing.assert_allclose(sc[:, I, :I], 1.0 / max(I, 1), rtol=0, atol=1e-15)
        assert (sc[:, I, I:] == 0).all()


def test_scores_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(5)
    hkv, group, n, d = 2, 2, 5 * BS + 3, 16
    q = rng.standard_normal((hkv * group, n, d))
    k = rng.standard_normal((hkv, n, d))
    sc = oracle.block_scores(q, k, skel=4)
    sums = sc.sum(-1)
    np.testing.assert_allclose(sums[:, 1:], 1.0, rtol=0, atol=1e-13)
    assert (sums[:, 0] == 0).all()
    # the same vector added to every key moves every z of a probe equally
    c = rng.standard_normal(d)
    np.testing.assert_allclose(oracle.block_scores(q, k + c, skel=4), sc, rtol=0, atol=1e-12)


def test_scores_selected_rows_match_full():
    rng = np.random.default_rng(11)
    hkv, group, n, d = 2, 2, 6 * BS, 8
    q = rng.standard_normal((hkv * group, n, d))
    k = rng.standard_normal((hkv, n, d))
    full = oracle.block_scores(q, k, skel=2)
    rows = np.array([[0, 5], [1, 0], [1, 3]])
    part = oracle.block_scores(q, k, skel=2, rows=rows)
    for r, (g, I) in enumerate(rows):
        np.testing.assert_array_equal(part[r], full[g, I])


def _planted(n, d, group, skel, row_of, hot_block, amp=60.0):
    """Keys: block hot_block along e_0, the rest 0; Q: zero except one row of
    head 0 (row_of), along e_0.  Returns (q, k)."""
    k = np.zeros((1, n, d))
    k[0, hot_block * BS:(hot_block + 1) * BS, 0] = 1.0
    q = np.zeros((group, n, d))
    q[0, row_of, 0] = amp
    return q, k


@pytest.mark.parametrize("m_hot", [0, 1, 3])
def test_scores_probe_rows_and_count(m_hot):
    """Only rows bs*I + m*(bs/skel) are probes, and a probe's own
    distribution is (nearly) one-hot on the block its query points at: with
    P probes and I candidates, that block scores (1 + (P-1)/I)/P and the
    others (P-1)/(I P).  A row between probes changes nothing."""
    group, skel, d = 2, 4, 4
    n, I, hot = 8 * BS, 5, 2
    P = group * skel
    q, k = _planted(n, d, group, skel, I * BS + m_hot * (BS // skel), hot)
    sc = oracle.block_scores(q, k, skel=skel, scale=1.0)[0, I, :I]
    want = np.full(I, (P - 1) / (I * P))
    want[hot] += 1.0 / P
    np.testing.assert_allclose(sc, want, rtol=0, atol=1e-12)
    q2, _ = _planted(n, d, group, skel, I * BS + m_hot * (BS // skel) + 1, hot)
    np.testing.assert_allclose(oracle.block_scores(q2, k, skel=skel, scale=1.0)[0, I, :I],
                               1.0 / I, rtol=0, atol=1e-15)


def test_scores_short_last_block_counts_only_rows_below_n():
    """Last query block holding rows 5*bs .. 5*bs+20: with skel = 4 (probe
    step 16) its probes are offsets 0 and 16, so P = 2 per head."""
    group, skel, d = 1, 4, 4
    n, I, hot = 5 * BS + 21, 5, 1
    q, k = _planted(n, d, group, skel, I * BS + 16, hot)
    sc = oracle.block_scores(q, k, skel=skel, scale=1.0)[0, I, :I]
    P = 2
    want = np.full(I, (P - 1) / (I * P))
    want[hot] += 1.0 / P
    np.testing.assert_allclose(sc, want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- selection

def _kept_lists(mask, nb):
    dense = oracle.mask_to_dense(mask, nb)
    return [[int(j) for j in np.nonzero(dense[0, I])[0]] for I in range(nb)]


def test_block_select_golden():
    gold = json.load(open(os.path.join(GOLD, "hand_block_select.json")))
    for case in gold["cases"]:
        score = np.array(case["score"], np.float32)[None]
        nb = score.shape[1]
        mask = oracle.block_select(score, case["alpha"])
        assert _kept_lists(mask, nb) == case["kept"], case


def test_block_select_properties():
    """The diagonal is always kept, nothing above it is, the largest
    candidate is kept, and a smaller alpha keeps a superset."""
    rng = np.random.default_rng(6)
    hkv, nb = 3, 70
    score = rng.random((hkv, nb, nb)).astype(np.float32) ** 3
    prev = None
    for alpha in [1.0, 0.5, 0.1, 0.01]:
        dense = oracle.mask_to_dense(oracle.block_select(score, alpha), nb)
        assert dense[:, np.arange(nb), np.arange(nb)].all()
        assert not dense[:, np.triu(np.ones((nb, nb), bool), 1)].any()
        for g in range(hkv):
            for I in range(1, nb):
                assert dense[g, I, int(np.argmax(score[g, I, :I]))]
        if prev is not None:
            assert (dense >= prev).all()
        prev = dense


# ----------------------------------------------------------------- block attention

def _sdpa(q, k, v, group, mask=None, causal=False):
    Q = torch.from_numpy(q)
    K = torch.from_numpy(k).repeat_interleave(group, dim=0)
    V = torch.from_numpy(v).repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(
        Q[None], K[None], V[None], attn_mask=None if mask is None else torch.from_numpy(mask),
        is_causal=causal)[0].numpy()


def _mask_from_dense(dense):
    hkv, nb, _ = dense.shape
    wpr = oracle.words_per_row(nb)
    padded = np.zeros((hkv, nb, wpr * 32), bool)
    padded[..., :nb] = dense
    return np.packbits(padded, axis=-1, bitorder="little").view(np.uint32).reshape(hkv, nb, wpr)


def test_block_attn_full_mask_is_dense_causal():
    rng = np.random.default_rng(7)
    hkv, group, n, d = 2, 2, 3 * BS + 9, 16
    q = rng.standard_normal((hkv * group, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    nb = 4
    dense = np.tril(np.ones((nb, nb), bool))[None].repeat(hkv, 0)
    dense |= np.triu(rng.random((hkv, nb, nb)) < 0.5, 1)   # bits above the diagonal change nothing
    out, lse = oracle.block_attn(q, k, v, _mask_from_dense(dense))
    np.testing.assert_allclose(out, _sdpa(q, k, v, group, causal=True), rtol=0, atol=1e-12)
    assert np.isfinite(lse).all()


def test_block_attn_diagonal_mask_is_block_local():
    rng = np.random.default_rng(8)
    hkv, group, n, d = 1, 3, 2 * BS + 30, 8
    q = rng.standard_normal((group, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    nb = 3
    out, _ = oracle.block_attn(q, k, v, _mask_from_dense(np.eye(nb, dtype=bool)[None]))
    allowed = np.zeros((n, n), bool)
    for I in range(nb):
        a, b = I * BS, min(n, (I + 1) * BS)
        allowed[a:b, a:b] = np.tril(np.ones((b - a, b - a), bool))
    np.testing.assert_allclose(out, _sdpa(q, k, v, group, mask=allowed), rtol=0, atol=1e-12)


def test_block_attn_first_block_only_matches_vertical_columns():
    """Keeping only key block 0 for every query block is the vertical set
    {0..bs-1} with no slash offsets, computed by the vertical-slash oracle."""
    rng = np.random.default_rng(9)
    hkv, group, n, d = 2, 2, 3 * BS, 16
    q = rng.standard_normal((hkv * group, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    dense = np.zeros((hkv, 3, 3), bool)
    dense[:, :, 0] = True
    out, lse = oracle.block_attn(q, k, v, _mask_from_dense(dense))
    vidx = np.tile(np.arange(BS, dtype=np.int32), (hkv, 1))
    vcnt = np.full(hkv, BS, np.int32)
    soff = np.full((hkv, 1), -1, np.int32)
    scnt = np.zeros(hkv, np.int32)
    ro, rl = oracle.attn(q, k, v, vidx, vcnt, soff, scnt)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-13)


def test_block_attn_empty_row_convention():
    rng = np.random.default_rng(10)
    n, d = 2 * BS, 4
    q, k, v = (rng.standard_normal((1, n, d)) for _ in range(3))
    dense = np.array([[[True, False], [False, False]]])
    out, lse = oracle.block_attn(q, k, v, _mask_from_dense(dense))
    assert (out[0, BS:] == 0).all() and np.isneginf(lse[0, BS:]).all()
    assert np.isfinite(lse[0, :BS]).all()
