"""GPU parity of the FlashPrefill block path (vs_block_discover,
vs_block_attn_prefill) against the fp64 oracle.

Scores.  The block means are summed in fp32 and held as a bf16 pair (hi +
lo, relative error about 2^-17), the probe products run in fp32 on the
matrix cores, and probabilities come from exp2 in fp32.  A probe logit z is
then off by at most scale * sum_d |q_d| |dkbar_d|, about 2^-15 * scale *
sum_d |q_d| max_j |k_jd| -- a few 1e-4 for unit Gaussians at d = 128 in the
worst case and ~1e-5 typically -- and a score, an average of probabilities,
by about twice that relatively.  The test allows 1e-3 relative plus 1e-6
absolute.

Mask.  The keep decision is an integer taken from floating point, so both
sides take it on the same fp32 scores: the GPU's mask must equal, bit for
bit, the oracle's fp32 selection applied to the scores the GPU returns.

Attention follows the vertical-slash tolerance (max-abs 2e-2, mean-abs 2e-3
on O and lse; empty rows exactly zero with lse -inf).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import vertical_slash_sparse_amd as vsa
import workloads
from tests.util import assert_attn_close, stratified_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu

REL, ABS = 1e-3, 1e-6
BS = 64


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(rng, hq, hkv, n, d, dtype="bf16"):
    q = rng.standard_normal((hq, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    if dtype == "bf16":
        return tuple(workloads.to_bf16_bits(x) for x in (q, k, v))
    return tuple(x.astype(np.float32) for x in (q, k, v))


def _mask_np(mask_t):
    return mask_t.cpu().numpy().view(np.uint32)


def _check_scores(got, want, what):
    err = np.abs(got - want)
    bound = REL * np.abs(want) + ABS
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert (err <= bound).all(), f"{what}: |diff| {err[worst]:.3e} > {bound[worst]:.3e} at {worst}"


DISCOVER_CASES = [
    # hq, hkv, n, d, skel, alpha
    (4, 1, 64, 128, 8, 0.5),
    (8, 2, 1000, 128, 8, 0.3),
    (16, 2, 2048 + 37, 64, 4, 0.1),
    (2, 2, 700, 128, 32, 0.5),
    (32, 8, 4096, 128, 8, 0.05),
    (16, 1, 3000, 128, 2, 1.0),
    (4, 2, 33 * 64 + 1, 64, 16, 0.2),
]


@pytest.mark.parametrize("case", DISCOVER_CASES,
                         ids=[f"h{c[0]}x{c[1]}-n{c[2]}-d{c[3]}-s{c[4]}-a{c[5]}" for c in DISCOVER_CASES])
def test_discover_vs_oracle(case):
    hq, hkv, n, d, skel, alpha = case
    _log(f"case: discover {case}")
    rng = np.random.default_rng(hq * 7 + n)
    q, k, _ = _inputs(rng, hq, hkv, n, d)
    qd, kd = to_dev(q), to_dev(k)
    mask, score = vsa.vs_block_discover(qd, kd, skel, alpha, want_score=True)
    mask_only = vsa.vs_block_discover(qd, kd, skel, alpha)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    _check_scores(got.astype(np.float64), oracle.block_scores(q, k, skel), f"{case} scores")
    want_mask = oracle.block_select(got, alpha)
    assert np.array_equal(_mask_np(mask), want_mask), f"{case} mask"
    assert np.array_equal(_mask_np(mask_only), want_mask), f"{case} mask without scores"


def _random_mask(rng, hkv, n, density, diag_prob, upper=True):
    nb = (n + BS - 1) // BS
    dense = rng.random((hkv, nb, nb)) < density
    diag = rng.random((hkv, nb)) < diag_prob
    idx = np.arange(nb)
    dense[:, idx, idx] = diag
    if not upper:
        dense &= np.tril(np.ones((nb, nb), bool))
    wpr = oracle.words_per_row(nb)
    padded = np.zeros((hkv, nb, wpr * 32), bool)
    padded[..., :nb] = dense
    return np.packbits(padded, axis=-1, bitorder="little").view(np.uint32).reshape(hkv, nb, wpr)


ATTN_CASES = [
    # hq, hkv, n, d, dtype, density, diag_prob
    (1, 1, 1, 64, "bf16", 1.0, 1.0),
    (2, 1, 65, 128, "bf16", 0.5, 1.0),
    (4, 4, 300, 64, "bf16", 0.3, 0.7),
    (8, 2, 1000, 128, "bf16", 0.2, 1.0),
    (16, 1, 777, 128, "bf16", 0.4, 0.9),
    (32, 8, 2048, 128, "bf16", 0.1, 1.0),
    (16, 2, 1500, 64, "fp32", 0.3, 0.8),
    (4, 1, 4096 + 130, 128, "bf16", 0.05, 1.0),
    (2, 2, 5000, 128, "bf16", 1.0, 1.0),
]


@pytest.mark.parametrize("case", ATTN_CASES,
                         ids=[f"h{c[0]}x{c[1]}-n{c[2]}-d{c[3]}-{c[4]}-p{c[5]}" for c in ATTN_CASES])
def test_block_attn_vs_oracle(case):
    hq, hkv, n, d, dtype, density, diag_prob = case
    _log(f"case: block attn {case}")
    rng = np.random.default_rng(hq * 13 + n)
    q, k, v = _inputs(rng, hq, hkv, n, d, dtype)
    mask = _random_mask(rng, hkv, n, density, diag_prob)
    out, lse = vsa.vs_block_attn_prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(mask.view(np.int32)))
    torch.cuda.synchronize()
    ro, rl = oracle.block_attn(q, k, v, mask)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"{case}")


def test_discover_then_attend():
    """The discovered mask drives the block-sparse kernel: rows agree with the
    oracle's attention under that mask."""
    _log("case: discover + attend")
    rng = np.random.default_rng(21)
    hq, hkv, n, d = 16, 4, 3000, 128
    q, k, v = _inputs(rng, hq, hkv, n, d)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    mask = vsa.vs_block_discover(qd, kd, 8, 0.6)
    out, lse = vsa.vs_block_attn_prefill(qd, kd, vd, mask)
    torch.cuda.synchronize()
    m = _mask_np(mask)
    dense = oracle.mask_to_dense(m, m.shape[1])
    assert dense[:, np.arange(m.shape[1]), np.arange(m.shape[1])].all()
    ro, rl = oracle.block_attn(q, k, v, m)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, "discover+attend")


def test_full_size_128k_sampled():
    """32/8 heads, n = 131072, d = 128 (the 128K layer's inputs): the whole
    mask against the oracle's selection on the GPU's scores, sampled score
    rows against the oracle, and sampled attention rows against the oracle
    under the GPU's mask."""
    _log("case: blocks 128k sampled")
    q, k, v = workloads.attention_inputs("zipf128k")
    hq, n, d = q.shape
    hkv = k.shape[0]
    nb = n // BS
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    skel, alpha = 32 // (hq // hkv), 0.2
    mask, score = vsa.vs_block_discover(qd, kd, skel, alpha, want_score=True)
    out, lse = vsa.vs_block_attn_prefill(qd, kd, vd, mask)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    m = _mask_np(mask)
    assert np.array_equal(m, oracle.block_select(got, alpha)), "128k mask"
    rng = np.random.default_rng(3)
    rows = np.array([[g, I] for g in range(hkv) for I in [0, 1, 2, nb // 2, nb - 1] +
                     list(rng.choice(nb, 3, replace=False))], np.int32)
    want = oracle.block_scores(q, k, skel, rows=rows)
    _check_scores(got[rows[:, 0], rows[:, 1]].astype(np.float64), want, "128k score rows")
    srows = stratified_rows(rng, hq, n)
    ro, rl = oracle.block_attn(q, k, v, m, rows=srows)
    og = to_f64(out)[srows[:, 0], srows[:, 1]]
    lg = lse.cpu().numpy().astype(np.float64)[srows[:, 0], srows[:, 1]]
    assert_attn_close(og, lg, ro, rl, "128k attention rows")


def test_full_size_256k_discover_sampled():
    """32/8 heads, n = 262144 (4096 blocks, 537 MB of score rows in the
    workspace): the whole mask against the oracle's selection on the GPU's
    scores, sampled score rows against the oracle, and sampled attention rows
    under the mask."""
    _log("case: blocks 256k sampled")
    q, k, v = workloads.block_structured_inputs("blocks128k", n=262144)
    hq, n, d = q.shape
    hkv = k.shape[0]
    nb = n // BS
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    skel, alpha = 8, 0.1
    mask, score = vsa.vs_block_discover(qd, kd, skel, alpha, want_score=True)
    out, lse = vsa.vs_block_attn_prefill(qd, kd, vd, mask)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    del score
    m = _mask_np(mask)
    assert np.array_equal(m, oracle.block_select(got, alpha)), "256k mask"
    rng = np.random.default_rng(4)
    rows = np.array([[g, I] for g in range(hkv) for I in [1, nb // 3, nb - 1] +
                     list(rng.choice(nb, 2, replace=False))], np.int32)
    want = oracle.block_scores(q, k, skel, rows=rows)
    _check_scores(got[rows[:, 0], rows[:, 1]].astype(np.float64), want, "256k score rows")
    srows = stratified_rows(rng, hq, n)
    ro, rl = oracle.block_attn(q, k, v, m, rows=srows)
    og = to_f64(out)[srows[:, 0], srows[:, 1]]
    lg = lse.cpu().numpy().astype(np.float64)[srows[:, 0], srows[:, 1]]
    assert_attn_close(og, lg, ro, rl, "256k attention rows")


def test_max_blocks_discover_sampled():
    """The largest discovery call: nb = 16384 key blocks (n = 1048576), one KV
    head of 4 query heads, unit Gaussian bf16 inputs.  The whole mask against
    the oracle's selection on the GPU's scores; sampled score rows, the last
    block among them, against the oracle."""
    _log("case: blocks nb=16384 discover sampled")
    rng = np.random.default_rng(12)
    hq, hkv, d = 4, 1, 128
    nb = 16384
    n = nb * BS
    q = workloads.to_bf16_bits(rng.standard_normal((hq, n, d), dtype=np.float32))
    k = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d), dtype=np.float32))
    skel, alpha = 8, 0.5
    mask, score = vsa.vs_block_discover(to_dev(q), to_dev(k), skel, alpha, want_score=True)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    del score
    assert np.array_equal(_mask_np(mask), oracle.block_select(got, alpha)), "nb=16384 mask"
    rows = np.array([[0, I] for I in (1, 5000, nb - 2, nb - 1)], np.int32)
    want = oracle.block_scores(q, k, skel, rows=rows)
    _check_scores(got[rows[:, 0], rows[:, 1]].astype(np.float64), want, "nb=16384 score rows")
