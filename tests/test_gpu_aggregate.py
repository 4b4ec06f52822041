"""GPU parity of vs_attn_aggregate: dense causal attention plus its weights
summed per KV head along key columns (a_v) and diagonals (a_s), against the
fp64 oracle.

Tolerance of the sums.  P is formed in fp32 from bf16 products and the lse of
the first pass; that lse normalises with the bf16-rounded probabilities the
PV product uses, whose relative error is at most 2^-9 per term, so P, and
every sum of P, is within a relative 2^-9 ~ 2e-3 of the fp64 value, plus
fp32 accumulation.  The test allows 5e-3 relative plus 1e-5 absolute.
out and lse follow the attention tolerance."""
import sys

import numpy as np
import pytest
import torch

import oracle
import vertical_slash_sparse_amd as vsa
import workloads
from tests.util import assert_attn_close, to_dev, to_f64

pytestmark = pytest.mark.gpu

REL, ABS = 5e-3, 1e-5


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_inputs(rng, hq, hkv, n, d):
    return tuple(workloads.to_bf16_bits(rng.standard_normal(shape)) for shape in
                 ((hq, n, d), (hkv, n, d), (hkv, n, d)))


def _check_sums(got, want, what):
    err = np.abs(got - want)
    bound = REL * np.abs(want) + ABS
    worst = int(np.argmax(err - bound))
    assert (err <= bound).all(), f"{what}: |diff| {err.flat[worst]:.3e} > {bound.flat[worst]:.3e} at {worst}"


CASES = [
    # hq, hkv, n, d
    (1, 1, 1, 64),
    (2, 1, 33, 128),
    (4, 4, 100, 64),
    (8, 2, 257, 128),
    (16, 1, 300, 64),
    (32, 8, 600, 128),
    (16, 2, 1000, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[f"h{c[0]}x{c[1]}-n{c[2]}-d{c[3]}" for c in CASES])
def test_aggregate_vs_oracle(case):
    hq, hkv, n, d = case
    _log(f"case: aggregate {case}")
    rng = np.random.default_rng(hq * 1000 + n)
    q, k, v = _bf16_inputs(rng, hq, hkv, n, d)
    out, lse, a_v, a_s = vsa.vs_attn_aggregate(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    r_v, r_s = oracle.aggregate(q, k)
    _check_sums(a_v.cpu().numpy().astype(np.float64), r_v, f"{case} a_v")
    _check_sums(a_s.cpu().numpy().astype(np.float64), r_s, f"{case} a_s")
    allk = [np.arange(n)] * hkv
    soff = np.stack(allk).astype(np.int32)
    scnt = np.full(hkv, n, np.int32)
    vidx = np.full((hkv, 1), -1, np.int32)
    vcnt = np.zeros(hkv, np.int32)
    ro, rl = oracle.attn(q, k, v, vidx, vcnt, soff, scnt)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"{case} attention")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.3])
def test_aggregate_any_finite_scale(scale):
    """Any finite scale: negative, zero (uniform rows) and large."""
    _log(f"case: aggregate scale {scale}")
    rng = np.random.default_rng(55)
    hq, hkv, n, d = 8, 2, 500, 128
    q, k, v = _bf16_inputs(rng, hq, hkv, n, d)
    out, lse, a_v, a_s = vsa.vs_attn_aggregate(to_dev(q), to_dev(k), to_dev(v), scale=scale)
    torch.cuda.synchronize()
    r_v, r_s = oracle.aggregate(q, k, scale=scale)
    _check_sums(a_v.cpu().numpy().astype(np.float64), r_v, f"scale {scale} a_v")
    _check_sums(a_s.cpu().numpy().astype(np.float64), r_s, f"scale {scale} a_s")
    soff = np.stack([np.arange(n)] * hkv).astype(np.int32)
    ro, rl = oracle.attn(q, k, v, np.full((hkv, 1), -1, np.int32), np.zeros(hkv, np.int32), soff,
                         np.full(hkv, n, np.int32), scale=scale)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"scale {scale}")


def test_aggregate_sums_total_group_times_n():
    """Rows of P sum to 1: each KV head's sums total G*n (4096 rows, G = 4)."""
    _log("case: aggregate totals")
    rng = np.random.default_rng(7)
    hq, hkv, n, d = 8, 2, 4096, 128
    q, k, v = _bf16_inputs(rng, hq, hkv, n, d)
    _, _, a_v, a_s = vsa.vs_attn_aggregate(to_dev(q), to_dev(k), to_dev(v))
    tv = a_v.double().sum(dim=1).cpu().numpy()
    ts = a_s.double().sum(dim=1).cpu().numpy()
    np.testing.assert_allclose(tv, 4 * n, rtol=REL)
    np.testing.assert_allclose(ts, 4 * n, rtol=REL)
    r_v, r_s = oracle.aggregate(q, k)
    _check_sums(a_v.cpu().numpy().astype(np.float64), r_v, "4096 a_v")
    _check_sums(a_s.cpu().numpy().astype(np.float64), r_s, "4096 a_s")


def test_aggregate_uniform_rows_closed_form():
    """Q = 0: every row is uniform over its keys, so a_v[j] = a_s[j] = G (H_n - H_j)."""
    _log("case: aggregate uniform")
    rng = np.random.default_rng(8)
    hq, hkv, n, d = 4, 1, 2000, 64
    q = np.zeros((hq, n, d), np.uint16)
    k = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    v = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    _, _, a_v, a_s = vsa.vs_attn_aggregate(to_dev(q), to_dev(k), to_dev(v))
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    want = 4 * (H[n] - H[:n])
    _check_sums(a_v[0].cpu().numpy().astype(np.float64), want, "uniform a_v")
    _check_sums(a_s[0].cpu().numpy().astype(np.float64), want, "uniform a_s")


def test_aggregate32k_one_kv_head_whole():
    """The 32K aggregation layer (32/8 heads, d = 128, n = 32768, the fixed
    32K layer's RoPE'd inputs): every entry of a_v and a_s of one KV head,
    drawn by seed, against the oracle over that head's 4 query heads, at the
    tolerance above.  A diagonal's partials add at most 512 rows of 2^-23
    rounding each per workgroup, at most 4 * 32768 * 2^-23 ~ 0.016 in all,
    well inside 5e-3 of the diagonal sums near o = 0 (G * H_n ~ 44)."""
    _log("case: aggregate32k one KV head")
    q, k, v = workloads.attention_inputs("fixed32k")
    hq, n, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    _, _, a_v, a_s = vsa.vs_attn_aggregate(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    g = int(np.random.default_rng(32).integers(hkv))
    gv = a_v[g].cpu().numpy().astype(np.float64)
    gs = a_s[g].cpu().numpy().astype(np.float64)
    del a_v, a_s
    _log(f"case: aggregate32k oracle on KV head {g}")
    r_v, r_s = oracle.aggregate(q[G * g:G * (g + 1)], k[g:g + 1])
    _check_sums(gv, r_v[0], f"aggregate32k a_v[{g}]")
    _check_sums(gs, r_s[0], f"aggregate32k a_s[{g}]")
    np.testing.assert_allclose(gv.sum(), G * n, rtol=REL)
    np.testing.assert_allclose(gs.sum(), G * n, rtol=REL)
