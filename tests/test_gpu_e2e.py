"""The end-to-end layer at n=262144: 32 query / 8 KV heads, d=128, bf16 with
RoPE, keys of the first four positions scaled by 4.  vs_index ->
vs_select (mass 0.95, uncapped, both kinds) -> vs_sparse_attn_prefill, each
stage checked against the oracle on the GPU's own inputs to that stage:
sampled indexer logits within 1e-3; the selection bit-exact against the
oracle's selection of the same fp32 logits; attention rows within the
attention tolerance against the oracle on the GPU's index sets, stratified
over the sequence: the edge rows, 2 rows from each of 64 query blocks spread
over the sequence for every head, and 2 whole interior query blocks of every
head (about 8400 rows)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import vertical_slash_sparse_amd as vsa
import workloads
from tests.util import INDEX_ATOL, assert_attn_close, stratified_rows, to_dev

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_e2e256k_stage_by_stage():
    w = workloads.WORKLOADS["e2e256k"]
    n, hq, hkv, d, mass = w["n"], w["hq"], w["hkv"], w["d"], w["mass"]
    _log("case: e2e256k inputs")
    q, k, v = workloads.attention_inputs("e2e256k")
    w1, w2 = workloads.indexer_weights(workloads.streams(w["seed"])["w"], 2 * d, w["hidden"])
    kd, vd = to_dev(k), to_dev(v)
    _log("case: e2e256k GPU pipeline")
    gv, gs = vsa.vs_index(kd, vd, to_dev(w1), to_dev(w2))
    vi, vc = vsa.vs_select(gv, vsa.VS_VERTICAL, mass, n)
    si, sc = vsa.vs_select(gs, vsa.VS_SLASH, mass, n)
    out, lse = vsa.vs_sparse_attn_prefill(to_dev(q), kd, vd, vi, vc, si, sc)
    torch.cuda.synchronize()

    _log("case: e2e256k indexer logits")
    gv_np, gs_np = gv.cpu().numpy(), gs.cpu().numpy()
    rng = np.random.default_rng(17)
    pos = np.unique(np.concatenate([[0, 1, 2, 3, 4, n - 1], rng.choice(n, 1000, replace=False)]))
    rv, rsl = oracle.index(k[:, pos], v[:, pos], w1, w2)
    assert np.abs(gv_np[:, pos] - rv).max() <= INDEX_ATOL
    assert np.abs(gs_np[:, pos] - rsl).max() <= INDEX_ATOL

    _log("case: e2e256k selection")
    lists = []
    for kind, lg, gi, gc in ((oracle.VERTICAL, gv_np, vi, vc), (oracle.SLASH, gs_np, si, sc)):
        ri, rc = oracle.select(lg, kind, mass, n)
        gi_np, gc_np = gi.cpu().numpy(), gc.cpu().numpy()
        np.testing.assert_array_equal(gc_np, rc, err_msg=f"kind {kind}: counts")
        np.testing.assert_array_equal(gi_np, ri, err_msg=f"kind {kind}: indices")
        lists += [gi_np, gc_np]

    _log("case: e2e256k attention rows")
    rows = stratified_rows(np.random.default_rng(19), hq, n)
    _log(f"case: e2e256k attention, {len(rows)} rows")
    _log(f"case: e2e256k attention, {len(rows)} rows")
    hs = torch.from_numpy(rows[:, 0].astype(np.int64)).cuda()
    ps = torch.from_numpy(rows[:, 1].astype(np.int64)).cuda()
    g_out = out[hs, ps].float().cpu().numpy().astype(np.float64)
    g_lse = lse[hs, ps].cpu().numpy().astype(np.float64)
    ro, rl = oracle.attn(q, k, v, *lists, rows=rows)
    assert_attn_close(g_out, g_lse, ro, rl, "e2e256k")


PREFILL_CASES = [
    # hq, hkv, n, mass, cap_v, cap_s
    (8, 2, 1500, 0.95, None, None),
    (16, 4, 3000 + 5, 0.6, 300, 200),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"h{c[0]}x{c[1]}-n{c[2]}-m{c[3]}" for c in PREFILL_CASES])
def test_vs_prefill_pipeline(case):
    """vs_prefill (index -> select x2 -> attention in one call), every stage
    against the oracle on the GPU's own inputs to that stage, and every row of
    the output against the oracle on the GPU's index sets."""
    hq, hkv, n, mass, cap_v, cap_s = case
    _log(f"case: vs_prefill {case}")
    rng = np.random.default_rng(n)
    d = 128
    tables = workloads.rope_tables(n, d)
    q = workloads.gaussian_heads(rng, hq, n, d, "bf16", tables)
    k = workloads.gaussian_heads(rng, hkv, n, d, "bf16", tables)
    v = workloads.gaussian_heads(rng, hkv, n, d, "bf16", None)
    w1, w2 = workloads.indexer_weights(rng, 2 * d, 128)
    out, lse, (vi, vc, si, sc) = vsa.vs_prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(w1), to_dev(w2),
                                                mass, cap_v, cap_s)
    gv, gs = vsa.vs_index(to_dev(k), to_dev(v), to_dev(w1), to_dev(w2))
    torch.cuda.synchronize()
    gv_np, gs_np = gv.cpu().numpy(), gs.cpu().numpy()
    rv, rs = oracle.index(k, v, w1, w2)
    assert np.abs(gv_np - rv).max() <= INDEX_ATOL
    assert np.abs(gs_np - rs).max() <= INDEX_ATOL
    lists = []
    for kind, lg, gi, gc, cap in ((oracle.VERTICAL, gv_np, vi, vc, cap_v or n), (oracle.SLASH, gs_np, si, sc, cap_s or n)):
        ri, rc = oracle.select(lg, kind, mass, cap)
        np.testing.assert_array_equal(gc.cpu().numpy(), rc, err_msg=f"kind {kind}: counts")
        np.testing.assert_array_equal(gi.cpu().numpy(), ri, err_msg=f"kind {kind}: indices")
        lists += [ri, rc]
    ro, rl = oracle.attn(q, k, v, *lists)
    from tests.util import to_f64
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"vs_prefill {case}")
