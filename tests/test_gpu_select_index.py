"""GPU parity of vs_select (bit-exact) and vs_index (max-abs 1e-3) against
the oracle, and the full-size pipelines at 128K and 256K tokens checked
stage by stage."""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import vertical_slash_sparse_amd as vsa
import workloads
from tests.util import INDEX_ATOL, assert_attn_close, stratified_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _select_both(logit: np.ndarray, kind: int, mass: float, cap: int):
    gi, gc = vsa.vs_select(to_dev(logit), kind, mass, cap)
    torch.cuda.synchronize()
    gi, gc = gi.cpu().numpy(), gc.cpu().numpy()
    ri, rc = oracle.select(logit, kind, mass, cap)
    return gi, gc, ri, rc


def _assert_same_selection(gi, gc, ri, rc, what):
    np.testing.assert_array_equal(gc, rc, err_msg=f"{what}: counts")
    np.testing.assert_array_equal(gi, ri, err_msg=f"{what}: indices")


SELECT_CASES = [
    # name, heads, n, mass, cap
    ("normal", 8, 131072, 0.95, 131072),
    ("normal-capped", 8, 131072, 0.95, 4096),
    ("normal-lowmass", 4, 50000, 0.3, 50000),
    ("wide", 2, 20000, 0.9, 20000),
    ("ties", 3, 10000, 0.7, 10000),
    ("ties-capped", 3, 10000, 0.99, 1234),
    ("equal", 2, 4097, 0.5, 4097),
    ("signed-zero", 1, 9, 0.5, 9),
    ("tiny-mass", 4, 3000, 1e-12, 3000),
    ("all-mass", 4, 3000, 1.0, 3000),
    ("cap-one", 4, 3000, 0.95, 1),
    ("n-one", 3, 1, 0.95, 1),
    ("far-tail", 2, 5000, 0.999999, 5000),
]


def _logits(name, heads, n, rng):
    if name.startswith("normal"):
        return rng.standard_normal((heads, n)).astype(np.float32)
    if name == "wide":
        return (rng.standard_normal((heads, n)) * 30).astype(np.float32)
    if name.startswith("ties"):
        return rng.choice(np.array([0.0, -0.25, -1.0, -2.5], np.float32), size=(heads, n))
    if name == "equal":
        return np.full((heads, n), 3.5, np.float32)
    if name == "signed-zero":
        return np.array([[-0.0, 0.0, -1.0, -0.0, 0.0, -3.0, 0.0, -0.0, -40.0]], np.float32)
    if name == "far-tail":
        return (rng.standard_normal((heads, n)) * 8).astype(np.float32)
    return rng.standard_normal((heads, n)).astype(np.float32) * 2


@pytest.mark.parametrize("kind", [vsa.VS_VERTICAL, vsa.VS_SLASH], ids=["vertical", "slash"])
@pytest.mark.parametrize("case", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_bit_exact(case, kind):
    name, heads, n, mass, cap = case
    _log(f"case: select {name} kind={kind}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    logit = _logits(name, heads, n, rng)
    _assert_same_selection(*_select_both(logit, kind, mass, cap), name)


def test_select_zipf_workload():
    """Zipf(1.1) score vectors at n=131072, mass 0.95, caps 4096 / 8192."""
    _log("case: select zipf128k")
    w = workloads.WORKLOADS["zipf128k"]
    vlog, slog = workloads.zipf_scores("zipf128k")
    gi, gc, ri, rc = _select_both(vlog, vsa.VS_VERTICAL, w["mass"], w["cap_v"])
    _assert_same_selection(gi, gc, ri, rc, "zipf vertical")
    assert (gc == w["cap_v"]).all()
    gi, gc, ri, rc = _select_both(slog, vsa.VS_SLASH, w["mass"], w["cap_s"])
    _assert_same_selection(gi, gc, ri, rc, "zipf slash")
    assert (gc == w["cap_s"]).all()


def test_index_small_vs_oracle():
    _log("case: index small")
    rng = np.random.default_rng(4)
    hkv, n, d = 3, 1000, 128
    k = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    v = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    w1, w2 = workloads.indexer_weights(rng, 2 * d, 128)
    gv, gs = vsa.vs_index(to_dev(k), to_dev(v), to_dev(w1), to_dev(w2))
    torch.cuda.synchronize()
    rv, rs = oracle.index(k, v, w1, w2)
    assert np.abs(gv.cpu().numpy() - rv).max() <= INDEX_ATOL
    assert np.abs(gs.cpu().numpy() - rs).max() <= INDEX_ATOL
    # ragged: n not a multiple of the 32-row step, one head
    gv, gs = vsa.vs_index(to_dev(k[:1, :77]), to_dev(v[:1, :77]), to_dev(w1), to_dev(w2))
    torch.cuda.synchronize()
    rv, rs = oracle.index(k[:1, :77], v[:1, :77], w1, w2)
    assert np.abs(gv.cpu().numpy() - rv).max() <= INDEX_ATOL
    assert np.abs(gs.cpu().numpy() - rs).max() <= INDEX_ATOL


INDEX_SHAPES = [
    # hkv, n, d, hidden
    (2, 1000, 64, 128),
    (3, 777, 128, 32),
    (1, 2048 + 5, 128, 64),
    (2, 1500, 64, 96),
    (2, 999, 128, 160),
    (4, 3000, 128, 256),
    (2, 333, 64, 256),
    (1, 31, 64, 224),
]


@pytest.mark.parametrize("case", INDEX_SHAPES, ids=[f"h{c[0]}-n{c[1]}-d{c[2]}-hid{c[3]}" for c in INDEX_SHAPES])
def test_index_shapes_vs_oracle(case):
    """Head dims 64 and 128 and hidden widths from 32 to 256 (multiples of
    32; up to four chunks of 32 hidden units leave some waves idle, more
    than four give a wave two chunks), weights N(0, 1/fan_in), every logit
    against the oracle within 1e-3."""
    hkv, n, d, hidden = case
    _log(f"case: index shape {case}")
    rng = np.random.default_rng(hkv * 131 + n + d + hidden)
    k = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    v = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d)))
    w1, w2 = workloads.indexer_weights(rng, 2 * d, hidden)
    gv, gs = vsa.vs_index(to_dev(k), to_dev(v), to_dev(w1), to_dev(w2))
    torch.cuda.synchronize()
    rv, rs = oracle.index(k, v, w1, w2)
    assert np.abs(gv.cpu().numpy() - rv).max() <= INDEX_ATOL
    assert np.abs(gs.cpu().numpy() - rs).max() <= INDEX_ATOL


def test_indexer_workload_full_size():
    """8 KV heads x 131072 positions: sampled logits vs the oracle, then the
    selection of the GPU logits bit-exact against the oracle's selection of
    the same logits."""
    _log("case: indexer128k")
    k, v, w1, w2 = workloads.indexer_inputs("indexer128k")
    gv, gs = vsa.vs_index(to_dev(k), to_dev(v), to_dev(w1), to_dev(w2))
    torch.cuda.synchronize()
    gv_np, gs_np = gv.cpu().numpy(), gs.cpu().numpy()
    rng = np.random.default_rng(9)
    pos = np.unique(np.concatenate([[0, 1, 131071], rng.choice(131072, 2000, replace=False)]))
    rv, rs = oracle.index(k[:, pos], v[:, pos], w1, w2)
    assert np.abs(gv_np[:, pos] - rv).max() <= INDEX_ATOL
    assert np.abs(gs_np[:, pos] - rs).max() <= INDEX_ATOL
    for kind, lg in ((vsa.VS_VERTICAL, gv_np), (vsa.VS_SLASH, gs_np)):
        gi, gc = vsa.vs_select(gv if kind == vsa.VS_VERTICAL else gs, kind, 0.95, 131072)
        torch.cuda.synchronize()
        ri, rc = oracle.select(lg, kind, 0.95, 131072)
        _assert_same_selection(gi.cpu().numpy(), gc.cpu().numpy(), ri, rc, f"indexer kind {kind}")


def test_zipf128k_layer_sampled():
    """The 128K layer: Zipf scores -> selection -> sparse attention, rows sampled."""
    _log("case: zipf128k layer")
    w = workloads.WORKLOADS["zipf128k"]
    q, k, v = workloads.attention_inputs("zipf128k")
    vlog, slog = workloads.zipf_scores("zipf128k")
    vi, vc = vsa.vs_select(to_dev(vlog), vsa.VS_VERTICAL, w["mass"], w["cap_v"])
    si, sc = vsa.vs_select(to_dev(slog), vsa.VS_SLASH, w["mass"], w["cap_s"])
    out, lse = vsa.vs_sparse_attn_prefill(to_dev(q), to_dev(k), to_dev(v), vi, vc, si, sc)
    torch.cuda.synchronize()
    ri, rc = oracle.select(vlog, oracle.VERTICAL, w["mass"], w["cap_v"])
    _assert_same_selection(vi.cpu().numpy(), vc.cpu().numpy(), ri, rc, "zipf vertical")
    lists = (vi.cpu().numpy(), vc.cpu().numpy(), si.cpu().numpy(), sc.cpu().numpy())
    out, lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    rows = stratified_rows(np.random.default_rng(11), 32, w["n"])
    ro, rl = oracle.attn(q, k, v, *lists, rows=rows)
    assert_attn_close(out[rows[:, 0], rows[:, 1]], lse[rows[:, 0], rows[:, 1]], ro, rl, "zipf128k")


def test_clustered128k_layer_sampled():
    """The 128K layer with clustered scores (selected columns and offsets in
    contiguous runs): both selections bit-exact, attention rows sampled."""
    _log("case: clustered128k layer")
    w = workloads.WORKLOADS["clustered128k"]
    q, k, v = workloads.attention_inputs("clustered128k")
    vlog, slog = workloads.clustered_scores("clustered128k")
    vi, vc = vsa.vs_select(to_dev(vlog), vsa.VS_VERTICAL, w["mass"], w["cap_v"])
    si, sc = vsa.vs_select(to_dev(slog), vsa.VS_SLASH, w["mass"], w["cap_s"])
    out, lse = vsa.vs_sparse_attn_prefill(to_dev(q), to_dev(k), to_dev(v), vi, vc, si, sc)
    torch.cuda.synchronize()
    for kind, lg, gi, gc, cap in ((oracle.VERTICAL, vlog, vi, vc, w["cap_v"]),
                                  (oracle.SLASH, slog, si, sc, w["cap_s"])):
        ri, rc = oracle.select(lg, kind, w["mass"], cap)
        _assert_same_selection(gi.cpu().numpy(), gc.cpu().numpy(), ri, rc, f"clustered kind {kind}")
    lists = (vi.cpu().numpy(), vc.cpu().numpy(), si.cpu().numpy(), sc.cpu().numpy())
    out, lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    rows = stratified_rows(np.random.default_rng(12), 32, w["n"])
    ro, rl = oracle.attn(q, k, v, *lists, rows=rows)
    assert_attn_close(out[rows[:, 0], rows[:, 1]], lse[rows[:, 0], rows[:, 1]], ro, rl, "clustered128k")


BOTH_CASES = [
    # heads, n, mass, cap_v, cap_s
    (8, 131072, 0.95, 131072, 131072),
    (8, 131072, 0.95, 4096, 8192),
    (3, 5000 + 7, 0.5, 100, 5007),
    (1, 1, 0.9, 1, 1),
    (5, 3000, 1.0, 3000, 17),
]


@pytest.mark.parametrize("case", BOTH_CASES, ids=[f"h{c[0]}-n{c[1]}-m{c[2]}-cv{c[3]}-cs{c[4]}" for c in BOTH_CASES])
def test_select_both_equals_two_selects(case):
    """vs_select_both runs both kinds as one chain: bit-identical to two
    vs_select calls and to the oracle's selections."""
    heads, n, mass, cap_v, cap_s = case
    _log(f"case: select both {case}")
    rng = np.random.default_rng(heads * 7 + n)
    vlog = (rng.standard_normal((heads, n)) * 2).astype(np.float32)
    slog = rng.choice(np.array([0.0, -0.5, -1.0, -3.0], np.float32), size=(heads, n)) if heads == 3 else \
        (rng.standard_normal((heads, n)) * 3).astype(np.float32)
    vi, vc, si, sc = vsa.vs_select_both(to_dev(vlog), to_dev(slog), mass, cap_v, cap_s)
    vi1, vc1 = vsa.vs_select(to_dev(vlog), vsa.VS_VERTICAL, mass, cap_v)
    si1, sc1 = vsa.vs_select(to_dev(slog), vsa.VS_SLASH, mass, cap_s)
    torch.cuda.synchronize()
    for a, b, what in ((vi, vi1, "v_idx"), (vc, vc1, "v_cnt"), (si, si1, "s_off"), (sc, sc1, "s_cnt")):
        assert torch.equal(a, b), what
    ri, rc = oracle.select(vlog, oracle.VERTICAL, mass, cap_v)
    _assert_same_selection(vi.cpu().numpy(), vc.cpu().numpy(), ri, rc, "both: vertical")
    ri, rc = oracle.select(slog, oracle.SLASH, mass, cap_s)
    _assert_same_selection(si.cpu().numpy(), sc.cpu().numpy(), ri, rc, "both: slash")


THRESH_CASES = [
    # name, heads, n, alpha, cap
    ("normal", 8, 131072, 0.01, 131072),
    ("normal-capped", 8, 131072, 0.001, 1000),
    ("tight", 4, 50000, 0.5, 50000),
    ("ties", 3, 10000, 0.3, 10000),
    ("ties-capped", 3, 10000, 0.05, 77),
    ("alpha-one", 2, 20000, 1.0, 20000),
    ("tiny-alpha", 2, 20000, 1e-12, 20000),
    ("n-one", 5, 1, 0.5, 1),
]


@pytest.mark.parametrize("case", [c + (k,) for c in THRESH_CASES for k in ("vertical", "slash")],
                         ids=[f"{c[0]}-{k}" for c in THRESH_CASES for k in ("vertical", "slash")])
def test_select_threshold_bit_exact(case):
    name, heads, n, alpha, cap, kname = case
    kind = vsa.VS_VERTICAL if kname == "vertical" else vsa.VS_SLASH
    _log(f"case: threshold select {case}")
    rng = np.random.default_rng(zlib.crc32(f"thresh-{name}-{kname}".encode()))
    if name.startswith("ties"):
        logit = rng.integers(-3, 1, size=(heads, n)).astype(np.float32) * 0.75
    else:
        logit = (rng.standard_normal((heads, n)) * 3).astype(np.float32)
    gi, gc = vsa.vs_select_threshold(to_dev(logit), kind, alpha, cap)
    torch.cuda.synchronize()
    ri, rc = oracle.select_threshold(logit, kind, alpha, cap)
    _assert_same_selection(gi.cpu().numpy(), gc.cpu().numpy(), ri, rc, f"threshold {case}")


def test_select_threshold_zipf_closed_form():
    """On Zipf(1.1) scores alpha = (K(K+1))^(-s/2) keeps exactly ranks 1..K."""
    _log("case: threshold zipf")
    w = workloads.WORKLOADS["zipf128k"]
    vlog, _ = workloads.zipf_scores("zipf128k")
    ranks = np.rint(np.exp(-vlog.astype(np.float64) / w["zipf_s"])).astype(np.int64)
    for K in (3, 50, 3000):
        alpha = (K * (K + 1.0)) ** (-w["zipf_s"] / 2)
        gi, gc = vsa.vs_select_threshold(to_dev(vlog), vsa.VS_VERTICAL, alpha, w["n"])
        torch.cuda.synchronize()
        gi, gc = gi.cpu().numpy(), gc.cpu().numpy()
        assert (gc == K).all(), (K, gc)
        for h in range(vlog.shape[0]):
            assert set(gi[h, :K].tolist()) == set(np.nonzero(ranks[h] <= K)[0].tolist())
