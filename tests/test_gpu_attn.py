"""GPU parity of vs_sparse_attn_prefill against the fp64 oracle.

Tolerance (bf16 products, fp32 softmax and accumulation vs fp64): max-abs
2e-2 and mean-abs 2e-3 on O and on the log-sum-exp.  Small cases compare
every element; full-size workloads compare sampled rows the oracle computes
one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import vertical_slash_sparse_amd as vsa
import workloads
from tests.util import assert_attn_close, sample_rows, stratified_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pad_lists(lists, cap=None):
    cap = cap or max(1, max(len(x) for x in lists))
    arr = np.full((len(lists), cap), -1, np.int32)
    for g, x in enumerate(lists):
        arr[g, :len(x)] = x
    return arr, np.array([len(x) for x in lists], np.int32)


def _run_gpu(q, k, v, vidx, vcnt, soff, scnt, scale=None):
    out, lse = vsa.vs_sparse_attn_prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(vidx), to_dev(vcnt),
                                          to_dev(soff), to_dev(scnt), scale=scale)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _inputs(rng, hq, hkv, n, d, dtype):
    q = rng.standard_normal((hq, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    if dtype == "bf16":
        return tuple(workloads.to_bf16_bits(x) for x in (q, k, v))
    return tuple(x.astype(np.float32) for x in (q, k, v))


def _random_sets(rng, hkv, n, pv, ps, drop_zero=False):
    vl, ol = [], []
    for _ in range(hkv):
        cols = np.nonzero(rng.random(n) < pv)[0]
        offs = np.nonzero(rng.random(n) < ps)[0]
        if drop_zero:
            offs = offs[offs != 0]
        vl.append(cols)
        ol.append(offs)
    vidx, vcnt = _pad_lists(vl)
    soff, scnt = _pad_lists(ol)
    return vidx, vcnt, soff, scnt


def test_small_workload_full():
    """1 head, n=1024, d=64, fp32 inputs, 16 verticals + 16 slashes."""
    _log("case: small workload (n=1024 d=64 fp32)")
    q, k, v = workloads.attention_inputs("small")
    lists = workloads.small_index_sets("small")
    out, lse = _run_gpu(q, k, v, *lists)
    ro, rl = oracle.attn(q, k, v, *lists)
    assert_attn_close(out, lse, ro, rl, "small")


CASES = [
    # n, d, hq, hkv, dtype, pv, ps, drop_zero
    (1, 64, 1, 1, "f32", 1.0, 1.0, False),
    (17, 128, 4, 1, "bf16", 0.2, 0.3, False),
    (64, 64, 2, 1, "bf16", 0.1, 0.2, True),
    (65, 128, 8, 1, "bf16", 0.3, 0.0, False),     # verticals only: gathered tiles
    (100, 128, 8, 2, "f32", 0.0, 0.25, False),    # slashes only
    (257, 128, 32, 8, "bf16", 0.05, 0.05, True),
    (300, 64, 16, 1, "bf16", 0.02, 0.1, False),   # group of 16
    (513, 128, 4, 4, "bf16", 0.01, 0.01, True),   # group of 1, very sparse
    (777, 64, 6, 3, "bf16", 0.03, 0.02, False),   # group of 2
    (1000, 128, 8, 2, "bf16", 0.0, 0.0, False),   # nothing selected: all rows empty
    (4100, 128, 12, 3, "bf16", 0.02, 0.03, False),  # 65 blocks: XCD head rotation, 3 KV heads
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}-d{c[1]}-h{c[2]}x{c[3]}-{c[4]}" for c in CASES])
def test_random_sets_vs_oracle(case):
    n, d, hq, hkv, dtype, pv, ps, drop_zero = case
    _log(f"case: random sets {case}")
    rng = np.random.default_rng(n * 7 + d)
    q, k, v = _inputs(rng, hq, hkv, n, d, dtype)
    lists = _random_sets(rng, hkv, n, pv, ps, drop_zero)
    out, lse = _run_gpu(q, k, v, *lists)
    ro, rl = oracle.attn(q, k, v, *lists)
    assert_attn_close(out, lse, ro, rl, str(case))


@pytest.mark.parametrize("which", ["offsets", "columns"])
def test_everything_selected_equals_dense(which):
    """All offsets 0..n-1 (or all columns) selected is dense causal attention;
    the oracle is pinned to fp64 SDPA in that case."""
    _log(f"case: dense via all {which}")
    rng = np.random.default_rng(21)
    hq, hkv, n, d = 8, 2, 700, 128
    q, k, v = _inputs(rng, hq, hkv, n, d, "bf16")
    allx = [np.arange(n)] * hkv
    none = [np.zeros(0, np.int64)] * hkv
    vidx, vcnt = _pad_lists(allx if which == "columns" else none)
    soff, scnt = _pad_lists(allx if which == "offsets" else none)
    out, lse = _run_gpu(q, k, v, vidx, vcnt, soff, scnt)
    ro, rl = oracle.attn(q, k, v, vidx, vcnt, soff, scnt)
    assert_attn_close(out, lse, ro, rl, which)


def test_value_ones_gives_ones():
    _log("case: V == 1")
    rng = np.random.default_rng(5)
    hq, hkv, n, d = 8, 2, 4096, 128
    q, k, _ = _inputs(rng, hq, hkv, n, d, "bf16")
    v = workloads.to_bf16_bits(np.ones((hkv, n, d)))
    lists = _random_sets(rng, hkv, n, 0.01, 0.02, drop_zero=True)
    out, lse = _run_gpu(q, k, v, *lists)
    nonempty = np.isfinite(lse)
    assert nonempty.any() and (~nonempty).any()
    assert np.abs(out[nonempty] - 1.0).max() <= 2e-2
    assert (out[~nonempty] == 0).all()


def _grid_cases():
    # work items are (KV head, 64-row block) pairs; the kernel's persistent
    # grid holds one workgroup per CU: item counts just past one and two
    # grids (the per-XCD queues, then stealing), and fewer items than queues
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    m1 = cus // 8 + 1
    return [(8, 32, 64 * m1), (8, 32, 64 * (2 * m1) - 17), (1, 4, 64 * 5 - 3)]


@pytest.mark.parametrize("case", _grid_cases(), ids=lambda c: f"h{c[1]}x{c[0]}-n{c[2]}")
def test_item_counts_around_the_persistent_grid(case):
    """Every item is taken exactly once: item counts past one and two grids
    of workgroups and below the number of queues, with uneven work per item
    (random sets), compared in full with the oracle."""
    hkv, hq, n = case
    _log(f"case: persistent grid items {case}")
    rng = np.random.default_rng(n + hkv)
    q, k, v = _inputs(rng, hq, hkv, n, 128, "bf16")
    lists = _random_sets(rng, hkv, n, 0.03, 0.05)
    out, lse = _run_gpu(q, k, v, *lists)
    ro, rl = oracle.attn(q, k, v, *lists)
    assert_attn_close(out, lse, ro, rl, f"grid items {case}")


def test_index_list_contract():
    """Lists may come in any order; duplicates and out-of-range entries are
    ignored; counts beyond the capacity are clamped."""
    _log("case: list contract")
    rng = np.random.default_rng(8)
    hq, hkv, n, d = 4, 1, 300, 64
    q, k, v = _inputs(rng, hq, hkv, n, d, "bf16")
    vraw = np.array([[3, 3, 7, 500, -2, 9, 9]], np.int32)
    oraw = np.array([[0, 0, 5, 1000, -1, 17]], np.int32)
    out, lse = _run_gpu(q, k, v, vraw, np.array([99], np.int32), oraw, np.array([6], np.int32))
    clean_v, cv = _pad_lists([np.array([3, 7, 9])])
    clean_o, co = _pad_lists([np.array([0, 5, 17])])
    ro, rl = oracle.attn(q, k, v, clean_v, cv, clean_o, co)
    assert_attn_close(out, lse, ro, rl, "contract")


SCALES = [-0.125, 0.0, -0.0, 0.5, -2.0]


@pytest.mark.parametrize("scale", SCALES, ids=[repr(s) for s in SCALES])
def test_any_finite_scale(scale):
    """The softmax scale may be any finite value: negative (every score's
    sign flips), zero (each row is the mean of V over its set) or large.
    Vertical-slash and block-sparse attention against the oracle at that
    scale."""
    _log(f"case: scale {scale}")
    rng = np.random.default_rng(int(abs(scale) * 1000) + 3)
    hq, hkv, n, d = 8, 2, 700, 128
    q, k, v = _inputs(rng, hq, hkv, n, d, "bf16")
    lists = _random_sets(rng, hkv, n, 0.05, 0.1)
    out, lse = _run_gpu(q, k, v, *lists, scale=scale)
    ro, rl = oracle.attn(q, k, v, *lists, scale=scale)
    assert_attn_close(out, lse, ro, rl, f"scale {scale}")
    nb = (n + 63) // 64
    dense = rng.random((hkv, nb, nb)) < 0.4
    dense[:, np.arange(nb), np.arange(nb)] = True
    wpr = oracle.words_per_row(nb)
    padded = np.zeros((hkv, nb, wpr * 32), bool)
    padded[..., :nb] = dense
    mask = np.packbits(padded, axis=-1, bitorder="little").view(np.uint32).reshape(hkv, nb, wpr)
    bo, bl = vsa.vs_block_attn_prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(mask.view(np.int32)),
                                       scale=scale)
    torch.cuda.synchronize()
    rbo, rbl = oracle.block_attn(q, k, v, mask, scale=scale)
    assert_attn_close(to_f64(bo), bl.cpu().numpy().astype(np.float64), rbo, rbl, f"block scale {scale}")


def test_long_lists_with_out_of_range_entries():
    """Lists of 1.5 M entries per KV head (the bit-setting pass covers more
    than 2^20 entries by striding), nearly all of them outside [0, n), with
    the in-range ones placed far down the lists: the sets are those entries."""
    _log("case: 1.5M-entry lists")
    rng = np.random.default_rng(15)
    hq, hkv, n, d = 4, 2, 3000, 64
    q, k, v = _inputs(rng, hq, hkv, n, d, "bf16")
    cap = 1_500_000
    raws, cleans = [], []
    for _ in range(2 * hkv):
        raw = rng.integers(n, 2**31 - 1, size=cap, dtype=np.int64)
        raw[rng.choice(cap, cap // 3, replace=False)] *= -1
        good = rng.choice(n, 40, replace=False)
        at = np.concatenate([[cap - 1], rng.choice(np.arange(1_100_000, cap - 1), 39, replace=False)])
        raw[at] = good
        raws.append(raw.astype(np.int32))
        cleans.append(np.sort(good))
    vraw, sraw = np.stack(raws[:hkv]), np.stack(raws[hkv:])
    cnt = np.full(hkv, cap, np.int32)
    out, lse = _run_gpu(q, k, v, vraw, cnt, sraw, cnt)
    vidx, vcnt = _pad_lists(cleans[:hkv])
    soff, scnt = _pad_lists(cleans[hkv:])
    ro, rl = oracle.attn(q, k, v, vidx, vcnt, soff, scnt)
    assert_attn_close(out, lse, ro, rl, "long lists")


def test_clustered_offsets_and_gathered_columns():
    """Slash offsets in a few runs (few active tiles) plus scattered columns,
    most of which no slash tile covers, so the gathered path carries them."""
    _log("case: clustered offsets")
    rng = np.random.default_rng(12)
    hq, hkv, n, d = 8, 2, 8192, 128
    q, k, v = _inputs(rng, hq, hkv, n, d, "bf16")
    vidx, vcnt, soff, scnt = workloads.clustered_offsets(rng, hkv, n, n_runs=3, run_len=40, local=64)
    extra = [np.sort(rng.choice(np.arange(4, n), 300, replace=False)) for _ in range(hkv)]
    vl = [np.union1d(vidx[g, :vcnt[g]], extra[g]) for g in range(hkv)]
    vidx, vcnt = _pad_lists(vl)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ws = torch.empty(vsa.vs_attn_workspace_bytes(hkv, n, vidx.shape[1], soff.shape[1]),
                     dtype=torch.uint8, device="cuda")
    out, lse = vsa.vs_sparse_attn_prefill(qd, kd, vd, to_dev(vidx), to_dev(vcnt), to_dev(soff),
                                          to_dev(scnt), workspace=ws)
    tiles = vsa.vs_attn_tile_counts(ws, hkv, n, vidx.shape[1], soff.shape[1], hq)
    assert tiles[1] > 0, "the gathered path was not exercised"
    bmp = tiles[2] // (hq // hkv)
    causal_tiles = hkv * sum((min((b + 1) * bmp, n) - 1) // tiles[3] + 1 for b in range((n + bmp - 1) // bmp))
    assert tiles[0] < causal_tiles
    out, lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    rows = sample_rows(np.random.default_rng(1), hq, n, 160)
    ro, rl = oracle.attn(q, k, v, vidx, vcnt, soff, scnt, rows=rows)
    assert_attn_close(out[rows[:, 0], rows[:, 1]], lse[rows[:, 0], rows[:, 1]], ro, rl, "clustered")


def test_dense_tile_count_is_causal_tile_count():
    _log("case: tile counts")
    rng = np.random.default_rng(2)
    hq, hkv, n, d = 8, 2, 2048, 64
    q, k, v = _inputs(rng, hq, hkv, n, d, "bf16")
    vidx, vcnt = _pad_lists([np.zeros(0, np.int64)] * hkv)
    soff, scnt = _pad_lists([np.arange(n)] * hkv)
    ws = torch.empty(vsa.vs_attn_workspace_bytes(hkv, n, vidx.shape[1], n), dtype=torch.uint8, device="cuda")
    vsa.vs_sparse_attn_prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(vidx), to_dev(vcnt),
                               to_dev(soff), to_dev(scnt), workspace=ws)
    dense, gath, rows, keys = vsa.vs_attn_tile_counts(ws, hkv, n, vidx.shape[1], n, hq)
    bmp = rows // (hq // hkv)
    expect = hkv * sum((min((b + 1) * bmp, n) - 1) // keys + 1 for b in range((n + bmp - 1) // bmp))
    assert dense == expect and gath == 0


def test_fixed32k_reduced_full_compare():
    """The fixed-budget layer recipe (32/8 heads, d=128, RoPE, 4 sinks + random
    columns, 64 local + random offsets) at n=4096, every element compared."""
    _log("case: fixed32k recipe at n=4096")
    n = 4096
    q, k, v = workloads.attention_inputs("fixed32k", n=n)
    rs = workloads.streams(7)
    lists = workloads.fixed_index_sets(rs["idx"], 8, n, 4, 121, 64, 241)
    out, lse = _run_gpu(q, k, v, *lists)
    ro, rl = oracle.attn(q, k, v, *lists)
    assert_attn_close(out, lse, ro, rl, "fixed32k@4096")


def test_fixed32k_full_size_sampled():
    """n=32768, 32/8 heads, 1000 columns / 2000 offsets per KV head."""
    _log("case: fixed32k full size")
    q, k, v = workloads.attention_inputs("fixed32k")
    lists = workloads.small_index_sets("fixed32k")
    out, lse = _run_gpu(q, k, v, *lists)
    rows = stratified_rows(np.random.default_rng(3), 32, 32768)
    ro, rl = oracle.attn(q, k, v, *lists, rows=rows)
    assert_attn_close(out[rows[:, 0], rows[:, 1]], lse[rows[:, 0], rows[:, 1]], ro, rl, "fixed32k")


SOLID_CASES = [
    # hq, hkv, n, d, dtype, n_runs, run_len, local
    (8, 2, 3000 + 17, 128, "bf16", 3, 300, 500),
    (4, 4, 2048, 64, "bf16", 2, 700, 130),
    (16, 1, 1500, 128, "f32", 1, 1000, 0),
    (8, 8, 4096 + 63, 128, "bf16", 5, 200, 2000),
]


@pytest.mark.parametrize("case", SOLID_CASES, ids=[f"h{c[0]}x{c[1]}-n{c[2]}-d{c[3]}-{c[4]}" for c in SOLID_CASES])
def test_solid_offset_runs_and_visible_columns(case):
    """Gap-free offset runs longer than a tile's 127-offset window make tiles
    whose every pair is selected (they run unmasked), and columns far below
    the diagonal make gathered chunks visible whole (unmasked too); the rest
    of the tiles, at the run edges and the diagonal, stay masked.  Every row
    against the oracle."""
    hq, hkv, n, d, dtype, n_runs, run_len, local = case
    _log(f"case: solid runs {case}")
    rng = np.random.default_rng(n + 31 * run_len)
    q, k, v = _inputs(rng, hq, hkv, n, d, dtype)
    _, _, soff, scnt = workloads.clustered_offsets(rng, hkv, n, n_runs=n_runs, run_len=run_len, local=local)
    cols = [np.union1d(np.arange(4), rng.choice(np.arange(4, n), 200, replace=False)) for _ in range(hkv)]
    vidx, vcnt = _pad_lists(cols)
    out, lse = _run_gpu(q, k, v, vidx, vcnt, soff, scnt)
    ro, rl = oracle.attn(q, k, v, vidx, vcnt, soff, scnt)
    assert_attn_close(out, lse, ro, rl, str(case))


def test_one_million_tokens_sampled():
    """n = 2^20 (1M positions), 4 query heads on 1 KV head, d = 128, bf16:
    64 columns (4 sinks, a run at 2^19 and random ones) and 64 offsets (a local
    band plus random ones up to n - 1), so positions, bitmap words and offsets
    run to their largest values; sampled rows, including the last ones,
    against the oracle.  Then the block path on the same inputs: discovery
    at its 16384-block limit and block attention, rows sampled."""
    n, hq, hkv, d = 1 << 20, 4, 1, 128
    _log("case: 1M tokens")
    rng = np.random.default_rng(2024)
    q = workloads.to_bf16_bits(rng.standard_normal((hq, n, d), dtype=np.float32))
    k = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d), dtype=np.float32))
    v = workloads.to_bf16_bits(rng.standard_normal((hkv, n, d), dtype=np.float32))
    cols = np.unique(np.concatenate([np.arange(4), np.arange(1 << 19, (1 << 19) + 20),
                                     rng.choice(np.arange(4, n), 40, replace=False)]))
    offs = np.unique(np.concatenate([np.arange(16), [n - 1, n - 2, n // 2],
                                     rng.choice(np.arange(16, n), 45, replace=False)]))
    vidx, vcnt = _pad_lists([cols])
    soff, scnt = _pad_lists([offs])
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out, lse = vsa.vs_sparse_attn_prefill(qd, kd, vd, to_dev(vidx), to_dev(vcnt), to_dev(soff), to_dev(scnt))
    torch.cuda.synchronize()
    rows = stratified_rows(np.random.default_rng(5), hq, n)
    ro, rl = oracle.attn(q, k, v, vidx, vcnt, soff, scnt, rows=rows)
    og = to_f64(out)[rows[:, 0], rows[:, 1]]
    lg = lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1]]
    del out, lse
    assert_attn_close(og, lg, ro, rl, "1M vertical-slash")

    _log("case: 1M tokens, block path")
    mask = vsa.vs_block_discover(qd, kd, 8, 0.9)
    out, lse = vsa.vs_block_attn_prefill(qd, kd, vd, mask)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().view(np.uint32)
    nb = n // 64
    assert m.shape == (hkv, nb, oracle.words_per_row(nb))
    diag = (m[0, np.arange(nb), np.arange(nb) // 32] >> (np.arange(nb) % 32)) & 1
    assert diag.all(), "every query block keeps its diagonal block"
    ro, rl = oracle.block_attn(q, k, v, m, rows=rows)
    assert_attn_close(to_f64(out)[rows[:, 0], rows[:, 1]], lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1]],
                      ro, rl, "1M block path")
