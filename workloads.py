"""Seeded synthetic inputs for vertical-slash sparse prefill.

This module only draws inputs: Gaussian Q/K/V with rotary position embedding
applied the way a backbone would emit them, index sets, score vectors and
indexer weights.  It contains none of the method's own arithmetic (no
attention, no indexer, no selection), so both the HIP path and the oracle can
be fed from it without sharing any of their computation.

Every array comes from ``numpy.random.Generator(PCG64(...))`` children of one
``SeedSequence``, so a (workload, seed) pair fixes every value.  bf16 arrays
are returned as raw ``uint16`` bit patterns (round-to-nearest-even from the
fp64/fp32 value); fp32 arrays as ``float32``.

Workloads (shapes follow LLaMA-3.1-8B attention: 32 query heads, 8 KV heads,
head dim 128, one of the backbones the VSPrefill pages evaluate on):

* ``small``   1 head, n=1024, d=64, fp32, fixed 16 verticals / 16 slashes
* ``fixed32k`` 32/8 heads, n=32768, bf16, RoPE, fixed 1000 verticals / 2000 slashes
* ``zipf128k`` 32/8 heads, n=131072, bf16, RoPE, Zipf(1.1) score vectors,
  selection at mass 0.95 capped at 4096 verticals / 8192 slashes
* ``clustered128k`` the zipf128k layer with the Zipf ranks ordered by distance
  to a few centres (position / offset 0 plus uniform draws) instead of
  randomly, so the selected columns and offsets come out as contiguous runs,
  the shape the pages' real heads show; a supplementary workload, not one of
  the pages' configurations
* ``qh32k`` the 32/8-head layer at n=32768 with one index set per query
  head: Zipf(1.1) vertical and slash scores per query head over random
  permutations, mass 0.95, caps 1024 / 2048
* ``varlen64k`` a packed batch of 16 sequences of 32/8 heads (lengths
  uniform in [1024, 8192]), per KV head and sequence 4 sink columns plus 3 %
  random columns and offsets 0..63 plus 6 % random offsets
* ``indexer128k`` 8 KV heads, n=131072, [RoPE(K) | V] 256-wide bf16 rows and
  random indexer weights W1 ~ N(0, 1/256), W2 ~ N(0, 1/128)
* ``e2e256k`` 32/8 heads, n=262144, bf16, RoPE, keys of the first 4 positions
  scaled by 4 (attention sinks), indexer -> selection at 0.95 uncapped
* ``blocks128k`` 32/8 heads, n=131072, bf16, no RoPE, planted block structure
  for the FlashPrefill block path: every 64-key block carries one of 32 unit
  topic directions (amplitude 8), every query block looks for the topic of a
  uniformly drawn earlier block (amplitude 8), and block 0 carries a sink
  direction shared by all queries (amplitude 8 on both sides)
"""
from __future__ import annotations

import numpy as np

ROPE_BASE = 500000.0

# name -> (seed, shape/recipe)
WORKLOADS = {
    "small": dict(seed=1001, hq=1, hkv=1, n=1024, d=64, dtype="f32",
                  rope=False, nv_fixed=4, nv_rand=12, ns_fixed=8, ns_rand=8),
    "fixed32k": dict(seed=1002, hq=32, hkv=8, n=32768, d=128, dtype="bf16",
                     rope=True, nv_fixed=4, nv_rand=996, ns_fixed=64, ns_rand=1936),
    "zipf128k": dict(seed=1003, hq=32, hkv=8, n=131072, d=128, dtype="bf16",
                     rope=True, zipf_s=1.1, mass=0.95, cap_v=4096, cap_s=8192),
    "clustered128k": dict(seed=1007, hq=32, hkv=8, n=131072, d=128, dtype="bf16",
                          rope=True, zipf_s=1.1, mass=0.95, cap_v=4096, cap_s=8192,
                          v_centers=8, s_centers=4),
    "qh32k": dict(seed=1008, hq=32, hkv=8, n=32768, d=128, dtype="bf16", rope=True,
                  zipf_s=1.1, mass=0.95, cap_v=1024, cap_s=2048),
    "varlen64k": dict(seed=1009, hq=32, hkv=8, d=128, dtype="bf16", rope=True, nseq=16,
                      len_lo=1024, len_hi=8192, nv_fixed=4, v_frac=0.03, ns_fixed=64, s_frac=0.06),
    "indexer128k": dict(seed=1004, hkv=8, n=131072, d=128, hidden=128, dtype="bf16",
                        rope=True, mass=0.95),
    "e2e256k": dict(seed=1005, hq=32, hkv=8, n=262144, d=128, hidden=128, dtype="bf16",
                    rope=True, sink=4, sink_scale=4.0, mass=0.95),
    "blocks128k": dict(seed=1006, hq=32, hkv=8, n=131072, d=128, dtype="bf16", rope=False,
                       block=64, topics=32, topic_amp=8.0, sink_amp=8.0, alpha=0.1, skel=8),
}

_STREAMS = ("q", "k", "v", "idx", "w", "score")


def streams(seed: int) -> dict:
    """Independent child generators, one per input kind."""
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(_STREAMS, children)}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32/fp64 values to bf16 (nearest, ties to even), once; return
    uint16 bits.  fp64 input passes through fp32 rounded to odd (truncate,
    then set the last bit when inexact), which keeps the final rounding to
    bf16 correct because fp32 carries more than two extra bits."""
    x = np.asarray(x)
    if x.dtype == np.float64:
        f = x.astype(np.float32)
        back = f.astype(np.float64)
        w = f.view(np.uint32)
        w = np.where(np.abs(back) > np.abs(x), w - np.uint32(1), w)  # toward zero
        w = np.where(back != x, w | np.uint32(1), w)
        f = w.astype(np.uint32).view(np.float32)
    f = np.ascontiguousarray(f if x.dtype == np.float64 else x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rope_tables(n: int, d: int, base: float = ROPE_BASE):
    """cos/sin tables [n, d/2] in fp64, rotate-half pairing (m, m + d/2)."""
    half = d // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x [n, d] -> rotated [n, d] in fp64 (the backbone's position embedding)."""
    half = x.shape[1] // 2
    x = x.astype(np.float64)
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=1)


def gaussian_heads(rng, heads: int, n: int, d: int, dtype: str, tables=None,
                   scale_rows: int = 0, row_scale: float = 1.0) -> np.ndarray:
    """[heads, n, d] N(0,1) draws, optionally rotated, optionally with the first
    ``scale_rows`` rows multiplied by ``row_scale`` after rotation; returned as
    bf16 bits or fp32."""
    out = np.empty((heads, n, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for h in range(heads):
        x = rng.standard_normal((n, d), dtype=np.float32)
        if tables is not None:
            x = _apply_rope(x, *tables)
        if scale_rows:
            x = x.astype(np.float64)
            x[:scale_rows] *= row_scale
        out[h] = to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)
    return out


def attention_inputs(name: str, n: int | None = None, seed: int | None = None):
    """Q [hq,n,d], K [hkv,n,d], V [hkv,n,d] for a workload (optionally at a
    smaller n for quick checks; the draw recipe is unchanged)."""
    w = WORKLOADS[name]
    n = n or w["n"]
    rs = streams(w["seed"] if seed is None else seed)
    tables = rope_tables(n, w["d"]) if w.get("rope") else None
    q = gaussian_heads(rs["q"], w["hq"], n, w["d"], w["dtype"], tables)
    k = gaussian_heads(rs["k"], w["hkv"], n, w["d"], w["dtype"], tables,
                       scale_rows=w.get("sink", 0), row_scale=w.get("sink_scale", 1.0))
    v = gaussian_heads(rs["v"], w["hkv"], n, w["d"], w["dtype"], None)
    return q, k, v


def _draw_distinct(rng, lo: int, hi: int, count: int) -> np.ndarray:
    """``count`` distinct integers uniform in [lo, hi), ascending."""
    count = min(count, max(hi - lo, 0))
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(hi - lo, size=count, replace=False).astype(np.int64) + lo)


def fixed_index_sets(rng, hkv: int, n: int, nv_fixed: int, nv_rand: int,
                     ns_fixed: int, ns_rand: int, s_rand_hi: int | None = None):
    """Per KV head: verticals {0..nv_fixed-1} plus nv_rand distinct random
    columns from [nv_fixed, n); slash offsets {0..ns_fixed-1} plus ns_rand
    distinct random offsets from [ns_fixed, s_rand_hi).  Returned as padded
    ascending int32 lists with counts."""
    s_rand_hi = n if s_rand_hi is None else s_rand_hi
    cap_v = min(n, nv_fixed + nv_rand)
    cap_s = min(n, ns_fixed + ns_rand)
    vidx = np.full((hkv, cap_v), -1, dtype=np.int32)
    soff = np.full((hkv, cap_s), -1, dtype=np.int32)
    vcnt = np.zeros(hkv, dtype=np.int32)
    scnt = np.zeros(hkv, dtype=np.int32)
    for g in range(hkv):
        cols = np.concatenate([np.arange(min(nv_fixed, n)), _draw_distinct(rng, nv_fixed, n, nv_rand)])
        offs = np.concatenate([np.arange(min(ns_fixed, n)), _draw_distinct(rng, ns_fixed, s_rand_hi, ns_rand)])
        vidx[g, :len(cols)] = cols
        soff[g, :len(offs)] = offs
        vcnt[g], scnt[g] = len(cols), len(offs)
    return vidx, vcnt, soff, scnt


def small_index_sets(name: str = "small", n: int | None = None, seed: int | None = None):
    """Index sets of the ``small`` / ``fixed32k`` workloads."""
    w = WORKLOADS[name]
    n = n or w["n"]
    rs = streams(w["seed"] if seed is None else seed)
    hi = (n - 1) if name == "small" else n  # small: random offsets in [8, n-1]
    return fixed_index_sets(rs["idx"], w["hkv"], n, w["nv_fixed"], w["nv_rand"],
                            w["ns_fixed"], w["ns_rand"], s_rand_hi=hi)


def zipf_logits(rng, heads: int, n: int, s: float) -> np.ndarray:
    """Per head, logits -s*ln(rank) with ranks 1..n in random order, so that
    softmax over the vector is exactly the Zipf(s) pmf; fp32 [heads, n]."""
    out = np.empty((heads, n), dtype=np.float32)
    for h in range(heads):
        ranks = rng.permutation(n).astype(np.float64) + 1.0
        out[h] = (-s * np.log(ranks)).astype(np.float32)
    return out


def zipf_scores(name: str = "zipf128k", n: int | None = None, seed: int | None = None):
    """Vertical and slash score vectors [hkv, n] fp32 of the Zipf workload."""
    w = WORKLOADS[name]
    n = n or w["n"]
    rs = streams(w["seed"] if seed is None else seed)
    vlog = zipf_logits(rs["score"], w["hkv"], n, w["zipf_s"])
    slog = zipf_logits(rs["score"], w["hkv"], n, w["zipf_s"])
    return vlog, slog


def banded_zipf_logits(rng, heads: int, n: int, s: float, centers: int) -> np.ndarray:
    """Per head, Zipf(s) logits -s*ln(rank) whose ranks grow with the distance
    of the index to the nearest of ``centers`` centres (index 0 plus uniform
    draws), equal distances in random order; fp32 [heads, n]."""
    out = np.empty((heads, n), dtype=np.float32)
    idx = np.arange(n, dtype=np.int64)
    for h in range(heads):
        c = np.concatenate([[0], rng.choice(np.arange(1, n), size=centers - 1, replace=False)])
        dist = np.abs(idx[:, None] - c[None, :]).min(axis=1)
        order = np.lexsort((rng.random(n), dist))
        ranks = np.empty(n, dtype=np.float64)
        ranks[order] = np.arange(1, n + 1, dtype=np.float64)
        out[h] = (-s * np.log(ranks)).astype(np.float32)
    return out


def clustered_scores(name: str = "clustered128k", n: int | None = None, seed: int | None = None):
    """Vertical and slash score vectors [hkv, n] fp32 of the clustered workload.
    The slash vector is position-indexed like the indexer's output (offset o
    scores at position n-1-o), so the banded ranks are drawn over offsets and
    reversed."""
    w = WORKLOADS[name]
    n = n or w["n"]
    rs = streams(w["seed"] if seed is None else seed)
    vlog = banded_zipf_logits(rs["score"], w["hkv"], n, w["zipf_s"], w["v_centers"])
    by_offset = banded_zipf_logits(rs["score"], w["hkv"], n, w["zipf_s"], w["s_centers"])
    return vlog, np.ascontiguousarray(by_offset[:, ::-1])


def qh_scores(name: str = "qh32k"):
    """Vertical and slash score vectors [hq, n] fp32, one pair per query head."""
    w = WORKLOADS[name]
    rs = streams(w["seed"])
    return (zipf_logits(rs["score"], w["hq"], w["n"], w["zipf_s"]),
            zipf_logits(rs["score"], w["hq"], w["n"], w["zipf_s"]))


def varlen_batch(name: str = "varlen64k"):
    """cu_seqlens (nseq + 1 ints), Q [hq, total, d], K, V [hkv, total, d] (bf16
    bits, RoPE restarting at each sequence) and per-sequence index lists
    stacked as [nseq, hkv, cap] with counts [nseq, hkv]."""
    w = WORKLOADS[name]
    rs = streams(w["seed"])
    lens = rs["idx"].integers(w["len_lo"], w["len_hi"] + 1, size=w["nseq"])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total, d = int(cu[-1]), w["d"]
    q = np.empty((w["hq"], total, d), np.uint16)
    k = np.empty((w["hkv"], total, d), np.uint16)
    v = np.empty((w["hkv"], total, d), np.uint16)
    per = []
    for s, n in enumerate(lens.tolist()):
        tables = rope_tables(n, d)
        a, b = int(cu[s]), int(cu[s + 1])
        q[:, a:b] = gaussian_heads(rs["q"], w["hq"], n, d, "bf16", tables)
        k[:, a:b] = gaussian_heads(rs["k"], w["hkv"], n, d, "bf16", tables)
        v[:, a:b] = gaussian_heads(rs["v"], w["hkv"], n, d, "bf16", None)
        per.append(fixed_index_sets(rs["idx"], w["hkv"], n, w["nv_fixed"], int(w["v_frac"] * n),
                                    w["ns_fixed"], int(w["s_frac"] * n)))
    cap_v = max(p[0].shape[1] for p in per)
    cap_s = max(p[2].shape[1] for p in per)
    vidx = np.full((w["nseq"], w["hkv"], cap_v), -1, np.int32)
    soff = np.full((w["nseq"], w["hkv"], cap_s), -1, np.int32)
    vcnt = np.zeros((w["nseq"], w["hkv"]), np.int32)
    scnt = np.zeros((w["nseq"], w["hkv"]), np.int32)
    for s, (vi, vc, si, sc) in enumerate(per):
        vidx[s, :, :vi.shape[1]] = vi
        soff[s, :, :si.shape[1]] = si
        vcnt[s], scnt[s] = vc, sc
    return cu, q, k, v, (vidx, vcnt, soff, scnt)


def indexer_weights(rng, d_in: int, hidden: int):
    """W1 [hidden, d_in] ~ N(0, 1/d_in), W2 [2, hidden] ~ N(0, 1/hidden), bf16 bits."""
    w1 = rng.standard_normal((hidden, d_in)) / np.sqrt(d_in)
    w2 = rng.standard_normal((2, hidden)) / np.sqrt(hidden)
    return to_bf16_bits(w1), to_bf16_bits(w2)


def indexer_inputs(name: str = "indexer128k", n: int | None = None, seed: int | None = None):
    """K_rope [hkv,n,d], V [hkv,n,d] (bf16 bits) and the indexer weights."""
    w = WORKLOADS[name]
    n = n or w["n"]
    rs = streams(w["seed"] if seed is None else seed)
    tables = rope_tables(n, w["d"])
    k = gaussian_heads(rs["k"], w["hkv"], n, w["d"], "bf16", tables,
                       scale_rows=w.get("sink", 0), row_scale=w.get("sink_scale", 1.0))
    v = gaussian_heads(rs["v"], w["hkv"], n, w["d"], "bf16", None)
    w1, w2 = indexer_weights(rs["w"], 2 * w["d"], w["hidden"])
    return k, v, w1, w2


def random_index_sets(rng, hkv: int, n: int, p_v: float, p_s: float):
    """Bernoulli(p) verticals and offsets per KV head (for edge-case tests)."""
    cap = n
    vidx = np.full((hkv, cap), -1, dtype=np.int32)
    soff = np.full((hkv, cap), -1, dtype=np.int32)
    vcnt = np.zeros(hkv, dtype=np.int32)
    scnt = np.zeros(hkv, dtype=np.int32)
    for g in range(hkv):
        cols = np.nonzero(rng.random(n) < p_v)[0]
        offs = np.nonzero(rng.random(n) < p_s)[0]
        vidx[g, :len(cols)] = cols
        soff[g, :len(offs)] = offs
        vcnt[g], scnt[g] = len(cols), len(offs)
    return vidx, vcnt, soff, scnt


def clustered_offsets(rng, hkv: int, n: int, n_runs: int, run_len: int, local: int):
    """Slash offsets in a few contiguous runs plus a local band (the shape real
    attention heads show); no verticals besides 4 sink columns."""
    vidx = np.tile(np.arange(4, dtype=np.int32), (hkv, 1))
    vcnt = np.full(hkv, 4, dtype=np.int32)
    lists = []
    for _ in range(hkv):
        starts = rng.choice(max(n - run_len - local, 1), size=n_runs, replace=False) + local
        offs = set(range(local))
        for s0 in starts:
            offs.update(range(int(s0), int(s0) + run_len))
        lists.append(np.array(sorted(o for o in offs if o < n), dtype=np.int32))
    cap = max(len(x) for x in lists)
    soff = np.full((hkv, cap), -1, dtype=np.int32)
    scnt = np.zeros(hkv, dtype=np.int32)
    for g, x in enumerate(lists):
        soff[g, :len(x)] = x
        scnt[g] = len(x)
    return vidx, vcnt, soff, scnt


def block_structured_inputs(name: str = "blocks128k", n: int | None = None,
                            seed: int | None = None):
    """Q [hq,n,d], K, V [hkv,n,d] with a planted block pattern (see the module
    docstring): per KV head, unit topic directions u_t; key block J adds
    topic_amp * u_{t(J)} to its keys, query block I adds topic_amp * u_{t(J')}
    for a uniformly drawn J' < I; block 0's keys and every query add
    sink_amp * w.  Gaussian N(0,1) elsewhere; bf16 bits."""
    w = WORKLOADS[name]
    n = n or w["n"]
    rs = streams(w["seed"] if seed is None else seed)
    hq, hkv, d, bs = w["hq"], w["hkv"], w["d"], w["block"]
    group = hq // hkv
    nb = (n + bs - 1) // bs
    q = np.empty((hq, n, d), np.uint16)
    k = np.empty((hkv, n, d), np.uint16)
    v = gaussian_heads(rs["v"], hkv, n, d, "bf16", None)
    for g in range(hkv):
        dirs = rs["idx"].standard_normal((w["topics"] + 1, d))
        dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
        topic_k = rs["idx"].integers(0, w["topics"], nb)
        look = np.zeros(nb, np.int64)
        for I in range(1, nb):
            look[I] = topic_k[rs["idx"].integers(0, I)]
        blk = np.arange(n) // bs
        kk = rs["k"].standard_normal((n, d), dtype=np.float32).astype(np.float64)
        kk += w["topic_amp"] * dirs[topic_k[blk]]
        kk[:min(bs, n)] += w["sink_amp"] * dirs[-1]
        k[g] = to_bf16_bits(kk)
        for hh in range(group):
            qq = rs["q"].standard_normal((n, d), dtype=np.float32).astype(np.float64)
            qq += w["topic_amp"] * dirs[look[blk]]
            qq += w["sink_amp"] * dirs[-1]
            q[g * group + hh] = to_bf16_bits(qq)
    return q, k, v
