"""GPU parity of the per-query-head and packed-batch (varlen) forms of the
vertical-slash prefill against the fp64 oracle, with the attention
tolerance (max-abs 2e-2, mean-abs 2e-3 on O and lse)."""
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


def _inputs(rng, hq, hkv, n, d, dtype):
    q = rng.standard_normal((hq, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    if dtype == "bf16":
        return tuple(workloads.to_bf16_bits(x) for x in (q, k, v))
    return tuple(x.astype(np.float32) for x in (q, k, v))


def _rand_lists(rng, heads, n, nv, ns, cap_v=None, cap_s=None):
    cap_v = cap_v or max(1, nv)
    cap_s = cap_s or max(1, ns)
    vidx = np.full((heads, cap_v), -1, np.int32)
    soff = np.full((heads, cap_s), -1, np.int32)
    vcnt = np.zeros(heads, np.int32)
    scnt = np.zeros(heads, np.int32)
    for h in range(heads):
        cols = np.sort(rng.choice(n, size=min(nv, n), replace=False))
        offs = np.unique(np.concatenate([[0], rng.choice(n, size=min(ns, n), replace=False)]))[:cap_s]
        vidx[h, :len(cols)] = cols
        soff[h, :len(offs)] = offs
        vcnt[h], scnt[h] = len(cols), len(offs)
    return vidx, vcnt, soff, scnt


QH_CASES = [
    # hq, hkv, n, d, dtype, nv, ns
    (4, 1, 300, 64, "bf16", 10, 20),
    (8, 2, 1000, 128, "bf16", 40, 60),
    (16, 2, 777, 128, "fp32", 5, 100),
    (32, 8, 2048, 128, "bf16", 64, 128),
    (16, 1, 513, 64, "bf16", 0, 1),
]


@pytest.mark.parametrize("case", QH_CASES, ids=[f"h{c[0]}x{c[1]}-n{c[2]}-d{c[3]}-{c[4]}" for c in QH_CASES])
def test_per_query_head_sets(case):
    hq, hkv, n, d, dtype, nv, ns = case
    _log(f"case: qh {case}")
    rng = np.random.default_rng(hq * 3 + n)
    q, k, v = _inputs(rng, hq, hkv, n, d, dtype)
    lists = _rand_lists(rng, hq, n, nv, ns)
    out, lse = vsa.vs_sparse_attn_prefill_qh(to_dev(q), to_dev(k), to_dev(v), *[to_dev(x) for x in lists])
    torch.cuda.synchronize()
    ro, rl = oracle.attn_qh(q, k, v, *lists)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"qh {case}")


VARLEN_CASES = [
    # hq, hkv, cu_seqlens, d, dtype, per_query_head
    (4, 1, [0, 100], 64, "bf16", False),
    (8, 2, [0, 300, 300, 1000, 1001], 128, "bf16", False),
    (8, 2, [0, 64, 700, 2000], 128, "bf16", True),
    (16, 2, [0, 1, 2, 3, 500], 64, "fp32", False),
    (32, 8, [0, 1024, 3072], 128, "bf16", True),
    # 40 sequences (empty, one-row and block-edge lengths among them), per query head, fp32, group of 8
    (16, 2, [0] + np.cumsum([0, 1, 63, 64, 65, 127, 128, 129, 0, 300] * 4).tolist(), 64, "fp32", True),
]


@pytest.mark.parametrize("case", VARLEN_CASES,
                         ids=[f"h{c[0]}x{c[1]}-{len(c[2]) - 1}seq-d{c[3]}-{c[4]}-{'qh' if c[5] else 'kv'}"
                              for c in VARLEN_CASES])
def test_varlen(case):
    hq, hkv, cu, d, dtype, per_qh = case
    _log(f"case: varlen {case}")
    rng = np.random.default_rng(sum(cu) + hq)
    total = cu[-1]
    q, k, v = _inputs(rng, hq, hkv, total, d, dtype)
    sets = hq if per_qh else hkv
    per_seq = []
    for s in range(len(cu) - 1):
        ln = max(cu[s + 1] - cu[s], 1)
        per_seq.append(_rand_lists(rng, sets, ln, min(ln, 20), min(ln, 40), cap_v=20, cap_s=41))
    stack = [np.stack([ps[i] for ps in per_seq]) for i in range(4)]
    out, lse = vsa.vs_sparse_attn_prefill_varlen(to_dev(q), to_dev(k), to_dev(v), cu,
                                                 *[to_dev(x) for x in stack], per_query_head=per_qh)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_varlen(q, k, v, cu, *stack, per_query_head=per_qh)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"varlen {case}")


def _zipf_logits(rng, heads, n, s=1.1):
    """Zipf(s) scores over a random permutation of ranks, one row per head."""
    out = np.empty((heads, n), np.float32)
    for h in range(heads):
        out[h] = (-s * np.log(rng.permutation(n) + 1.0)).astype(np.float32)
    return out


def test_per_query_head_sets_32k_sampled():
    """32/8 heads at n = 32768: every query head selects its own columns and
    offsets from its own Zipf scores (mass 0.95, caps 1024 / 2048); sampled
    rows against the oracle."""
    _log("case: qh 32k sampled")
    rng = np.random.default_rng(41)
    hq, hkv, n, d = 32, 8, 32768, 128
    q, k, v = workloads.attention_inputs("fixed32k")
    vi, vc = vsa.vs_select(to_dev(_zipf_logits(rng, hq, n)), vsa.VS_VERTICAL, 0.95, 1024)
    si, sc = vsa.vs_select(to_dev(_zipf_logits(rng, hq, n)), vsa.VS_SLASH, 0.95, 2048)
    out, lse = vsa.vs_sparse_attn_prefill_qh(to_dev(q), to_dev(k), to_dev(v), vi, vc, si, sc)
    torch.cuda.synchronize()
    lists = [t.cpu().numpy() for t in (vi, vc, si, sc)]
    rows = stratified_rows(rng, hq, n)
    ro, rl = oracle.attn_qh(q, k, v, *lists, rows=rows)
    og = to_f64(out)[rows[:, 0], rows[:, 1]]
    lg = lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1]]
    assert_attn_close(og, lg, ro, rl, "qh 32k")


def test_varlen_48k_sampled():
    """Three sequences (8192, 24576, 16384 rows) of the 32/8-head layer, per
    query head sets of 500 columns and 1000 offsets each; sampled rows."""
    _log("case: varlen 48k sampled")
    rng = np.random.default_rng(42)
    hq, hkv, d = 32, 8, 128
    cu = [0, 8192, 8192 + 24576, 8192 + 24576 + 16384]
    total = cu[-1]
    q, k, v = _inputs(rng, hq, hkv, total, d, "bf16")
    per_seq = [_rand_lists(rng, hq, cu[s + 1] - cu[s], 500, 1000, cap_v=500, cap_s=1001)
               for s in range(3)]
    stack = [np.stack([ps[i] for ps in per_seq]) for i in range(4)]
    out, lse = vsa.vs_sparse_attn_prefill_varlen(to_dev(q), to_dev(k), to_dev(v), cu,
                                                 *[to_dev(x) for x in stack], per_query_head=True)
    torch.cuda.synchronize()
    rows = stratified_rows(rng, hq, total)
    extra = np.array([[h, r] for h in (0, hq - 1) for r in (cu[1] - 1, cu[1], cu[2] - 1, cu[2])],
                     np.int32)
    rows = np.concatenate([rows, extra])
    ro, rl = oracle.attn_varlen(q, k, v, cu, *stack, per_query_head=True, rows=rows)
    og = to_f64(out)[rows[:, 0], rows[:, 1]]
    lg = lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1]]
    assert_attn_close(og, lg, ro, rl, "varlen 48k")


def _varlen_lists(rng, cu, sets, nv, ns, cap_v, cap_s, spill=0):
    """Per-sequence random lists stacked to [nseq, sets, cap]; `spill` more
    entries per head point past the sequence's end (the call must drop
    them, as the oracle does)."""
    per_seq = []
    for s in range(len(cu) - 1):
        ln = max(cu[s + 1] - cu[s], 1)
        vi, vc, so, sc = _rand_lists(rng, sets, ln, min(ln, nv), min(ln, ns), cap_v=cap_v, cap_s=cap_s)
        for h in range(sets):
            for arr, cnt, cap in ((vi, vc, cap_v), (so, sc, cap_s)):
                extra = min(spill, cap - cnt[h])
                arr[h, cnt[h]:cnt[h] + extra] = ln + np.sort(rng.choice(3 * ln + 64, size=extra,
                                                                         replace=False))
                cnt[h] += extra
        per_seq.append((vi, vc, so, sc))
    return [np.stack([ps[i] for ps in per_seq]) for i in range(4)]


def test_varlen_many_sequences_and_spilled_indices():
    """70 sequences of 0..400 rows (several empty, several of one row), so the
    sequence table spans more than one table write, with every list also
    holding indices past its sequence's end."""
    _log("case: varlen 70 sequences")
    rng = np.random.default_rng(43)
    hq, hkv, d = 8, 2, 128
    lens = rng.integers(0, 401, size=70)
    lens[[3, 17, 40]] = 0
    lens[[5, 6, 69]] = 1
    lens[10] = 64
    lens[11] = 65
    cu = [0] + np.cumsum(lens).tolist()
    total = cu[-1]
    q, k, v = _inputs(rng, hq, hkv, total, d, "bf16")
    stack = _varlen_lists(rng, cu, hkv, 12, 30, cap_v=20, cap_s=40, spill=5)
    out, lse = vsa.vs_sparse_attn_prefill_varlen(to_dev(q), to_dev(k), to_dev(v), cu,
                                                 *[to_dev(x) for x in stack])
    torch.cuda.synchronize()
    ro, rl = oracle.attn_varlen(q, k, v, cu, *stack)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, "varlen 70 seq")


def test_varlen_workspace_reuse_and_batch_counters():
    """One workspace serves a batch of long, densely selected sequences and
    then a batch of shorter ones: the second result matches the oracle (no
    stale selection survives), and the batch's tile counters equal the sums
    of the counters of single-sequence calls on the same lists."""
    _log("case: varlen workspace reuse")
    rng = np.random.default_rng(44)
    hq, hkv, d, cap_v, cap_s = 8, 2, 128, 64, 200
    cu1 = [0, 3000, 3100, 5000]
    cu2 = [0, 700, 1500, 1501, 2600]
    longest = max(int(np.diff(cu1).max()), int(np.diff(cu2).max()))
    nseq = max(len(cu1), len(cu2)) - 1
    ws = torch.empty(vsa.vs_attn_varlen_workspace_bytes(hkv, nseq, longest, cap_v, cap_s),
                     dtype=torch.uint8, device="cuda")
    for it, (cu, nv, ns) in enumerate(((cu1, 64, 199), (cu2, 10, 25))):
        total = cu[-1]
        q, k, v = _inputs(rng, hq, hkv, total, d, "bf16")
        stack = _varlen_lists(rng, cu, hkv, nv, ns, cap_v=cap_v, cap_s=cap_s)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        out, lse = vsa.vs_sparse_attn_prefill_varlen(qd, kd, vd, cu, *[to_dev(x) for x in stack],
                                                     workspace=ws)
        torch.cuda.synchronize()
        ro, rl = oracle.attn_varlen(q, k, v, cu, *stack)
        assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"varlen reuse {it}")
        ns_ = len(cu) - 1
        got = vsa.vs_attn_tile_counts(ws, ns_ * hkv, int(np.diff(cu).max()), cap_v, cap_s, ns_ * hq)
        want = [0, 0]
        for s in range(ns_):
            a, b = cu[s], cu[s + 1]
            if a == b:
                continue
            sws = torch.empty(vsa.vs_attn_workspace_bytes(hkv, b - a, cap_v, cap_s), dtype=torch.uint8,
                              device="cuda")
            vsa.vs_sparse_attn_prefill(qd[:, a:b].contiguous(), kd[:, a:b].contiguous(),
                                       vd[:, a:b].contiguous(), *[to_dev(x[s]) for x in stack],
                                       workspace=sws)
            c = vsa.vs_attn_tile_counts(sws, hkv, b - a, cap_v, cap_s, hq)
            want[0] += c[0]
            want[1] += c[1]
            assert c[2:] == got[2:]
        assert list(got[:2]) == want, (got, want)
