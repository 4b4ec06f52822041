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
from tests.util import assert_attn_close, to_dev, to_f64

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
