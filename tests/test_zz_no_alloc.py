"""vs_sparse_attn_prefill_noalloc, the attention entry point for callers that
cannot allocate (its workspace is the library's static per-GPU array),
against vs_sparse_attn_prefill with a workspace of its own: two calls in a
row on the same GPU, the second with a smaller input and different sets, so
that anything the first call left in the shared array would show.  The two
entry points run the same kernels, so outputs must be bit-identical; the
small case is also checked against the oracle."""
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


def _case(rng, hq, hkv, n, d, pv, ps):
    q, k, v = (workloads.to_bf16_bits(rng.standard_normal(s)) for s in
               ((hq, n, d), (hkv, n, d), (hkv, n, d)))
    vl = [np.nonzero(rng.random(n) < pv)[0] for _ in range(hkv)]
    ol = [np.nonzero(rng.random(n) < ps)[0] for _ in range(hkv)]
    cap_v, cap_s = max(1, max(map(len, vl))), max(1, max(map(len, ol)))
    vidx = np.full((hkv, cap_v), -1, np.int32)
    soff = np.full((hkv, cap_s), -1, np.int32)
    for g in range(hkv):
        vidx[g, :len(vl[g])] = vl[g]
        soff[g, :len(ol[g])] = ol[g]
    vcnt = np.array([len(x) for x in vl], np.int32)
    scnt = np.array([len(x) for x in ol], np.int32)
    return (q, k, v), (vidx, vcnt, soff, scnt)


def test_noalloc_matches_workspace_entry_point_twice():
    rng = np.random.default_rng(99)
    cases = [(32, 8, 5000, 128, 0.03, 0.05), (8, 2, 700, 64, 0.1, 0.02)]
    for i, (hq, hkv, n, d, pv, ps) in enumerate(cases):
        _log(f"case: noalloc call {i}: hq={hq} hkv={hkv} n={n} d={d}")
        (q, k, v), lists = _case(rng, hq, hkv, n, d, pv, ps)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        ld = [to_dev(x) for x in lists]
        ref_out, ref_lse = vsa.vs_sparse_attn_prefill(qd, kd, vd, *ld)
        out = torch.empty_like(qd)
        lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
        vsa.vs_sparse_attn_prefill_noalloc(qd, kd, vd, *ld, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"call {i}: out differs from the workspace entry point"
        assert torch.equal(lse, ref_lse), f"call {i}: lse differs from the workspace entry point"
        if n <= 1000:
            ro, rl = oracle.attn(q, k, v, *lists)
            assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"noalloc call {i}")


def test_noalloc_rejects_shapes_past_the_static_workspace():
    _log("case: noalloc size limit")
    hkv, hq, n, d = 8, 32, 1 << 20, 128
    assert vsa.vs_attn_workspace_bytes(hkv, n, n, n) > vsa.NOALLOC_SCRATCH_BYTES
    q = torch.empty((hq, 1, d), dtype=torch.bfloat16, device="cuda")
    L = vsa.lib()
    p = q.data_ptr()
    st = L.vs_sparse_attn_prefill_noalloc(p, p, p, vsa.VS_BF16, hq, hkv, n, d, 0.088, p, p, n, p, p, n,
                                          p, None, None)
    assert st == vsa.VS_ERR_WORKSPACE
