"""The binding on a side stream: every tensor a wrapper allocates (outputs,
workspaces, the pipeline's logits) must come from the pool of the stream its
kernels run on, so that work on another stream cannot be handed that memory
while they still use it.  vs_prefill runs on a side stream while the current
stream keeps allocating and overwriting memory; every output row is then
compared with the oracle on the GPU's own inputs to each stage."""
import sys

import numpy as np
import pytest
import torch

import oracle
import vertical_slash_sparse_amd as vsa
import workloads
from tests.util import INDEX_ATOL, assert_attn_close, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_prefill_on_side_stream_while_current_stream_allocates():
    _log("case: vs_prefill on a side stream")
    rng = np.random.default_rng(77)
    hq, hkv, n, d = 16, 4, 6000, 128
    tables = workloads.rope_tables(n, d)
    q = workloads.gaussian_heads(rng, hq, n, d, "bf16", tables)
    k = workloads.gaussian_heads(rng, hkv, n, d, "bf16", tables)
    v = workloads.gaussian_heads(rng, hkv, n, d, "bf16", None)
    w1, w2 = workloads.indexer_weights(rng, 2 * d, 128)
    qd, kd, vd, w1d, w2d = (to_dev(x) for x in (q, k, v, w1, w2))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out, lse, (vi, vc, si, sc) = vsa.vs_prefill(qd, kd, vd, w1d, w2d, 0.9, 500, 800, stream=side)
    # while the side stream runs: allocate and overwrite memory on the
    # current stream, sizes around those of the wrapper's temporaries
    ws_bytes = vsa.vs_attn_workspace_bytes(hkv, n, 500, 800)
    sel_bytes = vsa.vs_select_both_workspace_bytes(hkv, n)
    junk = []
    for r in range(40):
        for nbytes in (ws_bytes, sel_bytes, hkv * n * 4):
            t = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            t.fill_(0xA5 + r)
            junk.append(t)
        if r % 4 == 3:
            junk.clear()
    side.synchronize()
    torch.cuda.synchronize()
    gv, gs = vsa.vs_index(kd, vd, w1d, w2d)
    torch.cuda.synchronize()
    rv, rs = oracle.index(k, v, w1, w2)
    assert np.abs(gv.cpu().numpy() - rv).max() <= INDEX_ATOL
    lists = []
    for kind, lg, gi, gc, cap in ((oracle.VERTICAL, gv, vi, vc, 500), (oracle.SLASH, gs, si, sc, 800)):
        ri, rc = oracle.select(lg.cpu().numpy(), kind, 0.9, cap)
        np.testing.assert_array_equal(gc.cpu().numpy(), rc, err_msg=f"kind {kind}: counts")
        np.testing.assert_array_equal(gi.cpu().numpy(), ri, err_msg=f"kind {kind}: indices")
        lists += [ri, rc]
    ro, rl = oracle.attn(q, k, v, *lists)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, "side stream")
