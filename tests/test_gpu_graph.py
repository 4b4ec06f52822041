"""The C ABI under HIP graph capture.  No call allocates, synchronises or
records a memset (workspaces are cleared by the library's own kernels), so a
whole layer -- indexer, two selections, sparse attention -- can be captured
once and replayed.  Each replay must reproduce the eager results bit for bit,
with eager work on the same buffers in between."""
import sys

import numpy as np
import pytest
import torch

import vertical_slash_sparse_amd as vsa
import workloads
from tests.util import to_dev

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_layer_graph_replays_match_eager():
    _log("case: graph capture of index + select + attention")
    rng = np.random.default_rng(77)
    hq, hkv, n, d = 16, 4, 4096, 128
    q = to_dev(workloads.to_bf16_bits(rng.standard_normal((hq, n, d))))
    k = to_dev(workloads.to_bf16_bits(rng.standard_normal((hkv, n, d))))
    v = to_dev(workloads.to_bf16_bits(rng.standard_normal((hkv, n, d))))
    w1, w2 = workloads.indexer_weights(rng, 2 * d, 128)
    w1, w2 = to_dev(w1), to_dev(w2)
    cap = 512
    vlog = torch.empty((hkv, n), dtype=torch.float32, device="cuda")
    slog = torch.empty_like(vlog)
    vi = torch.empty((hkv, cap), dtype=torch.int32, device="cuda")
    vc = torch.empty((hkv,), dtype=torch.int32, device="cuda")
    si = torch.empty_like(vi)
    sc = torch.empty_like(vc)
    sws = torch.empty(vsa.vs_select_workspace_bytes(hkv, n), dtype=torch.uint8, device="cuda")
    aws = torch.empty(vsa.vs_attn_workspace_bytes(hkv, n, cap, cap), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")

    def layer():
        vsa.vs_index(k, v, w1, w2, vlog, slog)
        vsa.vs_select(vlog, vsa.VS_VERTICAL, 0.9, cap, vi, vc, sws)
        vsa.vs_select(slog, vsa.VS_SLASH, 0.9, cap, si, sc, sws)
        vsa.vs_sparse_attn_prefill(q, k, v, vi, vc, si, sc, out=out, lse=lse, workspace=aws)

    layer()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (vlog, slog, vi, vc, si, sc, out, lse)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(3):
        for t in (vlog, slog, out, lse):
            t.fill_(float("nan"))
        vi.fill_(-7)
        si.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = (vlog, slog, vi, vc, si, sc, out, lse)
        for a, b, name in zip(got, ref, ("vlog", "slog", "vi", "vc", "si", "sc", "out", "lse")):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
        layer()                      # eager work on the same buffers between replays
        torch.cuda.synchronize()
