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


def _replay_matches(layer, outs, names, poison):
    """Capture `layer`, then replay it three times, poisoning the outputs
    before each replay and running other eager work between replays."""
    layer()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(3):
        poison()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(outs, ref, names):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
        yield rep


def test_varlen_graph_replays_match_eager():
    """A packed batch writes its sequence table into the workspace with
    kernels whose arguments carry the values, so a captured call replays
    correctly even after an eager call of another batch on the same workspace."""
    _log("case: graph capture of a packed batch")
    rng = np.random.default_rng(78)
    hq, hkv, d, cap = 8, 2, 128, 64
    cu = [0, 700, 701, 2300, 2300, 3000]
    cu2 = [0, 3000]                      # the other batch, same rows
    total, nseq = cu[-1], len(cu) - 1
    q = to_dev(workloads.to_bf16_bits(rng.standard_normal((hq, total, d))))
    k = to_dev(workloads.to_bf16_bits(rng.standard_normal((hkv, total, d))))
    v = to_dev(workloads.to_bf16_bits(rng.standard_normal((hkv, total, d))))

    def lists(m):
        """[m, hkv, cap] ascending distinct positions below 700 (-1 padded) and counts."""
        out = []
        for _ in range(2):
            a = np.full((m, hkv, cap), -1, np.int32)
            for s_ in range(m):
                for h in range(hkv):
                    x = np.unique(rng.integers(0, 700, size=cap))
                    a[s_, h, :len(x)] = x
            out += [to_dev(a), to_dev((a >= 0).sum(-1).astype(np.int32))]
        return out

    L1, L2 = lists(nseq), lists(1)
    ws = torch.empty(vsa.vs_attn_varlen_workspace_bytes(hkv, nseq, 3000, cap, cap), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((hq, total), dtype=torch.float32, device="cuda")
    out2, lse2 = torch.empty_like(q), torch.empty_like(lse)

    def layer():
        vsa.vs_sparse_attn_prefill_varlen(q, k, v, cu, *L1, out=out, lse=lse, workspace=ws)

    def poison():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))

    for _ in _replay_matches(layer, (out, lse), ("out", "lse"), poison):
        # another batch through the same workspace between replays
        vsa.vs_sparse_attn_prefill_varlen(q, k, v, cu2, *L2, out=out2, lse=lse2, workspace=ws)
        torch.cuda.synchronize()


def test_block_path_graph_replays_match_eager():
    """FlashPrefill discovery (whose threshold pass reads back the scores it
    stored in the workspace) and the block attention, captured together."""
    _log("case: graph capture of block discovery + block attention")
    q, k, v = (to_dev(x) for x in workloads.block_structured_inputs("blocks128k", n=4096))
    hq, n, d = q.shape
    hkv = k.shape[0]
    nb = n // vsa.BLOCK
    mask = torch.empty((hkv, nb, vsa.block_words_per_row(n)), dtype=torch.int32, device="cuda")
    dws = torch.empty(vsa.vs_block_workspace_bytes(hkv, n, d), dtype=torch.uint8, device="cuda")
    aws = torch.empty(int(vsa.lib().vs_block_attn_workspace_bytes()), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")

    def layer():
        vsa.vs_block_discover(q, k, 8, 0.1, mask=mask, workspace=dws)
        vsa.vs_block_attn_prefill(q, k, v, mask, out=out, lse=lse, workspace=aws)

    def poison():
        mask.fill_(-1)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))

    for _ in _replay_matches(layer, (mask, out, lse), ("mask", "out", "lse"), poison):
        layer()
        torch.cuda.synchronize()
