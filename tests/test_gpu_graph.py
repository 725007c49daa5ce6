"""The decode step captured in one HIP graph (MI355X only). With every buffer allocated beforehand,
dsa_indexer_scores, dsa_topk (caller workspace, or the no-allocation form) and dsa_sparse_attn launch kernels only
(no allocation, copy or fill), so a serving loop can capture them. The graph is replayed several times, with the
program's own eager work (every output overwritten) and a synchronization between replays, and every replay must
reproduce the eager results bit for bit: scores, indices, outputs and lse."""

import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
from workloads import make

from gpu_cases import DEV, ld_for, say

pytestmark = pytest.mark.gpu


def _step(wl, b, bufs, noalloc):
    scores, idx, out, lse, tk_ws, at_ws = bufs
    dsa.indexer_scores(b, wl.q_idx, wl.w, wl.k_idx, wl.k_scale, scores)
    if noalloc:
        dsa.topk_noalloc(b, scores, wl.k, idx)
    else:
        dsa.topk(b, scores, wl.k, idx=idx, ws=tk_ws)
    dsa.sparse_attn(b, wl.q, wl.latent, idx, wl.sm_scale, wl.D_v, out=out, lse=lse, ws=at_ws)


def _scrub(bufs):
    scores, idx, out, lse, _, _ = bufs
    scores.fill_(float("nan"))
    idx.fill_(-7)
    out.fill_(0)
    lse.fill_(0)


@pytest.mark.parametrize("name,noalloc", [("decode_ragged_paged", False), ("decode_64x32k", False),
                                          ("decode_64x32k", True)])
def test_decode_step_graph_replays(name, noalloc):
    wl = make(name).to(DEV)
    b = dsa.Batch.from_workload(wl)
    n_q, k = wl.n_q, wl.k
    say(f"[graph] {name}: n_q={n_q} max_kv={wl.max_kv_len} top-k {'no-allocation form' if noalloc else 'workspace'}")
    bufs = (torch.empty((n_q, ld_for(wl.max_kv_len)), dtype=torch.float32, device=DEV),
            torch.empty((n_q, k), dtype=torch.int32, device=DEV),
            torch.empty((n_q, wl.H, wl.D_v), dtype=torch.bfloat16, device=DEV),
            torch.empty((n_q, wl.H), dtype=torch.float32, device=DEV),
            torch.empty(max(16, dsa.topk_workspace_size(b, k)), dtype=torch.uint8, device=DEV),
            torch.empty(max(16, dsa.sparse_attn_workspace_size(b, k, wl.H, wl.D_v)), dtype=torch.uint8, device=DEV))
    _scrub(bufs)
    _step(wl, b, bufs, noalloc)
    torch.cuda.synchronize()
    ref = [t.clone() for t in bufs[:4]]
    # one run on a side stream before the capture, as torch asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(wl, b, bufs, noalloc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(wl, b, bufs, noalloc)
    torch.cuda.synchronize()
    for rep in range(4):
        _scrub(bufs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        scores, idx, out, lse = bufs[:4]
        assert torch.equal(idx, ref[1]), f"replay {rep}: indices differ from the eager run"
        assert torch.equal(out.view(torch.int16), ref[2].view(torch.int16)), f"replay {rep}: outputs differ"
        assert torch.equal(lse.view(torch.int32), ref[3].view(torch.int32)), f"replay {rep}: lse differs"
        same_nan = torch.equal(torch.isnan(scores), torch.isnan(ref[0]))
        assert same_nan and torch.equal(torch.nan_to_num(scores), torch.nan_to_num(ref[0])), \
            f"replay {rep}: scores differ"
    say("  4 replays bit-identical to the eager step")
