"""Layout independence, run-to-run determinism and IndexCache at the 4K size, through the C ABI (MI355X only).

  paged = contiguous  the ragged decode batch (FP8 keys, 64-token pages in a seeded random physical order) and the
                      same tokens copied into a contiguous cache give bit-identical scores, top-k lists and
                      attention outputs (the slot map is the only difference; one page table serves both pools)
  determinism         ten runs of the whole 4K prefill step give bit-identical scores, lists, outputs and lse
  IndexCache          one indexer + top-k over the 4K prefill serves the attention of four layers, each with its
                      own queries and latent cache; every layer meets the attention bar on sampled rows against
                      the oracle given the shared index set
"""

import dataclasses

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
from workloads import make

from gpu_cases import DEV, attn_oracle, batch_of, bf16_to_f64, check_attn, ld_for, on_device, run_indexer, say, spread_rows

pytestmark = pytest.mark.gpu


def _contiguous_copy(wl):
    """The paged workload's tokens moved to a contiguous cache: slot(b, s) = b * stride + s."""
    stride = (wl.max_kv_len + 63) // 64 * 64
    pt = wl.page_table.numpy()
    lens = wl.kv_len.numpy()
    src = []
    for b in range(wl.num_seqs):
        s = np.arange(stride)
        s = np.minimum(s, lens[b] - 1)          # slots past the sequence repeat its last token (never read)
        src.append(pt[b, s // wl.page_size].astype(np.int64) * wl.page_size + s % wl.page_size)
    src = torch.from_numpy(np.concatenate(src))
    k_idx = wl.k_idx.view(torch.uint8)[src].view(wl.k_idx.dtype) if wl.k_idx.dtype != torch.bfloat16 else wl.k_idx[src]
    return dataclasses.replace(wl, k_idx=k_idx.contiguous(),
                               k_scale=None if wl.k_scale is None else wl.k_scale[src].contiguous(),
                               latent=wl.latent[src].contiguous(), page_table=None, seq_stride=stride)


def _run_all(wl):
    d = on_device(wl)
    b = batch_of(d)
    scores = run_indexer(d, b, fill=float("nan"))
    n_ws = dsa.topk_workspace_size(b, wl.k)
    ws = torch.empty(max(n_ws, 16), dtype=torch.uint8, device=DEV) if n_ws else None
    idx = dsa.topk(b, scores, wl.k, ws=ws)
    lse = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device=DEV)
    out, _ = dsa.sparse_attn(b, d.q, d.latent, idx, wl.sm_scale, wl.D_v, lse=lse)
    torch.cuda.synchronize()
    return scores.cpu(), idx.cpu(), out.view(torch.int16).cpu(), lse.cpu()


def test_paged_equals_contiguous_ragged_decode():
    wl = make("decode_ragged_paged")
    say(f"[layout] ragged paged decode n_q={wl.n_q} pages={wl.page_table.shape} vs contiguous copy")
    paged = _run_all(wl)
    cont = _run_all(_contiguous_copy(wl))
    q_pos = wl.q_pos.numpy()
    sp, sc = paged[0].numpy(), cont[0].numpy()
    for r in range(wl.n_q):
        p = int(q_pos[r])
        assert np.array_equal(sp[r, : p + 1].view(np.uint32), sc[r, : p + 1].view(np.uint32)), f"scores row {r}"
    for name, x, y in zip(("idx", "out", "lse"), paged[1:], cont[1:]):
        assert torch.equal(x, y), f"{name} differs between the paged and the contiguous layout"
    say("  scores, top-k, out and lse bit-identical")


def test_prefill_4k_deterministic_ten_runs():
    wl = make("prefill_4k")
    say("[determinism] prefill_4k, 10 runs of indexer + top-k + attention")
    first = _run_all(wl)
    for i in range(9):
        again = _run_all(wl)
        for name, x, y in zip(("scores", "idx", "out", "lse"), first, again):
            assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                               y.view(torch.int32) if y.dtype == torch.float32 else y), f"run {i + 2}: {name} differs"
    say("  10 runs bit-identical")


def test_indexcache_four_layers_4k():
    wl = make("prefill_4k")
    d = on_device(wl)
    b = batch_of(d)
    scores = run_indexer(d, b, fill=0.0)
    idx = dsa.topk(b, scores, wl.k)
    torch.cuda.synchronize()
    shared = idx.cpu().numpy()
    rows = spread_rows(wl.n_q, 16, seed=5)
    say(f"[indexcache 4k] 4 layers share one index set; {len(rows)} rows checked per layer")
    g = torch.Generator().manual_seed(22)
    for layer in range(4):
        wl_l = make("prefill_4k", parts=("attn",))
        if layer:
            sd = float(wl.q.float().std())
            wl_l.q = (wl.q.float() + sd * torch.randn(wl.q.shape, generator=g)).to(torch.bfloat16)
            wl_l.latent = (wl.latent.float() + sd * torch.randn(wl.latent.shape, generator=g)).to(torch.bfloat16)
        dl = on_device(wl_l)
        lse = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device=DEV)
        out, _ = dsa.sparse_attn(b, dl.q, dl.latent, idx, wl.sm_scale, wl.D_v, lse=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = attn_oracle(wl_l, rows, {r: shared[r] for r in rows})
        og, lg = bf16_to_f64(out), lse.cpu().numpy()
        check_attn(np.stack([og[r] for r in rows]), np.stack([lg[r] for r in rows]),
                   np.stack([o_ref[r] for r in rows]), np.stack([l_ref[r] for r in rows]), f"indexcache 4k layer {layer}")
        del dl, out, lse
