"""What the split-K form costs in accuracy (MI355X only). A decode batch of few rows splits each row's key list across
workgroups; every split keeps its own softmax output in bf16 and a second pass merges them with fp32 weights, so
the output is rounded to bf16 twice. The same rows, repeated until the batch has 256 rows, take the unsplit form
(one workgroup per row, one rounding). Both are compared with the oracle on the 64 x 32K decode batch with the
peaky draw (N(0,1) queries and latent, a softmax far from uniform), given the oracle's index lists.

Measured and gated: the split error relative to the output scale stays within the attention bar, and within a
small multiple of the unsplit error (at most one extra bf16 rounding, 2^-9 of the value)."""

import dataclasses

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
from workloads import make

from gpu_cases import DEV, attn_oracle, bf16_to_f64, say

pytestmark = pytest.mark.gpu


def _run(wl, idx):
    d = wl.to(DEV)
    b = dsa.Batch.from_workload(d)
    splits_ws = dsa.sparse_attn_workspace_size(b, wl.k, wl.H, wl.D_v)
    lse = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device=DEV)
    out, _ = dsa.sparse_attn(b, d.q, d.latent, torch.from_numpy(idx.astype(np.int32)).to(DEV), wl.sm_scale, wl.D_v,
                             lse=lse)
    torch.cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().numpy(), splits_ws


def test_split_partials_error():
    wl = make("decode_64x32k", peaky=True, parts=("attn",))
    rng = np.random.default_rng(31)
    rows = list(range(wl.n_q))
    idx = np.stack([np.sort(rng.choice(int(wl.q_pos[r]) + 1, wl.k, replace=False)) for r in rows])
    o_ref, l_ref = attn_oracle(wl, rows, {r: idx[r] for r in rows})
    ref = np.stack([o_ref[r] for r in rows])
    scale = float(np.abs(ref).max())

    out_s, lse_s, ws_s = _run(wl, idx)
    rep = 4   # 256 rows: one workgroup per row
    big = dataclasses.replace(wl, n_q=wl.n_q * rep, q=wl.q.repeat_interleave(rep, 0),
                              q_seq=wl.q_seq.repeat_interleave(rep), q_pos=wl.q_pos.repeat_interleave(rep))
    out_u, lse_u, ws_u = _run(big, np.repeat(idx, rep, axis=0))
    assert ws_s > 0 and ws_u == 0, "the few-row batch must split and the repeated one must not"
    err_s = float(np.abs(out_s - ref).max()) / scale
    err_u = float(np.abs(out_u[::rep] - ref).max()) / scale
    lerr_s = float(np.abs(lse_s - np.stack([l_ref[r] for r in rows])).max())
    say(f"[split precision] 64 x 32K peaky, k={wl.k}: max|d|/max|ref| split {err_s:.3e} (bf16 partials), "
        f"unsplit {err_u:.3e}; lse split {lerr_s:.2e}")
    assert err_s <= 2e-2 and lerr_s <= 1e-3
    assert err_s <= err_u + 2.0 ** -8, "the split form adds at most one bf16 rounding"
