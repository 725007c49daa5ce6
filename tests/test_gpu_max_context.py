"""The largest batch shapes the library accepts, end to end against the oracle (MI355X only): one sequence of
max_kv_len = 2^20 tokens (FP8 indexer keys), its last two positions as queries, k = 4096.

  indexer    every score of both rows (2^20 each) within the FP8 bar
  top-k      fed the oracle's fp32 scores: bit-exact (the windowed form, 128 chunks of 8,192 keys per row)
  attention  given the oracle's 4,096-entry lists: the attention bar (16 splits per row, merged)"""

import math

import numpy as np
import pytest
import torch

from workloads import Workload, fp8_encode_rows

from gpu_cases import say
from test_gpu_parity import _attn_case, _indexer_case, _oracle_idx, _topk_case

pytestmark = pytest.mark.gpu

L_MAX, K_MAX = 1 << 20, 4096


def _normal_bf16(rng, rows, cols, scale, chunk=1 << 16):
    out = torch.empty((rows, cols), dtype=torch.bfloat16)
    for r0 in range(0, rows, chunk):
        n = min(chunk, rows - r0)
        out[r0: r0 + n] = torch.from_numpy(rng.standard_normal((n, cols), dtype=np.float32) * scale).to(torch.bfloat16)
    return out


def _max_context_workload():
    rng = np.random.default_rng(2020)
    H_I, d_I, H, D_qk, D_v = 64, 128, 128, 576, 512
    raw = torch.from_numpy(rng.standard_normal((L_MAX, d_I), dtype=np.float32))
    k_idx, k_scale = fp8_encode_rows(raw)
    del raw
    q_idx = _normal_bf16(rng, 2 * H_I, d_I, 1 / math.sqrt(d_I)).view(2, H_I, d_I)
    w = torch.from_numpy((rng.random((2, H_I), dtype=np.float32) / 8).astype(np.float32))
    q = _normal_bf16(rng, 2 * H, D_qk, 1 / math.sqrt(D_qk)).view(2, H, D_qk)
    latent = _normal_bf16(rng, L_MAX, D_qk, 1 / math.sqrt(D_qk))
    return Workload(name="max_context", n_q=2, num_seqs=1, max_kv_len=L_MAX, H_I=H_I, d_I=d_I, H=H, D_qk=D_qk,
                    D_v=D_v, k=K_MAX, sm_scale=1 / math.sqrt(D_qk), k_dtype="fp8", q_idx=q_idx, w=w, k_idx=k_idx,
                    k_scale=k_scale, q=q, latent=latent, q_seq=torch.zeros(2, dtype=torch.int32),
                    q_pos=torch.tensor([L_MAX - 2, L_MAX - 1], dtype=torch.int32),
                    kv_len=torch.tensor([L_MAX], dtype=torch.int32), page_table=None, page_size=64,
                    seq_stride=L_MAX)


def test_max_context_and_k_end_to_end():
    wl = _max_context_workload()
    say(f"[max context] L={wl.max_kv_len} k={wl.k} rows=2, FP8 keys")
    rows = [0, 1]
    ref = _indexer_case(wl, rows)
    _topk_case(wl, ref, rows, "max context")
    _attn_case(wl, _oracle_idx(ref, wl.k), rows, "max context")
