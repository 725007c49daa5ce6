"""The decode indexer's balanced split when rounding each sequence up to whole chunks would need more workgroups
than the split aims for (MI355X only).

200 one-block sequences and one of 312 blocks (256 keys a block), FP8 keys in 64-token pages, one query per
sequence at its last position: ceil(total / 256) = 2 blocks per chunk would make 200 + 156 chunks, so the split
takes the smallest chunk size that fits (6 blocks: 200 + 52). Every score is checked against the oracle at the
FP8 tolerance; the split decides only which workgroup computes a score, never its value."""

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
import oracle
from workloads import bits_u16, bits_u8, fp8_encode_rows

from gpu_cases import DEV, indexer_rel_err, ld_for, say

pytestmark = pytest.mark.gpu


def test_balanced_split_needs_larger_chunks():
    rng = np.random.default_rng(31)
    lens = [200] * 200 + [312 * 256]
    num_seqs, H_I, d_I, page = len(lens), 64, 128, 64
    n_pages = [(L + page - 1) // page for L in lens]
    perm = rng.permutation(sum(n_pages)).astype(np.int32)
    pt = np.zeros((num_seqs, max(n_pages)), dtype=np.int32)
    off = 0
    for b, npg in enumerate(n_pages):
        pt[b, :npg] = perm[off: off + npg]
        off += npg
    raw = torch.from_numpy(rng.standard_normal((sum(n_pages) * page, d_I)).astype(np.float32))
    k_idx, k_scale = fp8_encode_rows(raw)
    q_idx = torch.from_numpy(rng.standard_normal((num_seqs, H_I, d_I)).astype(np.float32) / np.sqrt(d_I)).to(torch.bfloat16)
    w = torch.from_numpy(rng.random((num_seqs, H_I)).astype(np.float32) / 8)
    q_seq = np.arange(num_seqs, dtype=np.int32)
    q_pos = np.array([L - 1 for L in lens], dtype=np.int32)
    say(f"[indexer split] {num_seqs} sequences, lengths 200 x 200 and {lens[-1]}, FP8 keys in {sum(n_pages)} pages")
    b = dsa.Batch(num_seqs=num_seqs, max_kv_len=max(lens), q_seq=torch.from_numpy(q_seq).to(DEV),
                  q_pos=torch.from_numpy(q_pos).to(DEV), page_table=torch.from_numpy(pt).to(DEV), page_size=page)
    scores = torch.full((num_seqs, ld_for(max(lens))), float("nan"), dtype=torch.float32, device=DEV)
    dsa.indexer_scores(b, q_idx.to(DEV), w.to(DEV), k_idx.to(DEV), k_scale.to(DEV), scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    ref = oracle.indexer_scores_rows(list(range(num_seqs)), q_idx=bits_u16(q_idx), w=w.numpy(), k_idx=bits_u8(k_idx),
                                     k_scale=k_scale.numpy(), q_seq=q_seq, q_pos=q_pos, page_table=pt, page_size=page)
    worst = max(indexer_rel_err(got[r, : q_pos[r] + 1], ref[r], fp8=True) for r in range(num_seqs))
    say(f"  worst error / bound {worst:.3f}")
    assert worst <= 1.0
