"""Seeded random decode batches through the decode indexer and the fused indexer -> top-k (MI355X only): 1 to 11
sequences of 1 to 20,000 cached tokens with 1 to 3 queries each, bf16 or FP8 keys, contiguous caches or pages of
1 to 256 tokens in a random physical order. For each batch: every score 0..p of a spread of rows against the
oracle at the indexer tolerance, no entry past any row's position written, and the fused call's selection equal
to dsa_topk over dsa_indexer_scores bit for bit (both sum every score in the same order)."""

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
import oracle
from workloads import bits_u16, bits_u8

from gpu_cases import DEV, decode_batch, indexer_rel_err, ld_for, say, spread_rows

pytestmark = pytest.mark.gpu

PAGES = [None, 1, 4, 16, 32, 64, 256]


def _config(case):
    rng = np.random.default_rng(9000 + case)
    num_seqs = int(rng.integers(1, 12))
    lens = rng.integers(1, 20001, size=num_seqs)
    news = [int(min(L, rng.integers(1, 4))) for L in lens]
    fp8 = case % 3 != 2
    page = PAGES[case % len(PAGES)]
    k = int(rng.choice([7, 64, 2048]))
    return [int(L) for L in lens], news, fp8, page, k


@pytest.mark.parametrize("case", range(14))
def test_random_decode_batch(case):
    lens, news, fp8, page, k = _config(case)
    d = decode_batch(700 + case, lens, news, fp8, page)
    n_q, max_kv = len(d["q_pos"]), d["max_kv"]
    say(f"[decode random {case}] {len(lens)} sequences (max {max_kv}), {n_q} rows, {'fp8' if fp8 else 'bf16'} keys, "
        f"page {page}, k {k}")
    b = dsa.Batch(num_seqs=d["num_seqs"], max_kv_len=max_kv, q_seq=torch.from_numpy(d["q_seq"]).to(DEV),
                  q_pos=torch.from_numpy(d["q_pos"]).to(DEV), seq_stride=d["stride"],
                  page_table=None if d["pt"] is None else torch.from_numpy(d["pt"]).to(DEV), page_size=page or 64)
    q_idx, w, k_idx = d["q_idx"].to(DEV), d["w"].to(DEV), d["k_idx"].to(DEV)
    k_scale = None if d["k_scale"] is None else d["k_scale"].to(DEV)
    scores = torch.full((n_q, ld_for(max_kv) + 4), float("nan"), dtype=torch.float32, device=DEV)
    dsa.indexer_scores(b, q_idx, w, k_idx, k_scale, scores)
    unfused = dsa.topk(b, scores, k)
    fused = dsa.indexer_topk(b, q_idx, w, k_idx, k_scale, k)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for r in range(n_q):
        p = int(d["q_pos"][r])
        assert np.isnan(got[r, p + 1:]).all(), f"row {r} (p = {p}): an entry past p was written"
    rows = spread_rows(n_q, 10, seed=case)
    k_bits = bits_u8(d["k_idx"]) if fp8 else bits_u16(d["k_idx"])
    ref = oracle.indexer_scores_rows(rows, q_idx=bits_u16(d["q_idx"]), w=d["w"].numpy(), k_idx=k_bits,
                                     k_scale=None if d["k_scale"] is None else d["k_scale"].numpy(),
                                     q_seq=d["q_seq"], q_pos=d["q_pos"], seq_stride=d["stride"], page_table=d["pt"],
                                     page_size=page or 64)
    worst = max(indexer_rel_err(got[r, : int(d["q_pos"][r]) + 1], ref[r], fp8=fp8) for r in rows)
    same = int((fused.cpu() == unfused.cpu()).all(dim=1).sum())
    say(f"  worst indexer error / bound {worst:.3f}; fused rows identical to the two calls: {same} / {n_q}")
    assert worst <= 1.0
    assert same == n_q
