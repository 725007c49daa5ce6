"""Edge cases of the register-streamed decode indexer (one or two query rows a wave), through the C ABI (MI355X
only): two-row blocks that straddle two sequences (three queries per sequence), pages of 16, 32, 64 and 128 keys
(pages shorter than a 32-key tile put one tile's keys on several pages), positions on and around the tile
boundaries, sequences shorter than a tile, bf16 and FP8 keys. Every score 0..p of every row is checked against the oracle at the indexer tolerance, and
every entry past p must keep the fill value (the stores past a row's position are dropped, never written)."""

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
import oracle
from workloads import bits_u16, bits_u8

from gpu_cases import DEV, decode_batch, indexer_rel_err, ld_for, say

pytestmark = pytest.mark.gpu

def _check(d, label):
    n_q, max_kv = len(d["q_pos"]), d["max_kv"]
    say(f"[decode indexer] {label}: {d['num_seqs']} sequences, {n_q} rows, max_kv {max_kv}, "
        f"{'fp8' if d['fp8'] else 'bf16'} keys, page {d['page']}")
    b = dsa.Batch(num_seqs=d["num_seqs"], max_kv_len=max_kv, q_seq=torch.from_numpy(d["q_seq"]).to(DEV),
                  q_pos=torch.from_numpy(d["q_pos"]).to(DEV), seq_stride=d["stride"],
                  page_table=None if d["pt"] is None else torch.from_numpy(d["pt"]).to(DEV),
                  page_size=d["page"] or 64)
    ld = ld_for(max_kv) + 4   # room past every row's end that no store may touch
    scores = torch.full((n_q, ld), float("nan"), dtype=torch.float32, device=DEV)
    dsa.indexer_scores(b, d["q_idx"].to(DEV), d["w"].to(DEV), d["k_idx"].to(DEV),
                       None if d["k_scale"] is None else d["k_scale"].to(DEV), scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    k_bits = bits_u8(d["k_idx"]) if d["fp8"] else bits_u16(d["k_idx"])
    ref = oracle.indexer_scores_rows(list(range(n_q)), q_idx=bits_u16(d["q_idx"]), w=d["w"].numpy(), k_idx=k_bits,
                                     k_scale=None if d["k_scale"] is None else d["k_scale"].numpy(),
                                     q_seq=d["q_seq"], q_pos=d["q_pos"], seq_stride=d["stride"], page_table=d["pt"],
                                     page_size=d["page"] or 64)
    worst = 0.0
    for r in range(n_q):
        p = int(d["q_pos"][r])
        worst = max(worst, indexer_rel_err(got[r, : p + 1], ref[r], fp8=d["fp8"]))
        assert np.isnan(got[r, p + 1:]).all(), f"row {r} (p = {p}): an entry past p was written"
    say(f"  worst error / bound {worst:.3f}")
    assert worst <= 1.0


# sequence lengths around the 32-key tiles (and one of 5000), three queries each where they fit: two-row blocks
# then straddle sequences
LENS = [5000, 777, 3001, 64, 33, 32, 31, 2, 1, 97, 4096, 4097]


@pytest.mark.parametrize("fp8,page", [(True, 64), (True, None), (False, None), (False, 32)])
def test_three_rows_a_sequence(fp8, page):
    news = [min(3, L) for L in LENS]
    _check(decode_batch(41, LENS, news, fp8, page), "three rows a sequence")


@pytest.mark.parametrize("page", [16, 32, 128])
def test_page_sizes_one_row(page):
    lens = [9000, 129, 128, 127, 65, 1, 2050]
    _check(decode_batch(43, lens, [1] * len(lens), True, page), f"one row a sequence, pages of {page}")


@pytest.mark.parametrize("fp8,page", [(True, None), (False, 32), (False, None)])
def test_tile_boundaries_one_row(fp8, page):
    lens = [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 4095, 4096, 4097]
    _check(decode_batch(47, lens, [1] * len(lens), fp8, page), "positions around tile boundaries")


def test_two_rows_paged_bf16():
    lens = [20000, 7000, 300, 2]
    _check(decode_batch(53, lens, [2] * len(lens), False, 64), "two rows a sequence, bf16 keys in pages of 64")
