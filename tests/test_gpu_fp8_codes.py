"""Every finite E4M3 code through the FP8 indexer, bit for bit, through the C ABI (MI355X only).

Key s holds one E4M3 code in all of its 128 bytes; each query row has a single nonzero entry, +1 or -1, in one
dimension of head 0, and every other head's query is zero. A score is then one exact product,
w * max(0, sigma_s * (+-decode(code_s))), so the kernels' FP8 -> bf16 conversion is compared bit for bit with
the oracle's E4M3 decode for all 254 finite codes, negative ones included (through the -1 query). Scales are
powers of two, so the sigma product is exact too. Covered: one and two queries per sequence, contiguous and
paged (64-token pages in a shuffled order) caches: every FP8 form of the decode indexer.
"""

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
import oracle
from workloads import bits_u16

from gpu_cases import DEV, ld_for, say

pytestmark = pytest.mark.gpu

H_I, D_I, L, PAGE = 64, 128, 256, 64
CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # the 254 finite codes


def _keys():
    """[L, D_I] codes (key s = CODES[s], the last two keys zero) and their powers-of-two scales."""
    codes = np.zeros(L, dtype=np.uint8)
    codes[: CODES.size] = CODES
    k = np.repeat(codes[:, None], D_I, axis=1)
    sigma = np.ldexp(1.0, (np.arange(L) % 5) - 2).astype(np.float32)   # 1/4 .. 4
    return k, sigma


def _queries(signs, dim=5):
    q = torch.zeros((len(signs), H_I, D_I), dtype=torch.float32)
    for r, sg in enumerate(signs):
        q[r, 0, dim] = float(sg)
    return q.to(torch.bfloat16)


def _run(num_seqs, q_seq, q_pos, signs, paged, seed):
    k1, s1 = _keys()
    n_q = len(q_pos)
    if paged:
        pages_per_seq = L // PAGE
        perm = np.random.default_rng(seed).permutation(num_seqs * pages_per_seq).astype(np.int32)
        page_table = perm.reshape(num_seqs, pages_per_seq)
        pool = np.zeros((num_seqs * L, D_I), dtype=np.uint8)
        pool_sigma = np.zeros(num_seqs * L, dtype=np.float32)
        for b in range(num_seqs):
            for s in range(L):
                slot = page_table[b, s // PAGE] * PAGE + s % PAGE
                pool[slot] = k1[s]
                pool_sigma[slot] = s1[s]
        seq_stride = 0
    else:
        page_table = None
        pool = np.tile(k1, (num_seqs, 1))
        pool_sigma = np.tile(s1, num_seqs)
        seq_stride = L
    q = _queries(signs)
    w = torch.ones((n_q, H_I), dtype=torch.float32)
    q_seq_t = torch.tensor(q_seq, dtype=torch.int32)
    q_pos_t = torch.tensor(q_pos, dtype=torch.int32)

    b = dsa.Batch(num_seqs=num_seqs, max_kv_len=L, q_seq=q_seq_t.to(DEV), q_pos=q_pos_t.to(DEV),
                  seq_stride=seq_stride, page_table=None if page_table is None else torch.from_numpy(page_table).to(DEV),
                  page_size=PAGE)
    k_dev = torch.from_numpy(pool).to(DEV).view(torch.float8_e4m3fn)
    scores = torch.full((n_q, ld_for(L)), float("nan"), dtype=torch.float32, device=DEV)
    dsa.indexer_scores(b, q.to(DEV), w.to(DEV), k_dev, torch.from_numpy(pool_sigma).to(DEV), scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()

    ref = oracle.indexer_scores_rows(list(range(n_q)), q_idx=bits_u16(q), w=w.numpy(), k_idx=pool,
                                     k_scale=pool_sigma, q_seq=np.array(q_seq), q_pos=np.array(q_pos),
                                     seq_stride=seq_stride, page_table=page_table, page_size=PAGE)
    nonzero = 0
    for r in range(n_q):
        p = q_pos[r]
        want = ref[r].astype(np.float32)
        assert np.array_equal(want.astype(np.float64), ref[r]), "the expected scores are exact fp32 values"
        bad = np.flatnonzero(got[r, : p + 1].view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (f"row {r} (sign {signs[r]}): {bad.size} scores differ, first at s={bad[0]} "
                               f"(code 0x{int(k1[bad[0], 0]):02x}): gpu {got[r, bad[0]]!r} oracle {want[bad[0]]!r}")
        nonzero += int(np.count_nonzero(want))
    return nonzero


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_fp8_codes_two_queries_per_sequence(paged):
    # one sequence, its last two positions as queries (+1 and -1): the two-rows-per-workgroup decode form
    say(f"[fp8 codes] 1 sequence x 2 queries, paged={paged}")
    nz = _run(1, [0, 0], [L - 2, L - 1], [+1, -1], paged, seed=31)
    say(f"  all {CODES.size} finite codes bit-exact ({nz} nonzero scores)")
    assert nz == CODES.size - 2   # every nonzero code lands on exactly one of the two signs


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_fp8_codes_one_query_per_sequence(paged):
    # two sequences with the same keys, one query each (+1, -1): the one-row-per-workgroup decode form
    say(f"[fp8 codes] 2 sequences x 1 query, paged={paged}")
    nz = _run(2, [0, 1], [L - 1, L - 1], [+1, -1], paged, seed=37)
    say(f"  all {CODES.size} finite codes bit-exact ({nz} nonzero scores)")
    assert nz == CODES.size - 2
