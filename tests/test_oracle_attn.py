"""Pins of the oracle's sparse MQA attention (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sparse_attn, sparse_attn_rows, topk_select
from workloads import bits_u16, make


def test_golden_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attn_tiny.json")))
    out, lse = sparse_attn(np.array(g["q"]), np.array(g["C"]), math.log(3.0), g["D_v"])
    np.testing.assert_allclose(out, np.array(g["expected_out"]), rtol=1e-14)
    np.testing.assert_allclose(lse, [math.log(4.0), math.log(2430.0)], rtol=1e-14)


def _sdpa_causal(q, C, sm_scale, D_v):
    """Dense causal attention over a prefill from torch's scaled_dot_product_attention (fp64, CPU):
    heads are the batch of one query each... q [L, H, D], C [L, D] -> out [L, H, D_v]."""
    L, H, D = q.shape
    Q = torch.from_numpy(q).permute(1, 0, 2).contiguous()              # [H, L, D]
    K = torch.from_numpy(C).expand(H, L, D).contiguous()                # shared latent (MQA)
    V = torch.from_numpy(C[:, :D_v]).expand(H, L, D_v).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=sm_scale)
    return o.permute(1, 0, 2).numpy()


def _masked_dense_loops(q, C, sm_scale, D_v):
    """Dense causal attention written out with scalar Python loops over a full score matrix: entries above the
    diagonal are masked to -inf before a per-row softmax (max-subtracted exponentials over a plain sum).
    q [L, H, D], C [L, D] -> out [L, H, D_v], lse [L, H]."""
    L, H, D = q.shape
    out = np.zeros((L, H, D_v))
    lse = np.zeros((L, H))
    for h in range(H):
        z = [[-math.inf] * L for _ in range(L)]
        for t in range(L):
            for s in range(L):
                if s <= t:
                    z[t][s] = sm_scale * sum(float(q[t, h, d]) * float(C[s, d]) for d in range(D))
        for t in range(L):
            m = max(z[t])
            e = [math.exp(v - m) if v != -math.inf else 0.0 for v in z[t]]
            tot = sum(e)
            for d in range(D_v):
                out[t, h, d] = sum(e[s] * float(C[s, d]) for s in range(L)) / tot
            lse[t, h] = m + math.log(tot)
    return out, lse


@pytest.mark.parametrize("peaky", [False, True])
def test_k_at_least_context_equals_dense_causal(peaky):
    """With k >= p + 1 for every row, selection keeps every candidate and sparse attention is dense causal
    attention."""
    rng = np.random.default_rng(2)
    L, H, D, Dv = 37, 3, 12, 8
    sc = 1.0 if peaky else 1.0 / math.sqrt(D)
    q = rng.standard_normal((L, H, D)) * sc
    C = rng.standard_normal((L, D)) * sc
    k = L + 3
    ref = _sdpa_causal(q, C, 1.0 / math.sqrt(D), Dv)
    ref_loops, lse_loops = _masked_dense_loops(q, C, 1.0 / math.sqrt(D), Dv)
    np.testing.assert_allclose(ref_loops, ref, rtol=1e-10, atol=1e-12)   # the two dense references agree
    for r in range(L):
        idx = topk_select(rng.standard_normal(r + 1).astype(np.float32), k)   # any scores: all are kept
        sel = idx[idx != -1]
        out, lse = sparse_attn(q[r], C[sel], 1.0 / math.sqrt(D), Dv)
        np.testing.assert_allclose(out, ref[r], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(out, ref_loops[r], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, lse_loops[r], rtol=1e-12)
        # lse against the plain log-sum-exp of the causal row
        z = (q[r] @ C[: r + 1].T) / math.sqrt(D)
        np.testing.assert_allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=1e-12)


def test_rows_sum_to_one():
    """Softmax rows sum to 1: with every value row equal to the same vector c, the output is c."""
    rng = np.random.default_rng(4)
    H, D, Dv, n = 5, 10, 6, 33
    q = rng.standard_normal((H, D)) * 3
    C = rng.standard_normal((n, D))
    c = rng.standard_normal(Dv)
    C[:, :Dv] = c
    out, _ = sparse_attn(q, C, 0.7, Dv)
    np.testing.assert_allclose(out, np.tile(c, (H, 1)), rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(6)
    H, D, Dv = 4, 9, 5
    q = rng.standard_normal((H, D))
    C = rng.standard_normal((1, D))
    out, lse = sparse_attn(q, C, 0.3, Dv)                      # a single row: out = its value
    np.testing.assert_array_equal(out, np.tile(C[0, :Dv], (H, 1)))
    np.testing.assert_allclose(lse, 0.3 * (q @ C[0]), rtol=1e-14)
    C = rng.standard_normal((7, D))
    out, lse = sparse_attn(np.zeros((H, D)), C, 0.3, Dv)       # q = 0: the mean of the values
    np.testing.assert_allclose(out, np.tile(C[:, :Dv].mean(0), (H, 1)), rtol=1e-13)
    np.testing.assert_allclose(lse, np.full(H, math.log(7)), rtol=1e-14)
    out, lse = sparse_attn(q, np.zeros((0, D)), 0.3, Dv)       # nothing selected
    assert (out == 0).all() and np.isneginf(lse).all()


def test_order_padding_and_heads():
    rng = np.random.default_rng(8)
    H, D, Dv, n = 6, 16, 8, 20
    q = rng.standard_normal((H, D))
    C = rng.standard_normal((n, D))
    out, lse = sparse_attn(q, C, 0.25, Dv)
    perm = rng.permutation(n)
    o2, l2 = sparse_attn(q, C[perm], 0.25, Dv)                 # order of the index list is irrelevant
    np.testing.assert_allclose(o2, out, rtol=1e-12)
    np.testing.assert_allclose(l2, lse, rtol=1e-13)
    for h in range(H):                                          # each head equals a one-head run
        oh, lh = sparse_attn(q[h:h + 1], C, 0.25, Dv)
        np.testing.assert_allclose(oh[0], out[h], rtol=1e-13)
        np.testing.assert_allclose(lh[0], lse[h], rtol=1e-14)


def test_rows_wrapper_padding_paged_and_decoding():
    """The batch wrapper skips -1 entries, reads through the page table, and decodes bf16 exactly."""
    rng = np.random.default_rng(9)
    H, D, Dv, ps, L = 2, 8, 4, 4, 16
    q = torch.from_numpy(rng.standard_normal((1, H, D)).astype(np.float32)).to(torch.bfloat16)
    lat = torch.from_numpy(rng.standard_normal((L, D)).astype(np.float32)).to(torch.bfloat16)
    qb, lb = bits_u16(q), bits_u16(lat)
    idx = np.array([[1, 5, 9, 14, -1, -1]])
    o1, l1 = sparse_attn_rows([0], q=qb, latent=lb, idx=idx, q_seq=[0], sm_scale=0.5, D_v=Dv, seq_stride=L)
    order = [2, 0, 3, 1]
    pool = np.zeros_like(lb)
    for lp, phys in enumerate(order):
        pool[phys * ps:(phys + 1) * ps] = lb[lp * ps:(lp + 1) * ps]
    o2, l2 = sparse_attn_rows([0], q=qb, latent=pool, idx=idx, q_seq=[0], sm_scale=0.5, D_v=Dv,
                              page_table=np.array([order]), page_size=ps)
    assert np.array_equal(o1[0], o2[0]) and np.array_equal(l1[0], l2[0])
    qf = q.double().numpy()[0]
    Cf = lat.double().numpy()[[1, 5, 9, 14]]
    o3, l3 = sparse_attn(qf, Cf, 0.5, Dv)
    assert np.array_equal(o1[0], o3) and np.array_equal(l1[0], l3)


def test_workload_generator_shapes_and_determinism():
    """The seeded generator: the tiny prefill draws the same tensors twice, with the stated shapes."""
    a = make("tiny_prefill_256")
    b = make("tiny_prefill_256")
    for f in ("q_idx", "w", "k_idx", "q", "latent"):
        assert torch.equal(getattr(a, f), getattr(b, f))
    assert tuple(a.q_idx.shape) == (256, 4, 32) and tuple(a.k_idx.shape) == (256, 32)
    assert tuple(a.q.shape) == (256, 8, 80) and tuple(a.latent.shape) == (256, 80)
    assert a.k == 32 and abs(a.sm_scale - 1 / math.sqrt(80)) < 1e-15
    assert float(a.w.min()) >= 0 and float(a.w.max()) <= 1


def test_rows_skip_entries_outside_the_causal_range():
    """With q_pos given, entries past the query or negative are ignored: the result equals the list without them,
    and a list with nothing valid gives out = 0, lse = -inf."""
    rng = np.random.default_rng(4)
    L, H, Dqk, Dv = 40, 3, 16, 8
    q = rng.standard_normal((2, H, Dqk)).astype(np.float32)
    lat = rng.standard_normal((L, Dqk)).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lb = torch.from_numpy(lat).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    clean = np.array([[3, 7, 7, 20, -1, -1], [-1, -1, -1, -1, -1, -1]])
    noisy = np.array([[30, 3, -5, 7, 7, 20], [25, 39, -2, -1, 31, 26]])
    kw = dict(q=qb, latent=lb, q_seq=[0, 0], sm_scale=0.25, D_v=Dv, seq_stride=L, q_pos=[20, 24])
    o1, l1 = sparse_attn_rows([0, 1], idx=clean, **kw)
    o2, l2 = sparse_attn_rows([0, 1], idx=noisy, **kw)
    assert np.array_equal(o1[0], o2[0]) and np.array_equal(l1[0], l2[0])
    assert (o2[1] == 0).all() and np.isneginf(l2[1]).all()
