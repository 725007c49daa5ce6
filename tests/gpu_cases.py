"""Shared helpers of the GPU parity tests: run the HIP path through the binding, the oracle on the same seeded
inputs, and compare (not collected by pytest itself)."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import dsa_lightning_indexer_02_amd as dsa
import oracle
from workloads import bits_u16, bits_u8, fp8_encode_rows

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ld_for(max_kv: int) -> int:
    return (max_kv + 3) // 4 * 4


def on_device(wl):
    return wl.to(DEV)


def batch_of(wl_dev):
    return dsa.Batch.from_workload(wl_dev)


def oracle_kwargs(wl):
    """Addressing arguments of the oracle's row wrappers for a host workload."""
    return dict(q_seq=wl.q_seq.numpy(), seq_stride=wl.seq_stride,
                page_table=None if wl.page_table is None else wl.page_table.numpy(), page_size=wl.page_size)


def oracle_scores(wl, rows):
    """{row: float64 scores over 0..p} from the oracle (host workload)."""
    fp8 = wl.k_dtype == "fp8"
    kw = oracle_kwargs(wl)
    return oracle.indexer_scores_rows(
        rows, q_idx=bits_u16(wl.q_idx), w=wl.w.numpy(), k_idx=bits_u8(wl.k_idx) if fp8 else bits_u16(wl.k_idx),
        k_scale=wl.k_scale.numpy() if fp8 else None, q_pos=wl.q_pos.numpy(), **kw)


def indexer_rel_err(got, ref, fp8=False):
    """Worst ratio |gpu - oracle| / bound with bound = tol * max(|ref|, 1e-3 * max|ref_row|) (<= 1 passes)."""
    tol = 5e-2 if fp8 else 1e-2
    floor = 1e-3 * max(float(np.abs(ref).max()), 1e-30)
    bound = tol * np.maximum(np.abs(ref), floor)
    err = np.abs(got.astype(np.float64) - ref) / bound
    if not np.isfinite(err).all():   # an unwritten (NaN-filled) or non-finite score fails outright
        return float("inf")
    return float(err.max())


def run_indexer(wl_dev, b, fill=float("nan")):
    scores = torch.full((wl_dev.n_q, ld_for(wl_dev.max_kv_len)), fill, dtype=torch.float32, device=DEV)
    dsa.indexer_scores(b, wl_dev.q_idx, wl_dev.w, wl_dev.k_idx, wl_dev.k_scale, scores)
    return scores


def check_attn(out_gpu, lse_gpu, out_ref, lse_ref, label=""):
    """The 2e-2 max-abs bar, plus a scale-aware gate: max|diff| <= 2e-2 * max|ref| and lse within 1e-3."""
    d = np.abs(out_gpu.astype(np.float64) - out_ref)
    scale = float(np.abs(out_ref).max())
    dl = float(np.abs(lse_gpu.astype(np.float64) - lse_ref).max())
    say(f"  attn {label}: max|d|={d.max():.3e} max|ref|={scale:.3e} rel={d.max() / max(scale, 1e-30):.3e} "
        f"lse max|d|={dl:.3e}")
    assert d.max() <= 2e-2
    assert d.max() <= 2e-2 * scale
    assert dl <= 1e-3


def attn_oracle(wl, rows, idx_rows):
    """Oracle attention of `rows` given their index lists (host workload)."""
    kw = oracle_kwargs(wl)
    idx = {r: np.asarray(idx_rows[r], dtype=np.int64) for r in rows}   # the oracle reads idx[r] per row only
    return oracle.sparse_attn_rows(rows, q=bits_u16(wl.q), latent=bits_u16(wl.latent), idx=idx,
                                   sm_scale=wl.sm_scale, D_v=wl.D_v, **kw)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def spread_rows(n, count, seed=0):
    """A row sample: both ends, evenly spaced rows and seeded random rows."""
    rng = np.random.default_rng(seed)
    ev = np.linspace(0, n - 1, num=min(n, count // 2)).astype(int)
    rnd = rng.choice(n, size=min(n, count // 2), replace=False)
    return sorted(set(ev.tolist()) | set(rnd.tolist()) | {0, n - 1})


def log(msg):
    say(msg)


def decode_batch(seed, lens, news, fp8, page, H_I=64, D_I=128):
    """A seeded decode-style batch as host arrays and tensors: lens[b] cached tokens per sequence, the last
    news[b] of them queries; page = None for a contiguous cache, else pages of that many tokens in a seeded
    random physical order; FP8 keys (raw N(0,1), per-token scale) or bf16 keys N(0,1)/sqrt(d_I)."""
    rng = np.random.default_rng(seed)
    num_seqs, max_kv = len(lens), max(lens)
    q_seq = np.array([b for b in range(num_seqs) for _ in range(news[b])], dtype=np.int32)
    q_pos = np.array([lens[b] - news[b] + i for b in range(num_seqs) for i in range(news[b])], dtype=np.int32)
    n_q = len(q_pos)
    if page is None:
        stride = (max_kv + 63) // 64 * 64
        slots, pt = num_seqs * stride, None
    else:
        stride = 0
        n_pages = [(L + page - 1) // page for L in lens]
        perm = rng.permutation(sum(n_pages)).astype(np.int32)
        pt = np.zeros((num_seqs, max(n_pages)), dtype=np.int32)
        off = 0
        for b, npg in enumerate(n_pages):
            pt[b, :npg] = perm[off: off + npg]
            off += npg
        slots = sum(n_pages) * page
    raw = rng.standard_normal((slots, D_I)).astype(np.float32)
    if fp8:
        k_idx, k_scale = fp8_encode_rows(torch.from_numpy(raw))
    else:
        k_idx, k_scale = torch.from_numpy(raw / np.sqrt(D_I)).to(torch.bfloat16), None
    q_idx = torch.from_numpy(rng.standard_normal((n_q, H_I, D_I)).astype(np.float32) / np.sqrt(D_I)).to(torch.bfloat16)
    w = torch.from_numpy(rng.random((n_q, H_I)).astype(np.float32) / 8)
    return dict(num_seqs=num_seqs, max_kv=max_kv, q_seq=q_seq, q_pos=q_pos, stride=stride, pt=pt, page=page,
                k_idx=k_idx, k_scale=k_scale, q_idx=q_idx, w=w, fp8=fp8)


__all__ = ["say", "ld_for", "on_device", "batch_of", "oracle_scores", "indexer_rel_err", "run_indexer",
           "check_attn", "attn_oracle", "bf16_to_f64", "spread_rows", "decode_batch", "math"]
