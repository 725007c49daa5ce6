"""Seeded synthetic inputs shaped like the DSA pages' workloads.

Every tensor is drawn in fixed row chunks from numpy PCG64 streams keyed by (seed, tensor id, chunk id),
so any row can be regenerated alone (the oracle checks sampled rows of the 64K prefill without
materialising the whole 9.7 GB query tensor) and the draw does not depend on thread count.

Nothing here computes any part of DSA. The only transformations are scaling of random draws, dtype casts
(bfloat16 rounding, and the FP8 E4M3 per-token encoding that the decode workloads store their indexer keys
in, done with torch's own float8_e4m3fn cast), and index bookkeeping (positions, page tables).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

CHUNK = 4096          # query rows per chunk for row-sampled regeneration bookkeeping
_ELEMS = 1 << 22      # elements per random chunk (rows per chunk = _ELEMS // next_pow2(row elements))

# tensor ids of the random streams
T_QIDX, T_KIDX, T_W, T_Q, T_LATENT, T_NEEDLE, T_KVLEN, T_PAGES = range(8)

FP8_MAX = 448.0       # largest finite OCP E4M3 magnitude


# Workload table. Shapes, distributions and structure follow the five DSA workloads:
#   tiny causal prefill, 4K prefill, 64K prefill with planted needles, batched fp8 decode,
#   ragged paged fp8 decode.
CONFIGS = {
    "tiny_prefill_256": dict(seed=1, kind="prefill", L=256, H_I=4, d_I=32, H=8, D_qk=80, D_v=64, k=32,
                             k_dtype="bf16", unit_scale=True, w_scale=1.0, w_bf16=False),
    "prefill_4k": dict(seed=2, kind="prefill", L=4096, H_I=64, d_I=128, H=128, D_qk=576, D_v=512, k=2048,
                       k_dtype="bf16", unit_scale=False, w_scale=0.125, w_bf16=True),
    "prefill_64k": dict(seed=3, kind="prefill", L=65536, H_I=64, d_I=128, H=128, D_qk=576, D_v=512, k=2048,
                        k_dtype="bf16", unit_scale=False, w_scale=0.125, w_bf16=True,
                        needles_per_block=16, needle_block=4096, needle_gain=4.0),
    "decode_64x32k": dict(seed=4, kind="decode", num_seqs=64, q_per_seq=1, kv_len=32768, H_I=64, d_I=128,
                          H=128, D_qk=576, D_v=512, k=2048, k_dtype="fp8", w_scale=0.125, w_bf16=True),
    "decode_ragged_paged": dict(seed=5, kind="decode", num_seqs=8, q_per_seq=2, kv_min=16384, kv_max=131072,
                                page_size=64, H_I=64, d_I=128, H=128, D_qk=576, D_v=512, k=2048,
                                k_dtype="fp8", w_scale=0.125, w_bf16=True),
}


@dataclass
class Workload:
    """One batch of DSA inputs (torch CPU tensors unless moved) plus its addressing."""
    name: str
    n_q: int
    num_seqs: int
    max_kv_len: int
    H_I: int
    d_I: int
    H: int
    D_qk: int
    D_v: int
    k: int
    sm_scale: float
    k_dtype: str                      # "bf16" | "fp8"
    q_idx: torch.Tensor               # [n_q, H_I, d_I] bf16
    w: torch.Tensor                   # [n_q, H_I] fp32
    k_idx: torch.Tensor               # [slots, d_I] bf16 or float8_e4m3fn
    k_scale: Optional[torch.Tensor]   # [slots] fp32 (fp8 keys) or None
    q: torch.Tensor                   # [n_q, H, D_qk] bf16
    latent: torch.Tensor              # [slots, D_qk] bf16
    q_seq: torch.Tensor               # [n_q] int32
    q_pos: torch.Tensor               # [n_q] int32
    kv_len: torch.Tensor              # [num_seqs] int32
    page_table: Optional[torch.Tensor] = None   # [num_seqs, max_pages] int32
    page_size: int = 64
    seq_stride: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def slots(self) -> int:
        return int(self.latent.shape[0])

    def to(self, device) -> "Workload":
        import dataclasses
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)


# ----------------------------------------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------------------------------------

def _rng(seed: int, tid: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def _rows_per_chunk(row_elems: int) -> int:
    p2 = 1 << max(0, (row_elems - 1).bit_length())
    return max(1, _ELEMS // p2)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw_rows(seed, tid, n_rows, row_shape, kind, scale, rows=None):
    """float32 array [len(rows) or n_rows, *row_shape] of N(0,1)*scale or U(0,1)*scale draws."""
    row_elems = int(np.prod(row_shape)) if row_shape else 1
    rpc = _rows_per_chunk(row_elems)
    sc = np.float32(scale)

    def chunk(c):
        lo, hi = c * rpc, min(n_rows, (c + 1) * rpc)
        g = _rng(seed, tid, c)
        shape = (hi - lo,) + tuple(row_shape)
        a = g.standard_normal(shape, dtype=np.float32) if kind == "normal" else g.random(shape, dtype=np.float32)
        if sc != 1:
            a *= sc
        return a

    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        out = np.empty((len(rows),) + tuple(row_shape), dtype=np.float32)
        for c in np.unique(rows // rpc):
            a = chunk(int(c))
            sel = np.nonzero(rows // rpc == c)[0]
            out[sel] = a[rows[sel] - c * rpc]
        return out
    n_chunks = (n_rows + rpc - 1) // rpc
    out = np.empty((n_rows,) + tuple(row_shape), dtype=np.float32)

    def fill(c):
        out[c * rpc: min(n_rows, (c + 1) * rpc)] = chunk(c)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n_chunks)))
    return out


def _draw_bf16(seed, tid, n_rows, row_shape, scale, rows=None) -> torch.Tensor:
    """N(0,1)*scale rounded once to bfloat16 (torch round-to-nearest-even); chunked to bound host memory."""
    row_elems = int(np.prod(row_shape))
    rpc = _rows_per_chunk(row_elems)
    if rows is not None:
        return torch.from_numpy(_draw_rows(seed, tid, n_rows, row_shape, "normal", scale, rows)).to(torch.bfloat16)
    out = torch.empty((n_rows,) + tuple(row_shape), dtype=torch.bfloat16)
    n_chunks = (n_rows + rpc - 1) // rpc
    sc = np.float32(scale)

    def fill(c):
        lo, hi = c * rpc, min(n_rows, (c + 1) * rpc)
        a = _rng(seed, tid, c).standard_normal((hi - lo,) + tuple(row_shape), dtype=np.float32)
        if sc != 1:
            a *= sc
        out[lo:hi] = torch.from_numpy(a).to(torch.bfloat16)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n_chunks)))
    return out


def fp8_encode_rows(x: torch.Tensor):
    """Per-row FP8 E4M3 encoding used to store decode-workload indexer keys.

    sigma = max|x| / 448 per row (fp32); codes = float8_e4m3fn(x / sigma) via torch's round-to-nearest-even
    cast (clamped to +-448 against fp32 rounding of the quotient). Returns (codes float8_e4m3fn, sigma fp32).
    """
    x = x.float()
    amax = x.abs().amax(dim=-1)
    sigma = (torch.clamp(amax, min=torch.finfo(torch.float32).tiny) / FP8_MAX).float()
    codes = (x / sigma[:, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, sigma


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> numpy uint16 bit patterns (no value change)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_u8(t: torch.Tensor) -> np.ndarray:
    """float8 tensor -> numpy uint8 codes."""
    return t.contiguous().view(torch.uint8).numpy()


# ----------------------------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------------------------

def _w_tensor(cfg, seed, n_q, rows=None):
    w = torch.from_numpy(_draw_rows(seed, T_W, n_q, (cfg["H_I"],), "uniform", cfg["w_scale"], rows))
    if cfg.get("w_bf16"):
        w = w.to(torch.bfloat16).float()
    return w


def _q_scales(cfg, peaky):
    if cfg.get("unit_scale") or peaky:
        return 1.0, 1.0
    return 1.0 / math.sqrt(cfg["d_I"]), 1.0 / math.sqrt(cfg["D_qk"])


def _prefill_keys(cfg, seed, L):
    """Indexer keys of a prefill workload, with planted needles when the workload asks for them."""
    s_idx = 1.0 if cfg.get("unit_scale") else 1.0 / math.sqrt(cfg["d_I"])
    d_I = cfg["d_I"]
    if not cfg.get("needles_per_block"):
        return _draw_bf16(seed, T_KIDX, L, (d_I,), s_idx), None
    raw = _draw_rows(seed, T_KIDX, L, (d_I,), "normal", s_idx)
    u = _rng(seed, T_NEEDLE, 0).standard_normal(d_I)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    blk, per = cfg["needle_block"], cfg["needles_per_block"]
    pos = []
    for bidx in range((L + blk - 1) // blk):
        n_in = min(blk, L - bidx * blk)
        pos.append(bidx * blk + np.sort(_rng(seed, T_NEEDLE, 1 + bidx).choice(n_in, size=min(per, n_in),
                                                                                replace=False)))
    pos = np.concatenate(pos)
    raw[pos] += np.float32(cfg["needle_gain"]) * u[None, :]
    return torch.from_numpy(raw).to(torch.bfloat16), pos


def make(name: str, *, peaky: bool = False, parts=("indexer", "attn"), L: Optional[int] = None) -> Workload:
    """Build the named workload on the host.

    peaky: draw the attention q and latent as N(0,1) instead of N(0,1)/sqrt(D_qk), so the softmax is far
           from uniform (a stricter attention test than the workloads' own scale).
    parts: skip the indexer ("indexer") or attention ("attn") tensors to save time (skipped ones are empty).
    L:     override the prefill length (tests use shorter prefills with the same distributions).
    """
    cfg = dict(CONFIGS[name])
    seed = cfg["seed"]
    H_I, d_I, H, D_qk, D_v = cfg["H_I"], cfg["d_I"], cfg["H"], cfg["D_qk"], cfg["D_v"]
    s_qidx, s_q = _q_scales(cfg, peaky)
    meta = {}

    if cfg["kind"] == "prefill":
        Lq = int(L or cfg["L"])
        num_seqs, n_q, max_kv = 1, Lq, Lq
        q_seq = torch.zeros(n_q, dtype=torch.int32)
        q_pos = torch.arange(n_q, dtype=torch.int32)
        kv_len = torch.tensor([Lq], dtype=torch.int32)
        page_table, seq_stride, page_size = None, Lq, 64
        n_slots = Lq
        k_scale = None
        if "indexer" in parts:
            k_idx, needles = _prefill_keys(cfg, seed, Lq)
            if needles is not None:
                meta["needles"] = needles
        else:
            k_idx = torch.empty((0, d_I), dtype=torch.bfloat16)
    else:
        num_seqs, qps = cfg["num_seqs"], cfg["q_per_seq"]
        if "kv_len" in cfg:
            lens = np.full(num_seqs, cfg["kv_len"], dtype=np.int64)
        else:
            lens = _rng(seed, T_KVLEN, 0).integers(cfg["kv_min"], cfg["kv_max"], size=num_seqs, endpoint=True)
        n_q = num_seqs * qps
        q_seq = torch.arange(num_seqs, dtype=torch.int32).repeat_interleave(qps)
        q_pos = torch.tensor([int(lens[b]) - qps + i for b in range(num_seqs) for i in range(qps)],
                             dtype=torch.int32)
        kv_len = torch.tensor(lens, dtype=torch.int32)
        max_kv = int(lens.max())
        if "page_size" in cfg:
            page_size = cfg["page_size"]
            n_pages = [(int(x) + page_size - 1) // page_size for x in lens]
            total = int(sum(n_pages))
            perm = _rng(seed, T_PAGES, 0).permutation(total)
            max_pages = max(n_pages)
            pt = np.zeros((num_seqs, max_pages), dtype=np.int32)
            off = 0
            for b in range(num_seqs):
                pt[b, : n_pages[b]] = perm[off: off + n_pages[b]]
                off += n_pages[b]
            page_table = torch.from_numpy(pt)
            seq_stride = 0
            n_slots = total * page_size
        else:
            page_table, page_size = None, 64
            seq_stride = int(cfg["kv_len"])
            n_slots = num_seqs * seq_stride
        if "indexer" in parts:
            raw = torch.from_numpy(_draw_rows(seed, T_KIDX, n_slots, (d_I,), "normal", 1.0))
            k_idx, k_scale = fp8_encode_rows(raw)
            del raw
        else:
            k_idx, k_scale = torch.empty((0, d_I), dtype=torch.float8_e4m3fn), torch.empty(0)

    if "indexer" in parts:
        q_idx = _draw_bf16(seed, T_QIDX, n_q, (H_I, d_I), s_qidx)
        w = _w_tensor(cfg, seed, n_q)
    else:
        q_idx = torch.empty((0, H_I, d_I), dtype=torch.bfloat16)
        w = torch.empty((0, H_I))
    if "attn" in parts:
        q = _draw_bf16(seed, T_Q, n_q, (H, D_qk), s_q)
        latent = _draw_bf16(seed, T_LATENT, n_slots, (D_qk,), s_q)
    else:
        q = torch.empty((0, H, D_qk), dtype=torch.bfloat16)
        latent = torch.empty((0, D_qk), dtype=torch.bfloat16)

    return Workload(
        name=name, n_q=n_q, num_seqs=num_seqs, max_kv_len=max_kv, H_I=H_I, d_I=d_I, H=H, D_qk=D_qk, D_v=D_v,
        k=cfg["k"], sm_scale=1.0 / math.sqrt(D_qk), k_dtype=cfg["k_dtype"], q_idx=q_idx, w=w, k_idx=k_idx,
        k_scale=k_scale if cfg["k_dtype"] == "fp8" else None, q=q, latent=latent, q_seq=q_seq, q_pos=q_pos,
        kv_len=kv_len, page_table=page_table, page_size=page_size, seq_stride=seq_stride, meta=meta)


def make_prefill_batch(seqs, *, seed: int = 11, base: str = "prefill_4k") -> Workload:
    """A contiguous multi-sequence prefill batch with `base`'s shapes and distributions.

    seqs: [(kv_len, n_new), ...]; sequence b holds kv_len tokens in slots b*seq_stride .. b*seq_stride+kv_len-1
    (seq_stride = the largest kv_len rounded up to 64), and its n_new queries are its last n_new tokens
    (p = kv_len - n_new + i, a chunked prefill when n_new < kv_len). Rows are ordered by sequence.
    """
    cfg = dict(CONFIGS[base])
    H_I, d_I, H, D_qk, D_v = cfg["H_I"], cfg["d_I"], cfg["H"], cfg["D_qk"], cfg["D_v"]
    s_qidx, s_q = _q_scales(cfg, False)
    lens = [int(kv) for kv, _ in seqs]
    news = [int(nn) for _, nn in seqs]
    assert all(1 <= nn <= kv for kv, nn in zip(lens, news))
    num_seqs, n_q, max_kv = len(seqs), int(sum(news)), max(lens)
    seq_stride = (max_kv + 63) // 64 * 64
    n_slots = num_seqs * seq_stride
    q_seq = torch.tensor([b for b in range(num_seqs) for _ in range(news[b])], dtype=torch.int32)
    q_pos = torch.tensor([lens[b] - news[b] + i for b in range(num_seqs) for i in range(news[b])], dtype=torch.int32)
    k_idx = _draw_bf16(seed, T_KIDX, n_slots, (d_I,), s_qidx)
    q_idx = _draw_bf16(seed, T_QIDX, n_q, (H_I, d_I), s_qidx)
    w = _w_tensor(cfg, seed, n_q)
    q = _draw_bf16(seed, T_Q, n_q, (H, D_qk), s_q)
    latent = _draw_bf16(seed, T_LATENT, n_slots, (D_qk,), s_q)
    return Workload(
        name=f"{base}_batch", n_q=n_q, num_seqs=num_seqs, max_kv_len=max_kv, H_I=H_I, d_I=d_I, H=H, D_qk=D_qk,
        D_v=D_v, k=cfg["k"], sm_scale=1.0 / math.sqrt(D_qk), k_dtype="bf16", q_idx=q_idx, w=w, k_idx=k_idx,
        k_scale=None, q=q, latent=latent, q_seq=q_seq, q_pos=q_pos, kv_len=torch.tensor(lens, dtype=torch.int32),
        page_table=None, page_size=64, seq_stride=seq_stride)


def stratified_rows(n: int, n_even: int = 256, n_rand: int = 256, seed: int = 0) -> np.ndarray:
    """A fixed row sample of a batch of n query rows: n_even evenly spaced rows (both ends included) and n_rand
    seeded uniform rows drawn without replacement from the rest; sorted, int64. For n <= n_even + n_rand it is
    every row. The 64K prefill's oracle timing and its sampled parity check use the same sample."""
    if n <= n_even + n_rand:
        return np.arange(n, dtype=np.int64)
    even = np.unique(np.round(np.linspace(0, n - 1, num=n_even)).astype(np.int64))
    rest = np.setdiff1d(np.arange(n, dtype=np.int64), even)
    rnd = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x5A, n]))).choice(
        rest, size=n_rand, replace=False)
    return np.sort(np.concatenate([even, rnd]))


def regen_rows(name: str, tensor: str, rows, *, peaky: bool = False) -> torch.Tensor:
    """Regenerate selected query rows of `tensor` in {"q_idx", "w", "q"} exactly as make() draws them."""
    cfg = dict(CONFIGS[name])
    seed = cfg["seed"]
    if cfg["kind"] == "prefill":
        n_q = cfg["L"]
    else:
        n_q = cfg["num_seqs"] * cfg["q_per_seq"]
    s_qidx, s_q = _q_scales(cfg, peaky)
    if tensor == "q_idx":
        return _draw_bf16(seed, T_QIDX, n_q, (cfg["H_I"], cfg["d_I"]), s_qidx, rows=rows)
    if tensor == "w":
        return _w_tensor(cfg, seed, n_q, rows=rows)
    if tensor == "q":
        return _draw_bf16(seed, T_Q, n_q, (cfg["H"], cfg["D_qk"]), s_q, rows=rows)
    raise KeyError(tensor)
