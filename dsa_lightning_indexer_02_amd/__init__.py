"""Python binding of libdsa, the DeepSeek Sparse Attention hot path on AMD MI355X (gfx950).

Three calls mirror the C ABI in include/dsa.h, one per DSA step:
  indexer_scores -- lightning-indexer scores of every causal (query, key) pair
  topk           -- per-row causal top-k (ascending positions, -1 padded; ties to the lower position)
  sparse_attn    -- exact softmax MQA attention over the selected latent rows
and cache_append writes new tokens into the caches (FP8 indexer keys with per-token scales, latent rows).

This module only marshals arguments: torch tensors supply device pointers and the current HIP stream, and
every step runs in libdsa's HIP kernels. There is no fallback: if libdsa.so is missing or fails to load,
every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "DSAError",
    "Batch",
    "lib",
    "lib_path",
    "indexer_scores",
    "topk",
    "topk_workspace_size",
    "topk_noalloc",
    "sparse_attn",
    "sparse_attn_workspace_size",
    "cache_append",
    "block_topk",
    "block_topk_workspace_size",
    "block_cover",
    "indexer_topk",
    "indexer_topk_workspace_size",
    "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libdsa.so"

STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
          4: "DSA_ERR_HIP"}
DSA_BF16, DSA_FP8_E4M3FN = 0, 1


class DSAError(RuntimeError):
    """A non-OK dsa_status, with libdsa's message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class _CBatch(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("seq_stride", ctypes.c_int64),
        ("q_seq", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
    ]


_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """Load libdsa.so (built in-tree by dsa_lightning_indexer_02_amd.build); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise DSAError(4, f"{path} is not built (python -m dsa_lightning_indexer_02_amd.build)")
    L = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    BP = ctypes.POINTER(_CBatch)
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_last_error.argtypes = []
    L.dsa_indexer_scores.restype = ctypes.c_int
    L.dsa_indexer_scores.argtypes = [BP, P, P, P, ctypes.c_int, P, I32, I32, P, I64, P]
    L.dsa_topk_workspace_size.restype = ctypes.c_int
    L.dsa_topk_workspace_size.argtypes = [BP, I32, ctypes.POINTER(SZ)]
    L.dsa_topk.restype = ctypes.c_int
    L.dsa_topk.argtypes = [BP, P, I64, I32, P, P, SZ, P]
    L.dsa_topk_noalloc.restype = ctypes.c_int
    L.dsa_topk_noalloc.argtypes = [BP, P, I64, I32, P, P]
    L.dsa_sparse_attn_workspace_size.restype = ctypes.c_int
    L.dsa_sparse_attn_workspace_size.argtypes = [BP, I32, I32, I32, ctypes.POINTER(SZ)]
    L.dsa_sparse_attn.restype = ctypes.c_int
    L.dsa_sparse_attn.argtypes = [BP, P, P, P, I32, I32, I32, I32, F32, P, P, P, SZ, P]
    L.dsa_cache_append.restype = ctypes.c_int
    L.dsa_cache_append.argtypes = [BP, P, I32, P, I32, P, P, P, P]
    L.dsa_block_topk_workspace_size.restype = ctypes.c_int
    L.dsa_block_topk_workspace_size.argtypes = [BP, I32, I32, ctypes.POINTER(SZ)]
    L.dsa_block_topk.restype = ctypes.c_int
    L.dsa_block_topk.argtypes = [BP, P, I64, I32, I32, P, P, SZ, P]
    L.dsa_indexer_topk_workspace_size.restype = ctypes.c_int
    L.dsa_indexer_topk_workspace_size.argtypes = [BP, I32, I32, I32, ctypes.POINTER(SZ)]
    L.dsa_indexer_topk.restype = ctypes.c_int
    L.dsa_indexer_topk.argtypes = [BP, P, P, P, ctypes.c_int, P, I32, I32, I32, P, P, SZ, P]
    L.dsa_block_cover.restype = ctypes.c_int
    L.dsa_block_cover.argtypes = [BP, P, I32, I32, P, P]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise DSAError(status, lib().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, dim=None):
    if not t.is_cuda:
        raise DSAError(1, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise DSAError(1, f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise DSAError(1, f"{name} has dtype {t.dtype}, expected {dtype}")
    if dim is not None and t.dim() != dim:
        raise DSAError(1, f"{name} must have {dim} dims, got {t.dim()}")


@dataclass
class Batch:
    """Query rows and cache addressing shared by the three calls (see dsa_batch in include/dsa.h).

    q_seq, q_pos: int32 device tensors [num_q]; page_table: int32 device [num_seqs, max_pages] or None.
    """
    num_seqs: int
    max_kv_len: int
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    seq_stride: int = 0
    page_table: Optional[torch.Tensor] = None
    page_size: int = 64

    def __post_init__(self):
        _need(self.q_seq, "q_seq", torch.int32, 1)
        _need(self.q_pos, "q_pos", torch.int32, 1)
        if self.page_table is not None:
            _need(self.page_table, "page_table", torch.int32, 2)
        self._c = _CBatch(
            num_seqs=int(self.num_seqs), num_q=int(self.q_pos.shape[0]), max_kv_len=int(self.max_kv_len),
            page_size=int(self.page_size) if self.page_table is not None else 0,
            max_pages=int(self.page_table.shape[1]) if self.page_table is not None else 0, reserved=0,
            seq_stride=int(self.seq_stride), q_seq=self.q_seq.data_ptr(), q_pos=self.q_pos.data_ptr(),
            page_table=_ptr(self.page_table))

    @property
    def num_q(self) -> int:
        return int(self._c.num_q)

    @property
    def c(self):
        return ctypes.byref(self._c)

    @classmethod
    def from_workload(cls, wl) -> "Batch":
        """Batch of a workloads.Workload whose tensors are already on the device."""
        return cls(num_seqs=wl.num_seqs, max_kv_len=wl.max_kv_len, q_seq=wl.q_seq, q_pos=wl.q_pos,
                   seq_stride=wl.seq_stride, page_table=wl.page_table, page_size=wl.page_size)


def indexer_scores(batch: Batch, q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor,
                   k_scale: Optional[torch.Tensor], scores: torch.Tensor) -> torch.Tensor:
    """Fill scores[r, 0..q_pos[r]] with the indexer scores; returns `scores`."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    _need(k_idx, "k_idx", (torch.bfloat16, torch.float8_e4m3fn), 2)
    _need(scores, "scores", torch.float32, 2)
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.float32, 1)
    kd = DSA_FP8_E4M3FN if k_idx.dtype == torch.float8_e4m3fn else DSA_BF16
    H_I, d_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    _check(lib().dsa_indexer_scores(batch.c, _ptr(q_idx), _ptr(w), _ptr(k_idx), kd, _ptr(k_scale), H_I, d_I,
                                    _ptr(scores), int(scores.stride(0)), _stream()))
    return scores


def topk_workspace_size(batch: Batch, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_topk_workspace_size(batch.c, int(k), ctypes.byref(n)))
    return int(n.value)


def topk(batch: Batch, scores: torch.Tensor, k: int, idx: Optional[torch.Tensor] = None,
         ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k positions per row ([num_q, k] int32, ascending, -1 padded); returns idx."""
    _need(scores, "scores", torch.float32, 2)
    if idx is None:
        idx = torch.empty((batch.num_q, k), dtype=torch.int32, device=scores.device)
    _need(idx, "idx", torch.int32, 2)
    need = topk_workspace_size(batch, k)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_topk(batch.c, _ptr(scores), int(scores.stride(0)), int(k), _ptr(idx), _ptr(ws), nbytes,
                          _stream()))
    return idx


def topk_noalloc(batch: Batch, scores: torch.Tensor, k: int, idx: torch.Tensor) -> torch.Tensor:
    """dsa_topk_noalloc: the same selection as topk, using the library's own scratch array instead of a workspace
    (no allocation in the call; idx must be given). Returns idx."""
    _need(scores, "scores", torch.float32, 2)
    _need(idx, "idx", torch.int32, 2)
    _check(lib().dsa_topk_noalloc(batch.c, _ptr(scores), int(scores.stride(0)), int(k), _ptr(idx), _stream()))
    return idx


def sparse_attn_workspace_size(batch: Batch, k: int, H: int, D_v: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_sparse_attn_workspace_size(batch.c, int(k), int(H), int(D_v), ctypes.byref(n)))
    return int(n.value)


def sparse_attn(batch: Batch, q: torch.Tensor, latent: torch.Tensor, idx: torch.Tensor, sm_scale: float, D_v: int,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None):
    """Sparse MQA attention; returns (out [num_q, H, D_v] bf16, lse [num_q, H] fp32 or None)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(latent, "latent", torch.bfloat16, 2)
    _need(idx, "idx", torch.int32, 2)
    H, D_qk = int(q.shape[1]), int(q.shape[2])
    k = int(idx.shape[1])
    if out is None:
        out = torch.empty((batch.num_q, H, D_v), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    need = sparse_attn_workspace_size(batch, k, H, D_v)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_sparse_attn(batch.c, _ptr(q), _ptr(latent), _ptr(idx), k, H, D_qk, int(D_v), float(sm_scale),
                                 _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream()))
    return out, lse


def cache_append(batch: Batch, k_new: torch.Tensor, latent_new: torch.Tensor, k_pool: torch.Tensor,
                 k_scale: torch.Tensor, latent_pool: torch.Tensor) -> None:
    """Write the batch's rows (tokens at (q_seq, q_pos)) into the caches: FP8 keys + scales and latent rows."""
    _need(k_new, "k_new", torch.float32, 2)
    _need(latent_new, "latent_new", torch.bfloat16, 2)
    _need(k_pool, "k_pool", (torch.float8_e4m3fn, torch.uint8), 2)
    _need(k_scale, "k_scale", torch.float32, 1)
    _need(latent_pool, "latent_pool", torch.bfloat16, 2)
    _check(lib().dsa_cache_append(batch.c, _ptr(k_new), int(k_new.shape[1]), _ptr(latent_new),
                                  int(latent_new.shape[1]), _ptr(k_pool), _ptr(k_scale), _ptr(latent_pool), _stream()))


def block_topk_workspace_size(batch: Batch, block: int, k_blocks: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_block_topk_workspace_size(batch.c, int(block), int(k_blocks), ctypes.byref(n)))
    return int(n.value)


def block_topk(batch: Batch, scores: torch.Tensor, block: int, k_blocks: int, idx: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block selection with the budget k_blocks * block: [num_q, k_blocks * block] int32 positions, ascending, -1 padded."""
    _need(scores, "scores", torch.float32, 2)
    if idx is None:
        idx = torch.empty((batch.num_q, k_blocks * block), dtype=torch.int32, device=scores.device)
    _need(idx, "idx", torch.int32, 2)
    need = block_topk_workspace_size(batch, block, k_blocks)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_block_topk(batch.c, _ptr(scores), int(scores.stride(0)), int(block), int(k_blocks), _ptr(idx),
                                _ptr(ws), nbytes, _stream()))
    return idx


def block_cover(batch: Batch, idx: torch.Tensor, block: int, counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[num_q, 3] int32: useful tokens, distinct blocks touched, tokens read when whole blocks are read."""
    _need(idx, "idx", torch.int32, 2)
    if counts is None:
        counts = torch.empty((batch.num_q, 3), dtype=torch.int32, device=idx.device)
    _need(counts, "counts", torch.int32, 2)
    _check(lib().dsa_block_cover(batch.c, _ptr(idx), int(idx.shape[1]), int(block), _ptr(counts), _stream()))
    return counts


def indexer_topk_workspace_size(batch: Batch, H_I: int, d_I: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_indexer_topk_workspace_size(batch.c, int(H_I), int(d_I), int(k), ctypes.byref(n)))
    return int(n.value)


def indexer_topk(batch: Batch, q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor,
                 k_scale: Optional[torch.Tensor], k: int, idx: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer and top-k fused (scores stay on chip): [num_q, k] int32 positions, ascending, -1 padded."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    _need(k_idx, "k_idx", (torch.bfloat16, torch.float8_e4m3fn), 2)
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.float32, 1)
    kd = DSA_FP8_E4M3FN if k_idx.dtype == torch.float8_e4m3fn else DSA_BF16
    H_I, d_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    if idx is None:
        idx = torch.empty((batch.num_q, k), dtype=torch.int32, device=q_idx.device)
    _need(idx, "idx", torch.int32, 2)
    need = indexer_topk_workspace_size(batch, H_I, d_I, k)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_indexer_topk(batch.c, _ptr(q_idx), _ptr(w), _ptr(k_idx), kd, _ptr(k_scale), H_I, d_I, int(k),
                                  _ptr(idx), _ptr(ws), nbytes, _stream()))
    return idx

