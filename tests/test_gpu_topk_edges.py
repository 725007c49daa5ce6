"""dsa_topk edge cases against the oracle, bit-exact (MI355X only): ties, signed zeros, negatives, huge dynamic
range, all-equal rows, rows of length k-1 / k / k+1, both the one-pass and the chunked two-pass forms."""

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa
import oracle

from gpu_cases import DEV, ld_for, say

pytestmark = pytest.mark.gpu


def _run(scores: np.ndarray, pos: np.ndarray, k: int, label: str, pad: int = 0, shift: int = 0):
    """pad / shift: the rows are ld + pad wide and the tensor starts `shift` floats into its buffer, so rows need
    not be 16-byte aligned."""
    n_q, ld = scores.shape
    max_kv = int(pos.max()) + 1
    b = dsa.Batch(num_seqs=1, max_kv_len=max_kv, q_seq=torch.zeros(n_q, dtype=torch.int32, device=DEV),
                  q_pos=torch.from_numpy(pos.astype(np.int32)).to(DEV), seq_stride=max_kv)
    say(f"[topk-edge] {label}: n_q={n_q} max_kv={max_kv} k={k} pad={pad} shift={shift} "
        f"ws={dsa.topk_workspace_size(b, k)}")
    dev = torch.from_numpy(scores).to(DEV)
    if pad or shift:
        flat = torch.zeros(shift + n_q * (ld + pad), dtype=torch.float32, device=DEV)
        view = flat[shift:].view(n_q, ld + pad)
        view[:, :ld] = dev
        dev = view
    idx = dsa.topk(b, dev, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(n_q):
        exp = oracle.topk_select(scores[r, : pos[r] + 1], k)
        assert np.array_equal(got[r], exp), f"{label}: row {r} (p={pos[r]})"


def _mk(n_q, max_kv, gen, rng):
    ld = ld_for(max_kv)
    s = np.zeros((n_q, ld), dtype=np.float32)
    for r in range(n_q):
        s[r] = gen(ld, rng)
    return s


TIES = np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 2.0, 1e-30, -3e38], dtype=np.float32)


@pytest.mark.parametrize("k", [1, 7, 32, 2048, 4096])
def test_ties_and_signed_zeros_one_pass(k):
    rng = np.random.default_rng(k)
    n_q, max_kv = 600, 6000
    s = _mk(n_q, max_kv, lambda n, g: TIES[g.integers(0, len(TIES), n)], rng)
    pos = rng.integers(0, max_kv, n_q)
    pos[:4] = [k - 2 if k > 1 else 0, k - 1, k, max_kv - 1]
    _run(s, pos, k, f"ties k={k}")


def test_dynamic_range_and_equal_rows():
    rng = np.random.default_rng(7)
    n_q, max_kv = 520, 9000

    def gen(n, g):
        mode = g.integers(0, 3)
        if mode == 0:
            return np.full(n, 0.25, dtype=np.float32)                         # every score equal
        if mode == 1:
            e = g.uniform(-120, 120, n)
            return (np.sign(g.standard_normal(n)) * 2.0 ** e).astype(np.float32)
        return g.standard_normal(n).astype(np.float32)

    s = _mk(n_q, max_kv, gen, rng)
    pos = rng.integers(2000, max_kv, n_q)
    _run(s, pos, 2048, "dynamic range")


@pytest.mark.parametrize("n_q,max_kv", [(64, 32768), (16, 131072), (3, 70000), (40, 5000), (300, 65536),
                                        (256, 131072)])
def test_chunked_two_pass(n_q, max_kv):
    rng = np.random.default_rng(n_q)
    s = _mk(n_q, max_kv, lambda n, g: np.abs(g.standard_normal(n)).astype(np.float32) * 0.1, rng)
    # quantise some rows so chunk boundaries see ties
    s[::3] = np.round(s[::3] * 64) / 64
    pos = rng.integers(max_kv // 2, max_kv, n_q)
    pos[0] = max_kv - 1
    _run(s, pos, 2048, f"chunked {n_q}x{max_kv}")


def test_short_rows_keep_everything():
    n_q = 300
    pos = np.arange(n_q) % 50
    s = np.random.default_rng(0).standard_normal((n_q, ld_for(64))).astype(np.float32)
    _run(s, pos, 64, "short rows")


# Batches of >= 512 rows with rows of >= 8192 go through the streaming form (a sampled window, then an exact
# search inside it; a streaming bucket select when the window misses).

@pytest.mark.parametrize("k", [1, 7, 2048, 4096])
def test_stream_ties_and_signed_zeros(k):
    rng = np.random.default_rng(100 + k)
    n_q, max_kv = 520, 12000
    s = _mk(n_q, max_kv, lambda n, g: TIES[g.integers(0, len(TIES), n)], rng)
    pos = rng.integers(8192, max_kv, n_q)
    pos[:3] = [k - 1, k, max_kv - 1]
    _run(s, pos, k, f"stream ties k={k}")


def test_stream_gaussian_long_rows():
    rng = np.random.default_rng(11)
    n_q, max_kv = 520, 40000
    s = _mk(n_q, max_kv, lambda n, g: (0.14 + 0.03 * g.standard_normal(n)).astype(np.float32), rng)
    pos = rng.integers(8192, max_kv, n_q)
    pos[0] = max_kv - 1
    _run(s, pos, 2048, "stream gaussian")


def test_stream_segment_and_batch_boundaries():
    """The streaming form's pass over the row: each of the 4 waves walks a segment of ceil(n / 4) positions rounded
    up to 256, in steps of 1,024 positions (four 16-byte loads a lane), loads clamped to the segment's last
    aligned position. Row lengths whose segments end exactly on a step, one past it, one short of it, and whose
    last wave's segment is a few positions long or empty must come out exact."""
    rng = np.random.default_rng(21)
    n_q, max_kv = 520, 20000
    s = _mk(n_q, max_kv, lambda n, g: g.standard_normal(n).astype(np.float32), rng)
    lengths = [8192, 8193, 8191, 12288, 12289, 12287, 16384, 16385, 16383, 9216, 9217, 10240, 11264, 8448, 8449,
               12292, 12291, 16388, 19968, 19999, 20000, 2049, 2305, 2306, 3073, 3075, 4097]
    pos = rng.integers(8192, max_kv, n_q)
    for i, n in enumerate(lengths):
        pos[i] = n - 1
    _run(s, pos, 2048, "stream segment/batch boundaries")


def test_stream_window_miss_falls_back():
    # the sample reads 64 runs of 64 keys starting at floor(b * (n - 64) / 63); put the k + 100 largest keys
    # elsewhere, so every sampled key is 0 and the window cannot hold the k-th key
    k, n_q, n = 2048, 512, 20480
    starts = (np.arange(64, dtype=np.int64) * (n - 64)) // 63
    sampled = np.unique((starts[:, None] + np.arange(64)[None, :]).ravel())
    free = np.setdiff1d(np.arange(n), sampled)
    rng = np.random.default_rng(5)
    s = np.zeros((n_q, ld_for(n)), dtype=np.float32)
    for r in range(n_q):
        big = rng.choice(free, k + 100, replace=False)
        s[r, big] = 1.0 + rng.permutation(k + 100).astype(np.float32) / 4096.0
    pos = np.full(n_q, n - 1)
    _run(s, pos, k, "stream window miss")


@pytest.mark.parametrize("k", [1, 100, 2048, 4096])
def test_few_rows_adversarial_patterns(k):
    """Few long rows (the chunked form): large scores on a regular stride of positions only, or everywhere but
    there, all-equal rows, heavy ties and rows just above k must come out exact."""
    n_q, max_kv = 6, 32768
    rng = np.random.default_rng(k)
    s = _mk(n_q, max_kv, lambda n, g: g.standard_normal(n).astype(np.float32), rng)
    pos = np.full(n_q, max_kv - 1)
    S = 2048
    sampled = (np.arange(S) * max_kv) // S
    s[0, sampled] += 100.0                      # large scores on a stride of 16 positions
    mask = np.ones(max_kv, bool)
    mask[sampled] = False
    s[1, : max_kv][mask] += 100.0              # large scores everywhere but on that stride
    s[2] = 0.5                                 # all equal: every key reaches the threshold
    s[3] = np.round(s[3] * 2) / 2              # a handful of distinct values, heavy ties
    pos[4] = k + 1 if k + 1 < max_kv else max_kv - 1   # just above k
    pos[5] = 3000
    _run(s, pos, k, f"sample-miss k={k}")


def test_few_rows_window_miss_with_region_overflow():
    """The chunked form when the sampled window misses and a chunk overflows one wave's LDS region: the first
    1024 positions (one region of the first 4096-key chunk) all hold the largest keys, the sampled runs hold
    values in [0.5, 1) and every other position 0. The sample then puts the window's bottom above all but a few
    hundred of the row's keys, so fewer than k keys reach it; the overflowing chunk writes its own top-k, whose
    lower part lies below the window, and the selection must not take those over the other chunks' keys."""
    k, n_q, n = 2048, 8, 32768
    starts = (np.arange(64, dtype=np.int64) * (n - 64)) // 63
    sampled = np.unique((starts[:, None] + np.arange(64)[None, :]).ravel())
    rng = np.random.default_rng(77)
    s = np.zeros((n_q, ld_for(n)), dtype=np.float32)
    for r in range(n_q):
        s[r, sampled] = (0.5 + 0.5 * rng.random(len(sampled))).astype(np.float32)
        s[r, :1024] = (2.0 + rng.permutation(1024) / 4096.0).astype(np.float32)
    pos = np.full(n_q, n - 1)
    pos[1] = n - 7
    _run(s, pos, k, "window miss + region overflow")


def test_few_rows_up_to_128k():
    rng = np.random.default_rng(9)
    n_q, max_kv = 5, 1 << 17
    s = _mk(n_q, max_kv, lambda n, g: g.standard_normal(n).astype(np.float32), rng)
    pos = np.array([max_kv - 1, 2047, 2048, 70000, 100000])
    _run(s, pos, 2048, "few rows up to 128K")


@pytest.mark.parametrize("pad,shift", [(1, 0), (2, 0), (3, 4)])
def test_stream_rows_not_16_byte_aligned(pad, shift):
    """The streaming form reads 16 bytes per lane when every row is 16-byte aligned and 4 bytes otherwise (a row
    stride that is not a multiple of 4 floats; the library requires the scores to start 16-byte aligned): both
    must give the same exact result."""
    rng = np.random.default_rng(40 + pad + shift)
    n_q, max_kv = 520, 11000
    s = _mk(n_q, max_kv, lambda n, g: TIES[g.integers(0, len(TIES), n)], rng)
    s[::2] = rng.standard_normal((n_q // 2, s.shape[1])).astype(np.float32)
    pos = rng.integers(8192, max_kv, n_q)
    pos[:2] = [8191, max_kv - 1]
    _run(s, pos, 2048, f"stream unaligned pad={pad} shift={shift}", pad=pad, shift=shift)
