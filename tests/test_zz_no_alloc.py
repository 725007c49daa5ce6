"""dsa_topk_noalloc (the top-k for callers that cannot allocate) against dsa_topk, through the C ABI (MI355X only).

Two calls in a row on one GPU share the library's scratch array: a 64 x 32768 decode-shaped batch (the chunked plan,
which uses the array), then a smaller 16-row batch of ragged lengths up to 20000; each must give exactly dsa_topk's
indices (bit-exact, the bar for index work). A batch whose plan needs more scratch than the library holds is
refused on the host with DSA_ERR_UNSUPPORTED.
"""

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_02_amd as dsa

from gpu_cases import DEV, ld_for, say

pytestmark = pytest.mark.gpu


def _batch(pos, max_kv):
    n = len(pos)
    return dsa.Batch(num_seqs=n, max_kv_len=max_kv, q_seq=torch.arange(n, dtype=torch.int32, device=DEV),
                     q_pos=torch.as_tensor(np.asarray(pos, dtype=np.int32), device=DEV), seq_stride=ld_for(max_kv))


def _case(n_q, max_kv, seed, label):
    rng = np.random.default_rng(seed)
    pos = rng.integers(max_kv // 3, max_kv, n_q)
    pos[0] = max_kv - 1
    b = _batch(pos, max_kv)
    ld = ld_for(max_kv)
    s = torch.from_numpy(rng.standard_normal((n_q, ld)).astype(np.float32))
    s[::2] = torch.round(s[::2] * 8) / 8          # ties across chunk boundaries
    s = s.to(DEV)
    need = dsa.topk_workspace_size(b, 2048)
    say(f"[noalloc] {label}: n_q={n_q} max_kv={max_kv} plan workspace={need} B")
    assert need <= (16 << 20)
    ref = dsa.topk(b, s, 2048)
    got = torch.full_like(ref, -7)
    dsa.topk_noalloc(b, s, 2048, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), f"{label}: dsa_topk_noalloc differs from dsa_topk"
    return need


def test_noalloc_matches_topk_twice():
    n1 = _case(64, 32768, 1, "first call")
    n2 = _case(16, 20000, 2, "second call, smaller")
    assert n1 > 0 and n2 > 0, "both batches must take the plan that uses the scratch array"


def test_noalloc_refuses_oversized_batches():
    pos = np.full(300, 131071)
    b = _batch(pos, 131072)
    need = dsa.topk_workspace_size(b, 4096)
    assert need > (16 << 20)
    s = torch.empty((1, 4), dtype=torch.float32, device=DEV)   # never read: the call returns before any launch
    idx = torch.empty((1, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(dsa.DSAError) as e:
        dsa.topk_noalloc(b, s, 4096, idx)
    assert e.value.status == 2 and "scratch" in e.value.message
