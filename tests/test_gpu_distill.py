"""GPU parity of the forward of the indexer's dense-distillation loss (O7)
against the oracle, per query: several micro-block sizes and head layouts,
rows from position 0 (no candidate, one candidate) to deep in the context."""
import numpy as np
import pytest
import torch

import gen
import oracle
from qsa_check import dev

pytestmark = pytest.mark.gpu

# fp32 sums of exp2 over the attended tokens and of the loss terms over the
# blocks, against the double oracle: ~1e-6 relative per sum; the loss is a
# difference of terms of size ~10, so 1e-4 absolute leaves a wide margin
KL_ATOL, KL_RTOL = 1e-4, 1e-4


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


@pytest.mark.parametrize("Hkv,r,L,n_q", [(2, 4, 3000, 300), (4, 4, 2048, 2048), (1, 1, 1500, 200), (4, 16, 5000, 96),
                                         (2, 32, 4000, 77)])
def test_distill_kl_matches_oracle(qsa, Hkv, r, L, n_q):
    Hq, Hi, D = 8 * Hkv, 8, 128
    seed = 700 + 10 * Hkv + r
    print("[case] distill kl", Hkv, r, L, n_q, flush=True)
    t0 = L - n_q
    Q = gen.normal(seed, 1, (n_q, Hq, D))
    K = gen.normal(seed, 2, (L, Hkv, D))
    iq = gen.normal(seed, 4, (n_q, Hi, 64))
    ik = gen.idx_keys(seed, 0, L, 0, L, 64, 512, r)
    blocks = oracle.compress(ik, r)
    adesc = qsa.attn_desc(Hq, Hkv, D)
    idesc = qsa.index_desc(r, 64, Hi)
    kl = torch.empty(n_q, dtype=torch.float32, device="cuda")
    ws = qsa.workspace(qsa.qsa_distill_kl_workspace_size(adesc, n_q))
    cmp = dev(blocks) if len(blocks) else torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_distill_kl_prefill(adesc, idesc, dev(Q), dev(K), dev(iq), cmp, t0, kl, ws)
    torch.cuda.synchronize()
    g = kl.cpu().numpy().astype(np.float64)
    o = oracle.distill_kl(Q, K, iq, blocks, t0, r, 1.0 / Hi)
    err = np.abs(g - o)
    worst = int(np.argmax(err - KL_RTOL * np.abs(o)))
    assert np.all(err <= KL_ATOL + KL_RTOL * np.abs(o)), \
        f"row {worst}: gpu {g[worst]} oracle {o[worst]} (max abs err {err.max()})"
    assert np.all(g[(t0 + np.arange(n_q)) // r == 0] == 0.0)
