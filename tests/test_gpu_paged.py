"""GPU parity of the packed variable-length batch over a paged K/V pool: new
rows of several sequences appended to cached prefixes of different lengths
(one sequence gets a single row, like a decode step), K/V scattered over
shuffled pages. Selections and outputs are checked against the oracle per
sequence (on the sequence's contiguous K/V), and the paged attention against
the contiguous-K/V prefill call, which must agree bit for bit."""
import numpy as np
import pytest
import torch

import gen
import oracle
from qsa_check import check_attention, check_selection, dev, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("r,k,page", [(4, 128, 64), (1, 256, 16), (16, 64, 16)])
def test_paged_varlen_prefill(qsa, r, k, page):
    from block_sparse_long_09_amd.pipeline import PagedBatchPath
    Hq, Hkv, Hi, D = 32, 4, 8, 128
    pos0 = [0, 3000, 777, 12345, 5, 20000]
    n = [300, 64, 1, 500, 40, 77]
    B = len(pos0)
    L = [p + m for p, m in zip(pos0, n)]
    max_len = (max(L) + page - 1) // page * page
    max_pages = max_len // page
    _say("paged varlen r", r, "k", k, "page", page)
    rng = np.random.default_rng(7)
    Ks = [gen.normal(600 + b, 2, (L[b], Hkv, D)) for b in range(B)]
    Vs = [gen.normal(600 + b, 3, (L[b], Hkv, D)) for b in range(B)]
    iks = [gen.idx_keys(600 + b, 0, L[b], 0, L[b], 64, 512, r) for b in range(B)]
    Qs = [gen.normal(600 + b, 1, (n[b], Hq, D)) for b in range(B)]
    iqs = [gen.normal(600 + b, 4, (n[b], Hi, 64)) for b in range(B)]
    # shuffled pages
    pages_of = [(L[b] + page - 1) // page for b in range(B)]
    n_pages = sum(pages_of) + 3
    perm = rng.permutation(n_pages)
    table = np.zeros((B, max_pages), np.int32)
    kpool = np.zeros((n_pages, page, Hkv, D), np.uint16)
    vpool = np.zeros((n_pages, page, Hkv, D), np.uint16)
    nxt = 0
    for b in range(B):
        for pg in range(pages_of[b]):
            phys = int(perm[nxt]); nxt += 1
            table[b, pg] = phys
            s0, s1 = pg * page, min(L[b], (pg + 1) * page)
            kpool[phys, : s1 - s0] = Ks[b][s0:s1]
            vpool[phys, : s1 - s0] = Vs[b][s0:s1]
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    total = int(cu[-1])
    ik_cache = np.zeros((B, max_len, 64), np.uint16)
    for b in range(B):
        ik_cache[b, : L[b]] = iks[b]
    ik_d = dev(ik_cache)
    cmp = torch.zeros((B, max_len // r, 64), dtype=torch.bfloat16, device="cuda")
    for b in range(B):  # the cached prefix's block keys
        if pos0[b] // r:
            qsa.qsa_compress_keys(ik_d[b], cmp[b], r, 0, pos0[b] // r)
    path = PagedBatchPath(Hq, Hkv, Hi, B, max(n), max_len, r=r, k=k)
    cu_d = torch.from_numpy(cu).cuda()
    p0_d = torch.tensor(pos0, dtype=torch.int32, device="cuda")
    out, lse = path(dev(np.concatenate(Qs)), dev(kpool), dev(vpool), torch.from_numpy(table).cuda(),
                    dev(np.concatenate(iqs)), ik_d, cmp, cu_d, p0_d, pos0, n)
    torch.cuda.synchronize()
    g_sel = path.sel[:total].cpu().numpy()
    g_cnt = path.cnt[:total].cpu().numpy()
    desc = qsa.attn_desc(Hq, Hkv, D)
    for b in range(B):
        rows = slice(int(cu[b]), int(cu[b + 1]))
        blocks = oracle.compress(iks[b], r)
        assert np.array_equal(host_bits(cmp[b])[: L[b] // r], blocks), f"block keys of sequence {b}"
        o_sel, o_cnt, band, _ = oracle.select(iqs[b], blocks, pos0[b], r, k, 1.0 / Hi)
        check_selection(g_sel[rows], g_cnt[rows], o_sel, o_cnt, band,
                        lambda i: oracle.scores(iqs[b][i], blocks[: (pos0[b] + i) // r], 1.0 / Hi))
        o_out, o_lse = oracle.sparse_attn(Qs[b], Ks[b], Vs[b], pos0[b], r, g_sel[rows], g_cnt[rows])
        check_attention(out[rows], lse[rows], o_out, o_lse, f"paged sequence {b}")
        # the contiguous-K/V prefill call on the same selection: bit-identical
        ref_out = torch.empty((n[b], Hq, D), dtype=torch.bfloat16, device="cuda")
        ref_lse = torch.empty((n[b], Hq), dtype=torch.float32, device="cuda")
        qsa.qsa_sparse_attn_prefill(desc, r, dev(Qs[b]), dev(Ks[b]), dev(Vs[b]), pos0[b],
                                    path.sel[rows], path.cnt[rows], ref_out, ref_lse)
        torch.cuda.synchronize()
        assert torch.equal(ref_out.view(torch.int16), out[rows].view(torch.int16)), f"sequence {b}"
        assert torch.equal(ref_lse, lse[rows]), f"sequence {b} lse"
