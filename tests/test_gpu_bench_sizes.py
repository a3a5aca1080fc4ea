"""GPU parity of the calls the benchmark times beside the QSA step, at the
sizes it times them, on sampled rows the oracle computes one by one:
  - the dense GQA comparator over the 16384 queries of the 1M-token prefill
    (the sparse/dense ratio at 1M rests on it), against O6;
  - the distillation-loss forward over the 32768 queries of the 32K prefill,
    against O7;
  - the packed paged batch of eight sequences with cached prefixes of 128K to
    1,040,384 tokens (the prefix-cache serving case), per sequence against
    O2-O5 on the sequence's own contiguous K/V."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import gen
import oracle
from gen.configs import CONFIGS, PAGED
from gen.device import (idx_keys_to_device, normal_to_device, paged_batch_layout, paged_batch_to_device,
                        paged_sequence_host)
from qsa_check import check_attention, check_selection

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


def _say(*a):
    print("[case]", *a, flush=True)


def test_dense_prefill_1m_sampled_rows(qsa):
    # the comparator exactly as the benchmark launches it: one call over all
    # 16384 queries at positions 1,032,192 .. 1,048,575 against K/V [0, 1M)
    W = CONFIGS["c5a"]
    _say("dense prefill 1M, 16384 rows")
    K = normal_to_device(W.seed, 2, (W.L, W.Hkv, W.D))
    V = normal_to_device(W.seed, 3, (W.L, W.Hkv, W.D))
    Q = normal_to_device(W.seed, 1, (W.n_q, W.Hq, W.D))
    desc = qsa.attn_desc(W.Hq, W.Hkv, W.D)
    out = torch.empty((W.n_q, W.Hq, W.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((W.n_q, W.Hq), dtype=torch.float32, device="cuda")
    qsa.qsa_dense_attn_prefill(desc, Q, K, V, W.q_pos0, out, lse)
    torch.cuda.synchronize()
    del K, V, Q
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, W.n_q // 2, W.n_q - 1], rng.integers(0, W.n_q, 6)]))
    Kh = gen.normal(W.seed, 2, (W.L, W.Hkv, W.D))
    Vh = gen.normal(W.seed, 3, (W.L, W.Hkv, W.D))

    def ref(i):
        # one oracle call per row (each a single-row O6 over the 1M prefix);
        # the calls leave the interpreter lock, so the rows run side by side
        q = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=i * W.Hq * W.D)
        return oracle.dense_attn(q, Kh, Vh, W.q_pos0 + i)

    with ThreadPoolExecutor(max_workers=min(len(rows), 16)) as ex:
        refs = list(ex.map(ref, [int(i) for i in rows]))
    for i, (o_out, o_lse) in zip(rows, refs):
        i = int(i)
        check_attention(out[i:i + 1], lse[i:i + 1], o_out, o_lse, f"dense 1M row {i}")
    _say("dense 1M rows checked:", len(rows))


def test_distill_kl_32k_sampled_rows(qsa):
    # the loss over the 32K prefill's 32768 queries in one call, as timed
    W = CONFIGS["c2"]
    _say("distillation loss 32K, 32768 rows")
    K = normal_to_device(W.seed, 2, (W.L, W.Hkv, W.D))
    Q = normal_to_device(W.seed, 1, (W.n_q, W.Hq, W.D))
    iq = normal_to_device(W.seed, 4, (W.n_q, W.Hi, W.di))
    ik = idx_keys_to_device(W.seed, 1, W.L, W.di, W.needle_window, W.r)[0]
    cmp = torch.zeros((W.n_blk, W.di), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(ik, cmp, W.r, 0, W.n_blk)
    adesc = qsa.attn_desc(W.Hq, W.Hkv, W.D)
    idesc = qsa.index_desc(W.r, W.k, W.Hi, W.di)
    kl = torch.empty(W.n_q, dtype=torch.float32, device="cuda")
    ws = qsa.workspace(qsa.qsa_distill_kl_workspace_size(adesc, W.n_q))
    qsa.qsa_distill_kl_prefill(adesc, idesc, Q, K, iq, cmp, 0, kl, ws)
    torch.cuda.synchronize()
    g = kl.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 3, 4, 5, 4096, 16384, W.n_q - 3, W.n_q - 2, W.n_q - 1],
                                     rng.integers(W.n_q - 1024, W.n_q, 6), rng.integers(0, W.n_q, 4)]))
    assert len(rows) >= 16
    Kh = gen.normal(W.seed, 2, (W.L, W.Hkv, W.D))
    blocks = oracle.compress(gen.idx_keys(W.seed, 0, W.L, 0, W.L, W.di, W.needle_window, W.r), W.r)
    for i in rows:
        i = int(i)
        q = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=i * W.Hq * W.D)
        iqr = gen.normal(W.seed, 4, (1, W.Hi, W.di), e0=i * W.Hi * W.di)
        o = float(oracle.distill_kl(q, Kh, iqr, blocks, i, W.r, W.w)[0])
        # the same bar as the smaller distillation parity cases (1e-4 abs + 1e-4 rel)
        assert abs(g[i] - o) <= 1e-4 + 1e-4 * abs(o), f"row {i}: gpu {g[i]} oracle {o}"
    _say("distillation rows checked:", len(rows))


def test_paged_batch_c6_sampled_rows(qsa):
    # the packed batch as the benchmark runs it: eight sequences, cached
    # prefixes of 128K .. 1,040,384 tokens, 1 .. 4096 new rows, 256-token
    # shuffled pages; two rows per sequence at least (first and last new row)
    from block_sparse_long_09_amd.pipeline import PagedBatchPath
    W = PAGED["c6"]
    _say("paged batch c6")
    I = paged_batch_to_device(W)
    B = W.batch
    cmp = torch.zeros((B, I["max_len"] // W.r, W.di), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        qsa.qsa_compress_keys(I["ik"][b], cmp[b], W.r, 0, W.prefix[b] // W.r)
    path = PagedBatchPath(W.Hq, W.Hkv, W.Hi, B, max(W.new), I["max_len"], r=W.r, k=W.k, D=W.D, di=W.di)
    path.compress(I["ik"], cmp, W.prefix, W.new)
    path.select(I["iq"], cmp, I["cu"], I["q_pos0"], I["total"])
    path.attend(I["Q"], I["kpool"], I["vpool"], I["table"], I["cu"], I["q_pos0"], I["total"])
    torch.cuda.synchronize()
    total = I["total"]
    g_sel = path.sel[:total].cpu().numpy()
    g_cnt = path.cnt[:total].cpu().numpy()
    g_out = path.out[:total].cpu()
    g_lse = path.lse[:total].cpu()
    table = I["table_host"]
    del I, path, cmp
    torch.cuda.empty_cache()
    cu = np.concatenate([[0], np.cumsum(W.new)])
    key_len = paged_batch_layout(W)[2]
    rng = np.random.default_rng(17)
    n_rows = 0
    for b in range(B):
        n = W.new[b]
        loc = sorted({0, n - 1} | ({int(rng.integers(0, n))} if n > 2 else set()))
        L_b = W.prefix[b] + n
        # indexer keys are laid out [B, max_len, di] (max_len: the pages' span)
        blocks = oracle.compress(gen.idx_keys(W.seed, b, key_len, 0, L_b, W.di, W.needle_window, W.r), W.r)
        Kb = paged_sequence_host(W, table, b, 2, L_b)
        Vb = paged_sequence_host(W, table, b, 3, L_b)
        for i in loc:
            row = int(cu[b] + i)
            t = W.prefix[b] + i
            q = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=row * W.Hq * W.D)
            iqr = gen.normal(W.seed, 4, (1, W.Hi, W.di), e0=row * W.Hi * W.di)
            o_sel, o_cnt, band, _ = oracle.select(iqr, blocks, t, W.r, W.k, W.w)
            check_selection(g_sel[row:row + 1], g_cnt[row:row + 1], o_sel, o_cnt, band,
                            lambda _: oracle.scores(iqr[0], blocks[: t // W.r], W.w))
            o_out, o_lse = oracle.sparse_attn(q, Kb, Vb, t, W.r, g_sel[row:row + 1], g_cnt[row:row + 1])
            check_attention(g_out[row:row + 1], g_lse[row:row + 1], o_out, o_lse, f"c6 seq {b} row {i}")
            n_rows += 1
        _say("c6 sequence", b, "prefix", W.prefix[b], "rows", loc)
    assert n_rows >= 2 * B - 2  # the two single-row sequences give one row each

