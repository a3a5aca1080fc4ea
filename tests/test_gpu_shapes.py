"""GPU parity for the shapes the C ABI accepts beyond the benchmarked ones:
every supported query-heads-per-KV-head group size on the prefill and the
split-KV decode attention, the smallest budgets (k = 1: the own block only;
k = 2: one candidate) through the whole path, and the prefill indexer on
several sequences with their own first positions in one call."""
import numpy as np
import pytest
import torch

import gen
import oracle
from qsa_check import check_attention, check_selection, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


def _say(*a):
    print("[case]", *a, flush=True)


def _seed_ends_short(scores, keep, rho=16):
    """Whether the many-query indexer's seed for one (query, split) lies above
    the split's keep-th best score, so that its buffer ends short and the split
    is scanned again. scores: the split's candidates' scores in block order.
    Follows the kernel's sampling: 64-block tiles 0, rho, 2 rho, ... of the
    split; lane c of a 32-candidate subtile keeps the four best sampled
    scores of candidates c, c + 32, ...; the seed is the m-th best of those
    128, m = ceil(2.5 keep S / n). None when the split is not seeded."""
    n = len(scores)
    j = np.arange(n)
    sampled = (j // 64) % rho == 0
    S = int(sampled.sum())
    m = -(-(5 * keep * S) // (2 * n))
    if n < 4 * keep or m > 96:
        return None
    kept = []
    for c in range(32):
        kept.extend(np.sort(scores[sampled & (j % 32 == c)])[::-1][:4])
    seed = np.sort(np.asarray(kept))[::-1][m - 1]
    return int((scores >= seed).sum()) < keep


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (8, 2), (16, 1), (64, 4), (12, 4)])
def test_attention_head_groups(qsa, Hq, Hkv):
    # prefill rows at the start and at the end of a 1500-token context, then
    # decode of three sequences with ragged lengths, all on the oracle's
    # selections (budget 256 tokens, r = 4)
    D, Hi, r, k, L, seed = 128, 4, 4, 64, 1500, 700 + Hq + Hkv
    _say("head groups", Hq, Hkv)
    K = gen.normal(seed, 2, (L, Hkv, D))
    V = gen.normal(seed, 3, (L, Hkv, D))
    blocks = oracle.compress(gen.idx_keys(seed, 0, L, 0, L, 64, 0, r), r)
    desc = qsa.attn_desc(Hq, Hkv, D)
    for q0, n in [(0, 37), (L - 45, 45)]:
        Q = gen.normal(seed, 1, (n, Hq, D), e0=q0 * Hq * D)
        iq = gen.normal(seed, 4, (n, Hi, 64), e0=q0 * Hi * 64)
        o_sel, o_cnt, _, _ = oracle.select(iq, blocks, q0, r, k, 1.0 / Hi)
        out = torch.empty((n, Hq, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((n, Hq), dtype=torch.float32, device="cuda")
        qsa.qsa_sparse_attn_prefill(desc, r, dev(Q), dev(K), dev(V), q0,
                                    torch.from_numpy(np.ascontiguousarray(o_sel)).cuda(),
                                    torch.from_numpy(np.ascontiguousarray(o_cnt)).cuda(), out, lse)
        torch.cuda.synchronize()
        o_out, o_lse = oracle.sparse_attn(Q, K, V, q0, r, o_sel, o_cnt)
        check_attention(out, lse, o_out, o_lse, f"prefill G={Hq // Hkv} rows {q0}..")
    # decode: sequence b reads the first kv_len[b] tokens of its own cache
    B, max_len = 3, L
    kv_len = np.array([L, 701, 3], np.int32)
    Kc = gen.normal(seed + 1, 2, (B, max_len, Hkv, D))
    Vc = gen.normal(seed + 1, 3, (B, max_len, Hkv, D))
    Qd = gen.normal(seed + 1, 1, (B, Hq, D))
    sel = np.full((B, k), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        t = int(kv_len[b]) - 1
        ikb = gen.idx_keys(seed + 1, b, max_len, 0, max_len, 64, 0, r)
        iqb = gen.normal(seed + 1, 4, (1, Hi, 64), e0=b * Hi * 64)
        s, c, _, _ = oracle.select(iqb, oracle.compress(ikb, r), t, r, k, 1.0 / Hi)
        sel[b], cnt[b] = s[0], c[0]
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = qsa.workspace(qsa.qsa_sparse_attn_workspace_size(desc, B, 1, k, r))
    qsa.qsa_sparse_attn_decode(desc, r, dev(Qd), dev(Kc), dev(Vc), torch.from_numpy(kv_len).cuda(),
                               torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(), out, lse, ws)
    torch.cuda.synchronize()
    for b in range(B):
        t = int(kv_len[b]) - 1
        o_out, o_lse = oracle.sparse_attn(Qd[b][None], Kc[b], Vc[b], t, r, sel[b:b + 1], cnt[b:b + 1])
        check_attention(out[b:b + 1], lse[b:b + 1], o_out, o_lse, f"decode G={Hq // Hkv} seq {b}")


@pytest.mark.parametrize("k", [1, 2])
def test_smallest_budgets_end_to_end(qsa, k):
    # k = 1 keeps only the query's own block (nothing is scored); k = 2 keeps
    # the best earlier block beside it. Prefill from position 0 (the first
    # rows have no earlier block) and decode at ragged lengths.
    from block_sparse_long_09_amd.pipeline import DecodePath, PrefillPath
    Hq, Hkv, Hi, D, r, L, seed = 16, 2, 8, 128, 4, 2000, 930 + k
    _say("smallest budget", k)
    Q = gen.normal(seed, 1, (L, Hq, D))
    K = gen.normal(seed, 2, (L, Hkv, D))
    V = gen.normal(seed, 3, (L, Hkv, D))
    iq = gen.normal(seed, 4, (L, Hi, 64))
    ik = gen.idx_keys(seed, 0, L, 0, L, 64, 0, r)
    path = PrefillPath(Hq, Hkv, Hi, r, k, n_q_max=L, max_len=L)
    cmp = torch.zeros((L // r, 64), dtype=torch.bfloat16, device="cuda")
    out, lse = path(dev(Q), dev(K), dev(V), dev(iq), dev(ik), cmp, 0, L)
    torch.cuda.synchronize()
    g_sel = path.sel[:L].cpu().numpy()
    g_cnt = path.cnt[:L].cpu().numpy()
    blocks = oracle.compress(ik, r)
    o_sel, o_cnt, band, _ = oracle.select(iq, blocks, 0, r, k, 1.0 / Hi)
    assert np.array_equal(g_cnt, o_cnt)
    if k == 1:
        assert np.array_equal(g_sel, o_sel)  # the own block, nothing to rank
    else:
        check_selection(g_sel, g_cnt, o_sel, o_cnt, band,
                        lambda i: oracle.scores(iq[i], blocks[: i // r], 1.0 / Hi))
    o_out, o_lse = oracle.sparse_attn(Q, K, V, 0, r, g_sel, g_cnt)
    check_attention(out, lse, o_out, o_lse, f"prefill k={k}")
    # decode of three sequences sharing the same caches' layout
    B = 3
    kv_len = np.array([L, 999, 2], np.int32)
    Kc = gen.normal(seed + 1, 2, (B, L, Hkv, D))
    Vc = gen.normal(seed + 1, 3, (B, L, Hkv, D))
    Qd = gen.normal(seed + 1, 1, (B, Hq, D))
    iqd = gen.normal(seed + 1, 4, (B, Hi, 64))
    ikd = np.stack([gen.idx_keys(seed + 1, b, L, 0, L, 64, 0, r) for b in range(B)])
    cmpd = torch.zeros((B, L // r, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(dev(ikd), cmpd, r, 0, L // r)
    dpath = DecodePath(Hq, Hkv, Hi, B, L, r=r, k=k)
    kvl = torch.from_numpy(kv_len).cuda()
    dout, dlse = dpath(dev(Qd), dev(Kc), dev(Vc), dev(iqd), cmpd, kvl, kvl - 1)
    torch.cuda.synchronize()
    d_sel = dpath.sel[:, 0].cpu().numpy()
    d_cnt = dpath.cnt[:, 0].cpu().numpy()
    for b in range(B):
        t = int(kv_len[b]) - 1
        bl = oracle.compress(ikd[b], r)
        s, c, bd, _ = oracle.select(iqd[b][None], bl, t, r, k, 1.0 / Hi)
        check_selection(d_sel[b:b + 1], d_cnt[b:b + 1], s, c, bd,
                        lambda i: oracle.scores(iqd[b], bl[: t // r], 1.0 / Hi))
        o_out, o_lse = oracle.sparse_attn(Qd[b][None], Kc[b], Vc[b], t, r, d_sel[b:b + 1], d_cnt[b:b + 1])
        check_attention(dout[b:b + 1], dlse[b:b + 1], o_out, o_lse, f"decode k={k} seq {b}")


@pytest.mark.parametrize("n_q", [20, 200])
def test_index_topk_batched_prefill(qsa, n_q):
    # three sequences, each with its own first query position (one from 0,
    # two ragged ones), in one call: the few-query kernel at 20 rows, the
    # many-query one at 200
    B, Hi, r, k, seed = 3, 8, 4, 128, 960 + n_q
    pos = [0, 3000, 1517]
    end = max(pos) + n_q
    N = end // r + 1
    _say("batched prefill indexer", n_q)
    iq = gen.normal(seed, 4, (B, n_q, Hi, 64))
    ik = np.stack([gen.idx_keys(seed, b, N * r, 0, N * r, 64, 512, r) for b in range(B)])
    blocks = [oracle.compress(ik[b], r) for b in range(B)]
    cmp = torch.zeros((B, N, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(dev(ik), cmp, r, 0, N)
    d = qsa.index_desc(r, k, Hi)
    sel = torch.empty((B, n_q, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, n_q), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_workspace_size(d, B, n_q, end))
    q_pos0 = torch.tensor(pos, dtype=torch.int32, device="cuda")
    qsa.qsa_index_topk(d, dev(iq), cmp, q_pos0, end, sel, cnt, ws)
    torch.cuda.synchronize()
    g_sel, g_cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        o_sel, o_cnt, band, _ = oracle.select(iq[b], blocks[b], pos[b], r, k, 1.0 / Hi)
        check_selection(g_sel[b], g_cnt[b], o_sel, o_cnt, band,
                        lambda i: oracle.scores(iq[b][i], blocks[b][: (pos[b] + i) // r], 1.0 / Hi))


def test_index_topk_seeded_buffers_that_end_short(qsa):
    # At a budget of 512 blocks the many-query indexer first scores every
    # 16th 64-block tile of its candidate split and seeds each query's
    # threshold from that sample. Here the keys of exactly those tiles (one
    # split: it starts at block 0) are scaled by 8, so each seed lands among
    # their scores and fewer than k - 1 candidates reach it: such a buffer ends
    # short and its split is scanned again from an unseeded threshold. Three
    # of every eight consecutive queries (one wave's share) have zero indexer
    # vectors (all scores 0, every candidate tied): their buffers fill, so
    # they keep their first scan while their neighbours rescan.
    B, n_q, Hi, r, k, seed = 4, 4096, 8, 4, 512, 977
    pos0 = 40000
    end = pos0 + n_q
    N = end // r + 1
    _say("seeded buffers that end short")
    blocks = gen.normal(seed, 5, (B, N, 64))
    x = gen.bf16_to_f64(blocks)
    x[:, (np.arange(N) // 64) % 16 == 0] *= 8.0
    blocks = gen.f32_to_bf16(x.astype(np.float32))
    iq = gen.normal(seed, 4, (B, n_q, Hi, 64))
    iq[:, (np.arange(n_q) % 8) < 3] = 0
    d = qsa.index_desc(r, k, Hi)
    sel = torch.empty((B, n_q, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, n_q), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_workspace_size(d, B, n_q, end))
    q_pos0 = torch.full((B,), pos0, dtype=torch.int32, device="cuda")
    qsa.qsa_index_topk(d, dev(iq), dev(blocks), q_pos0, end, sel, cnt, ws)
    torch.cuda.synchronize()
    g_sel, g_cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    rows = [0, 1, 2, 3, 7, 8, 100, 1001, 2047, 2050, 4093, 4094, 4095]
    # the pattern does force the rescan: queries with nonzero vectors are
    # seeded above their split's (k - 1)-th score (one split from block 0)
    for qi in (3, 7, 1003, 4095):
        sc = oracle.scores(iq[0, qi], blocks[0][: (pos0 + qi) // r], 1.0 / Hi)
        assert _seed_ends_short(sc, k - 1) is True, qi
    for b in range(B):
        for qi in rows:
            o_sel, o_cnt, band, _ = oracle.select(iq[b, qi:qi + 1], blocks[b], pos0 + qi, r, k, 1.0 / Hi)
            check_selection(g_sel[b, qi:qi + 1], g_cnt[b, qi:qi + 1], o_sel, o_cnt, band,
                            lambda i: oracle.scores(iq[b, qi], blocks[b][: (pos0 + qi) // r], 1.0 / Hi))


def test_index_topk_varlen_seeded_buffers_that_end_short(qsa):
    # The same forced rescan on the packed-batch indexer (three 4-wave
    # workgroups per CU, one tile per barrier): the keys of the sampled tiles
    # of every candidate split (every 16th 64-block tile from the split's
    # start; the split length follows from the plan's split count) are scaled
    # by 8. Three sequences with their own cached prefixes; three of every
    # eight rows have zero indexer vectors.
    B, Hi, r, k, seed = 3, 8, 4, 512, 981
    pos0 = [150000, 140000, 160000]
    n = [200, 64, 150]
    max_q, end = max(n), max(p + m for p, m in zip(pos0, n))
    N = end // r + 1
    _say("varlen seeded buffers that end short")
    d = qsa.index_desc(r, k, Hi)
    info = qsa.qsa_index_topk_plan_info(d, B, max_q, end, packed=True)
    assert info.sample_stride == 16
    max_cand = (end - 1) // r
    split_len = ((max_cand + info.splits - 1) // info.splits + 63) // 64 * 64
    blk = np.arange(N)
    sampled = ((blk % split_len) // 64) % 16 == 0
    blocks = gen.normal(seed, 5, (B, N, 64))
    x = gen.bf16_to_f64(blocks)
    x[:, sampled] *= 8.0
    blocks = gen.f32_to_bf16(x.astype(np.float32))
    iqs = [gen.normal(seed + b, 4, (n[b], Hi, 64)) for b in range(B)]
    for b in range(B):
        iqs[b][(np.arange(n[b]) % 8) < 3] = 0
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    total = int(cu[-1])
    sel = torch.empty((total, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((total,), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_varlen_workspace_size(d, B, max_q, end))
    qsa.qsa_index_topk_varlen(d, dev(np.concatenate(iqs)), dev(blocks), torch.from_numpy(cu).cuda(),
                              torch.tensor(pos0, dtype=torch.int32, device="cuda"), max_q, end, sel, cnt, ws)
    torch.cuda.synchronize()
    g_sel, g_cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    # the pattern does force the rescan: in every seeded split of a query
    # with a nonzero vector the seed lies above the split's (k - 1)-th score
    for b in range(B):
        qi = n[b] - 1
        sc = oracle.scores(iqs[b][qi], blocks[b][: (pos0[b] + qi) // r], 1.0 / Hi)
        short = [_seed_ends_short(sc[s0:s0 + split_len], k - 1) for s0 in range(0, len(sc), split_len)]
        assert True in short and False not in short, (b, short)
    for b in range(B):
        for qi in sorted({0, 1, 2, 3, 5, n[b] // 2, n[b] - 1}):
            row = int(cu[b]) + qi
            o_sel, o_cnt, band, _ = oracle.select(iqs[b][qi:qi + 1], blocks[b], pos0[b] + qi, r, k, 1.0 / Hi)
            check_selection(g_sel[row:row + 1], g_cnt[row:row + 1], o_sel, o_cnt, band,
                            lambda i: oracle.scores(iqs[b][qi], blocks[b][: (pos0[b] + qi) // r], 1.0 / Hi))


@pytest.mark.parametrize("Hi,n_q,w", [(8, 256, 0.3), (4, 256, 0.3), (8, 20, 0.3),
                                      (1, 256, None), (2, 256, None), (16, 256, None)])
def test_index_topk_seeded_head_counts_and_weights(qsa, Hi, n_q, w):
    # the many-query kernel (each query has ~5000 candidates; seeded from 2
    # heads up) at every head count it is built for, and a head weight that is not a power of
    # two (0.3), which is applied in the epilogue (sum * w) instead of being
    # folded into the bf16 queries, also on the few-query kernel
    B, r, k, seed = 1, 4, 512, 990 + Hi + n_q
    w = 1.0 / Hi if w is None else w
    pos = 20000
    end = pos + n_q
    N = end // r + 1
    _say("head weight", w, "Hi", Hi, "n_q", n_q)
    iq = gen.normal(seed, 4, (B, n_q, Hi, 64))
    ik = gen.idx_keys(seed, 0, N * r, 0, N * r, 64, 512, r)
    blocks = oracle.compress(ik, r)
    cmp = torch.zeros((B, N, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(dev(ik[None]), cmp, r, 0, N)
    d = qsa.index_desc(r, k, Hi, idx_head_weight=w)
    if n_q >= 64:  # no sample at one head (its kernel has no registers to spare)
        assert qsa.qsa_index_topk_plan_info(d, B, n_q, end).sample_stride == (16 if Hi >= 2 else 0)
    sel = torch.empty((B, n_q, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, n_q), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_workspace_size(d, B, n_q, end))
    qsa.qsa_index_topk(d, dev(iq), cmp, torch.tensor([pos], dtype=torch.int32, device="cuda"), end, sel, cnt, ws)
    torch.cuda.synchronize()
    g_sel, g_cnt = sel.cpu().numpy()[0], cnt.cpu().numpy()[0]
    o_sel, o_cnt, band, _ = oracle.select(iq[0], blocks, pos, r, k, w)
    check_selection(g_sel, g_cnt, o_sel, o_cnt, band, lambda i: oracle.scores(iq[0][i], blocks[: (pos + i) // r], w))


def test_index_topk_seeded_budget_1024(qsa):
    # a budget of 1024 blocks seeds from every 32nd tile: 2 x 8192 queries
    # over ~10K-12K candidates each, one candidate split
    B, n_q, Hi, r, k, seed = 2, 8192, 8, 4, 1024, 995
    pos0 = 40000
    end = pos0 + n_q
    N = end // r + 1
    _say("seeded budget 1024")
    d = qsa.index_desc(r, k, Hi)
    info = qsa.qsa_index_topk_plan_info(d, B, n_q, end)
    assert info.sample_stride == 32 and info.splits == 1
    blocks = gen.normal(seed, 5, (B, N, 64))
    iq = gen.normal(seed, 4, (B, n_q, Hi, 64))
    sel = torch.empty((B, n_q, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, n_q), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_workspace_size(d, B, n_q, end))
    q_pos0 = torch.full((B,), pos0, dtype=torch.int32, device="cuda")
    qsa.qsa_index_topk(d, dev(iq), dev(blocks), q_pos0, end, sel, cnt, ws)
    torch.cuda.synchronize()
    g_sel, g_cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for qi in (0, 1, 63, 64, 4095, 4096, 8190, 8191):
            o_sel, o_cnt, band, _ = oracle.select(iq[b, qi:qi + 1], blocks[b], pos0 + qi, r, k, 1.0 / Hi)
            check_selection(g_sel[b, qi:qi + 1], g_cnt[b, qi:qi + 1], o_sel, o_cnt, band,
                            lambda i: oracle.scores(iq[b, qi], blocks[b][: (pos0 + qi) // r], 1.0 / Hi))


@pytest.mark.parametrize("q_pos0,n_q,chunk", [(0, 16384, 4096), (4096, 10000, 4096)])
def test_chunked_prefill_two_streams_matches_chunk_by_chunk(qsa, q_pos0, n_q, chunk):
    # chunk c's attention beside chunk c + 1's compression and indexer on two
    # streams gives the bits of the chunks run one after the other (the
    # second case starts after a cached prefix and ends with a ragged chunk)
    from block_sparse_long_09_amd.pipeline import ChunkedPrefill, PrefillPath
    Hq, Hkv, Hi, D, r, k, seed = 16, 2, 4, 128, 4, 512, 1010 + q_pos0
    L = q_pos0 + n_q
    _say("chunked prefill", q_pos0, n_q, chunk)
    Q, K, V = dev(gen.normal(seed, 1, (n_q, Hq, D))), dev(gen.normal(seed, 2, (L, Hkv, D))), dev(gen.normal(seed, 3, (L, Hkv, D)))
    iq = dev(gen.normal(seed, 4, (n_q, Hi, 64)))
    ik = dev(gen.idx_keys(seed, 0, L, 0, L, 64, 512, r))
    cmp_a = torch.zeros((L // r, 64), dtype=torch.bfloat16, device="cuda")
    cmp_b = torch.zeros_like(cmp_a)
    if q_pos0 // r:
        qsa.qsa_compress_keys(ik, cmp_a, r, 0, q_pos0 // r)
        qsa.qsa_compress_keys(ik, cmp_b, r, 0, q_pos0 // r)
    seq = PrefillPath(Hq, Hkv, Hi, r, k, n_q_max=chunk, max_len=L)
    ref_out = torch.empty((n_q, Hq, D), dtype=torch.bfloat16, device="cuda")
    ref_lse = torch.empty((n_q, Hq), dtype=torch.float32, device="cuda")
    for c0 in range(0, n_q, chunk):
        n = min(chunk, n_q - c0)
        o, l = seq(Q[c0:c0 + n], K, V, iq[c0:c0 + n], ik, cmp_a, q_pos0 + c0, n)
        ref_out[c0:c0 + n] = o
        ref_lse[c0:c0 + n] = l
    torch.cuda.synchronize()
    cp = ChunkedPrefill(Hq, Hkv, Hi, r, k, chunk=chunk, max_len=L)
    for _ in range(2):  # twice: the alternating selection buffers are reused
        out = torch.full((n_q, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((n_q, Hq), 7.0, dtype=torch.float32, device="cuda")
        cp(Q, K, V, iq, ik, cmp_b, q_pos0, n_q, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(cmp_b, cmp_a)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
