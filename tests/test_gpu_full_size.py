"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, checked on sampled rows the oracle computes one by one; plus
decode edge cases (exact-tie fallback of the split merge, ragged lengths)."""
import numpy as np
import pytest
import torch

import gen
import oracle
from gen.configs import CONFIGS
from gen.device import idx_keys_to_device, normal_to_device
from qsa_check import check_attention, check_selection, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


def _say(*a):
    print("[case]", *a, flush=True)


def _rows_of(t):
    return t.cpu().numpy()


def _prefill_full(qsa, W, rows):
    """Run the whole prefill workload on the GPU (chunked like the benchmark)
    and return GPU selections/outputs of the requested query rows."""
    from block_sparse_long_09_amd.pipeline import PrefillPath
    K = normal_to_device(W.seed, 2, (W.L, W.Hkv, W.D))
    V = normal_to_device(W.seed, 3, (W.L, W.Hkv, W.D))
    Q = normal_to_device(W.seed, 1, (W.n_q, W.Hq, W.D))
    iq = normal_to_device(W.seed, 4, (W.n_q, W.Hi, W.di))
    ik = idx_keys_to_device(W.seed, 1, W.L, W.di, W.needle_window, W.r)[0]
    cmp = torch.zeros((W.n_blk, W.di), dtype=torch.bfloat16, device="cuda")
    if W.q_pos0 // W.r:
        qsa.qsa_compress_keys(ik, cmp, W.r, 0, W.q_pos0 // W.r)
    chunk = W.chunk or W.n_q
    path = PrefillPath(W.Hq, W.Hkv, W.Hi, W.r, W.k, n_q_max=chunk, max_len=W.q_pos0 + W.n_q, D=W.D, di=W.di)
    sel = np.empty((len(rows), W.k), np.int32)
    cnt = np.empty(len(rows), np.int32)
    out = torch.empty((len(rows), W.Hq, W.D), dtype=torch.bfloat16)
    lse = torch.empty((len(rows), W.Hq), dtype=torch.float32)
    rows = np.asarray(rows)
    for c0 in range(0, W.n_q, chunk):
        q0 = W.q_pos0 + c0
        path(Q[c0:c0 + chunk], K, V, iq[c0:c0 + chunk], ik, cmp, q0, chunk)
        mine = np.nonzero((rows >= c0) & (rows < c0 + chunk))[0]
        if len(mine):
            loc = torch.from_numpy(rows[mine] - c0).cuda()
            sel[mine] = path.sel[loc].cpu().numpy()
            cnt[mine] = path.cnt[loc].cpu().numpy()
            out[mine] = path.out[loc].cpu()
            lse[mine] = path.lse[loc].cpu()
    torch.cuda.synchronize()
    return sel, cnt, out, lse


def _oracle_prefill_rows(W, rows):
    """Oracle selection and attention of individual query rows (fresh inputs
    from the generator, only what those rows read)."""
    ik = gen.idx_keys(W.seed, 0, W.L, 0, W.L, W.di, W.needle_window, W.r)
    blocks = oracle.compress(ik, W.r)
    K = gen.normal(W.seed, 2, (W.L, W.Hkv, W.D))
    V = gen.normal(W.seed, 3, (W.L, W.Hkv, W.D))
    res = []
    for i in rows:
        i = int(i)
        t = W.q_pos0 + i
        q = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=i * W.Hq * W.D)
        iq = gen.normal(W.seed, 4, (1, W.Hi, W.di), e0=i * W.Hi * W.di)
        s, c, band, _ = oracle.select(iq, blocks, t, W.r, W.k, W.w)
        res.append((t, q, iq, s, c, band))
    return blocks, K, V, res


@pytest.mark.parametrize("name", ["c5a", "c3", "c2"])
def test_prefill_full_size_sampled_rows(qsa, name):
    W = CONFIGS[name]
    _say("prefill full size", name)
    rng = np.random.default_rng(7)
    chunk = W.chunk or W.n_q
    edge = [0, 1, chunk - 1, chunk, W.n_q - 1]
    rows = np.unique(np.concatenate([[e for e in edge if e < W.n_q], rng.integers(0, W.n_q, 24)]))
    g_sel, g_cnt, g_out, g_lse = _prefill_full(qsa, W, rows)
    blocks, K, V, res = _oracle_prefill_rows(W, rows)
    n_band = 0
    for gi, (t, q, iq, o_sel, o_cnt, band) in enumerate(res):
        n_band += check_selection(g_sel[gi:gi + 1], g_cnt[gi:gi + 1], o_sel, o_cnt, band,
                                  lambda _: oracle.scores(iq[0], blocks[: t // W.r], W.w))
        o_out, o_lse = oracle.sparse_attn(q, K, V, t, W.r, g_sel[gi:gi + 1], g_cnt[gi:gi + 1])
        check_attention(g_out[gi:gi + 1], g_lse[gi:gi + 1], o_out, o_lse, f"{name} row {rows[gi]}")
    _say(name, "rows in the tie band:", n_band, "of", len(rows))


def test_prefill_attention_large_kv_sampled_rows(qsa):
    """K and V of 300,000 tokens (614 MB): rows at the start of the context
    (lists of 1..12 blocks, ragged against the 32-token chunks), in the middle
    and at the end match the oracle on the oracle's selections, and the same
    rows given only the K/V prefix they need give the same bits."""
    Hq, Hkv, Hi, D, di, r, k, seed = 32, 4, 8, 128, 64, 4, 512, 4242
    L = 300_000
    _say("prefill attention, large K/V, L", L)
    K = normal_to_device(seed, 2, (L, Hkv, D))
    V = normal_to_device(seed, 3, (L, Hkv, D))
    Kh = gen.normal(seed, 2, (L, Hkv, D))
    Vh = gen.normal(seed, 3, (L, Hkv, D))
    blocks = oracle.compress(gen.idx_keys(seed, 0, L, 0, L, di, 4096, r), r)
    desc = qsa.attn_desc(Hq, Hkv, D)
    for q0, n in [(0, 45), (150_001, 37), (L - 29, 29)]:
        _say("rows", q0, "..", q0 + n - 1)
        Qh = gen.normal(seed, 1, (n, Hq, D), e0=q0 * Hq * D)
        iqh = gen.normal(seed, 4, (n, Hi, di), e0=q0 * Hi * di)
        o_sel, o_cnt, _, _ = oracle.select(iqh, blocks, q0, r, k, 1.0 / Hi)
        sel = torch.from_numpy(np.ascontiguousarray(o_sel)).cuda()
        cnt = torch.from_numpy(np.ascontiguousarray(o_cnt)).cuda()
        Q = dev(Qh)
        out = torch.empty((n, Hq, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((n, Hq), dtype=torch.float32, device="cuda")
        qsa.qsa_sparse_attn_prefill(desc, r, Q, K, V, q0, sel, cnt, out, lse)
        out1 = torch.empty_like(out)
        lse1 = torch.empty_like(lse)
        qsa.qsa_sparse_attn_prefill(desc, r, Q, K[:q0 + n], V[:q0 + n], q0, sel, cnt, out1, lse1)
        torch.cuda.synchronize()
        o_out, o_lse = oracle.sparse_attn(Qh, Kh, Vh, q0, r, o_sel, o_cnt)
        check_attention(out, lse, o_out, o_lse, f"rows {q0}..")
        assert torch.equal(out.view(torch.int16), out1.view(torch.int16)) and torch.equal(lse, lse1)


@pytest.mark.parametrize("name", ["c4", "c5b"])
def test_decode_full_size_sampled_rows(qsa, name):
    from block_sparse_long_09_amd.pipeline import DecodePath
    W = CONFIGS[name]
    _say("decode full size", name)
    Kc = normal_to_device(W.seed, 2, (W.batch, W.L, W.Hkv, W.D))
    Vc = normal_to_device(W.seed, 3, (W.batch, W.L, W.Hkv, W.D))
    Q = normal_to_device(W.seed, 1, (W.batch, W.Hq, W.D))
    iq = normal_to_device(W.seed, 4, (W.batch, W.Hi, W.di))
    ik = idx_keys_to_device(W.seed, W.batch, W.L, W.di, W.needle_window, W.r)
    cmp = torch.empty((W.batch, W.n_blk, W.di), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(ik, cmp, W.r, 0, W.n_blk)
    del ik
    kvl = torch.full((W.batch,), W.L, dtype=torch.int32, device="cuda")
    path = DecodePath(W.Hq, W.Hkv, W.Hi, W.batch, W.L, r=W.r, k=W.k, D=W.D, di=W.di)
    out, lse = path(Q, Kc, Vc, iq, cmp, kvl, kvl - 1)
    torch.cuda.synchronize()
    g_sel = path.sel[:, 0].cpu().numpy()
    g_cnt = path.cnt[:, 0].cpu().numpy()
    del Kc, Vc
    t = W.L - 1
    for b in sorted({0, W.batch // 2, W.batch - 1}):
        ikb = gen.idx_keys(W.seed, b, W.L, 0, W.L, W.di, W.needle_window, W.r)
        blocks = oracle.compress(ikb, W.r)
        iqb = gen.normal(W.seed, 4, (1, W.Hi, W.di), e0=b * W.Hi * W.di)
        o_sel, o_cnt, band, _ = oracle.select(iqb, blocks, t, W.r, W.k, W.w)
        check_selection(g_sel[b:b + 1], g_cnt[b:b + 1], o_sel, o_cnt, band,
                        lambda _: oracle.scores(iqb[0], blocks[: t // W.r], W.w))
        Kb = gen.normal(W.seed, 2, (W.L, W.Hkv, W.D), e0=b * W.L * W.Hkv * W.D)
        Vb = gen.normal(W.seed, 3, (W.L, W.Hkv, W.D), e0=b * W.L * W.Hkv * W.D)
        qb = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=b * W.Hq * W.D)
        o_out, o_lse = oracle.sparse_attn(qb, Kb, Vb, t, W.r, g_sel[b:b + 1], g_cnt[b:b + 1])
        check_attention(out[b:b + 1], lse[b:b + 1], o_out, o_lse, f"{name} seq {b}")


def test_decode_integer_ties_exact_fallback(qsa):
    # integer inputs make many exactly equal scores; the split lists' best
    # omitted score then ties the threshold and the merge must fall back to the
    # exact selection over all stored scores: bit-exact against the oracle
    from block_sparse_long_09_amd.pipeline import DecodePath
    B, L, Hq, Hkv, Hi, r, k = 3, 120003, 32, 4, 8, 4, 512
    _say("decode ties fallback")
    kv_len = np.array([120003, 77777, 4099], np.int32)
    ik = np.stack([gen.ints(31 + b, 5, (L, 64), -2, 2) for b in range(B)])
    iq = gen.ints(31, 4, (B, Hi, 64), -1, 1)
    cmp = torch.empty((B, L // r, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(dev(ik), cmp, r, 0, L // r)
    path = DecodePath(Hq, Hkv, Hi, B, L, r=r, k=k)
    kvl = torch.from_numpy(kv_len).cuda()
    path.select(dev(iq), cmp, kvl - 1)
    torch.cuda.synchronize()
    g_sel = path.sel[:, 0].cpu().numpy()
    g_cnt = path.cnt[:, 0].cpu().numpy()
    for b in range(B):
        t = int(kv_len[b]) - 1
        o_sel, o_cnt, _, _ = oracle.select(iq[b][None], oracle.compress(ik[b], r), t, r, k, 1.0 / Hi)
        assert g_cnt[b] == o_cnt[0]
        assert np.array_equal(g_sel[b], o_sel[0]), f"sequence {b}"


def test_decode_many_splits_normal_inputs_match(qsa):
    # decode path with ~200 splits and ragged lengths, against the oracle
    from block_sparse_long_09_amd.pipeline import DecodePath
    B, L, Hq, Hkv, Hi, r, k = 4, 800001, 32, 4, 8, 4, 512
    _say("decode many splits")
    kv_len = np.array([800001, 800000, 1025 * 4 + 3, 517], np.int32)
    ik = torch.empty((B, L, 64), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        ik[b] = dev(gen.idx_keys(41, b, L, 0, L, 64, 4096, r))
    iq = gen.normal(41, 4, (B, Hi, 64))
    cmp = torch.empty((B, L // r, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(ik, cmp, r, 0, L // r)
    path = DecodePath(Hq, Hkv, Hi, B, L, r=r, k=k)
    kvl = torch.from_numpy(kv_len).cuda()
    path.select(dev(iq), cmp, kvl - 1)
    torch.cuda.synchronize()
    g_sel = path.sel[:, 0].cpu().numpy()
    g_cnt = path.cnt[:, 0].cpu().numpy()
    for b in range(B):
        t = int(kv_len[b]) - 1
        blocks = oracle.compress(gen.idx_keys(41, b, L, 0, L, 64, 4096, r), r)
        o_sel, o_cnt, band, _ = oracle.select(iq[b][None], blocks, t, r, k, 1.0 / Hi)
        check_selection(g_sel[b:b + 1], g_cnt[b:b + 1], o_sel, o_cnt, band,
                        lambda _: oracle.scores(iq[b], blocks[: t // r], 1.0 / Hi))


def _bf16_bits(x):
    """float32 array -> bf16 bit patterns (round to nearest even)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _bf16_float(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("k", [16, 512, 1024])
def test_decode_clustered_selection(qsa, k):
    # sequence 0 has a run of 1200 blocks whose keys lean towards the query, so
    # the whole top-k falls into one or two splits, overflows their lists and
    # the merge must fall back to the stored scores; sequence 1 is plain
    from block_sparse_long_09_amd.pipeline import DecodePath
    B, L, Hq, Hkv, Hi, r = 2, 300003, 32, 4, 8, 4
    _say("decode clustered", k)
    kv_len = np.array([300003, 299999], np.int32)
    iq = gen.normal(51, 4, (B, Hi, 64))
    ik = np.stack([gen.normal(51 + b, 5, (L, 64)) for b in range(B)])
    lean = _bf16_float(iq[0]).mean(axis=0)  # mean query direction of sequence 0
    c0 = 100000
    ik[0, c0:c0 + 4800] = _bf16_bits(_bf16_float(ik[0, c0:c0 + 4800]) + 1.5 * lean[None, :])
    cmp = torch.empty((B, L // r, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(dev(ik), cmp, r, 0, L // r)
    path = DecodePath(Hq, Hkv, Hi, B, L, r=r, k=k)
    kvl = torch.from_numpy(kv_len).cuda()
    path.select(dev(iq), cmp, kvl - 1)
    torch.cuda.synchronize()
    g_sel = path.sel[:, 0].cpu().numpy()
    g_cnt = path.cnt[:, 0].cpu().numpy()
    for b in range(B):
        t = int(kv_len[b]) - 1
        blocks = oracle.compress(ik[b], r)
        o_sel, o_cnt, band, _ = oracle.select(iq[b][None], blocks, t, r, k, 1.0 / Hi)
        if b == 0:  # the cluster really holds the selection
            inside = np.count_nonzero((o_sel[0] >= c0 // r) & (o_sel[0] < (c0 + 4800) // r))
            assert inside >= min(k - 1, 1200) * 0.9, inside
        check_selection(g_sel[b:b + 1], g_cnt[b:b + 1], o_sel, o_cnt, band,
                        lambda _: oracle.scores(iq[b], blocks[: t // r], 1.0 / Hi))
