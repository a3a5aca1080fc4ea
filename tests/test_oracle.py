"""Pins of the CPU oracle against facts fixed outside the oracle itself:
a hand-worked example, closed forms, algebraic identities, brute-force
enumeration on tiny inputs, the O(n^2 / r) pair count, and a library routine
(PyTorch's scaled_dot_product_attention in float64) for dense attention.
Each test is chosen so that a plausible slip in the oracle (off-by-one block,
dropped ReLU, wrong sign, wrong tie order, wrong GQA head map, missing causal
mask on the diagonal block) fails it.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from gen.configs import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    return gen.f32_to_bf16(np.asarray(x, np.float32))


def widen(a):
    return gen.bf16_to_f64(a)


# ------------------------------------------------------------- worked example
def _parse_worked():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "worked_example.txt")) if l.strip() and l[0] != "#"]
    keys = np.array([float(v) for v in rows[0][1:]]).reshape(12, 2)
    blocks = np.array([float(v) for v in rows[1][1:]]).reshape(3, 2)
    queries = []
    for r in rows[2:]:
        t = int(r[1])
        q = np.array([float(v) for v in r[2:6]]).reshape(2, 2)
        i_s, i_sel = r.index("scores"), r.index("sel")
        sc = [float(v) for v in r[i_s + 1:i_sel]]
        sel = [int(v) for v in r[i_sel + 1:]]
        queries.append((t, q, sc, sel))
    return keys, blocks, queries


def test_worked_example():
    keys, blocks, queries = _parse_worked()
    cb = oracle.compress(bf(keys), 4)
    assert np.array_equal(widen(cb), blocks)
    for t, q, sc, sel in queries:
        b = t // 4
        got = oracle.scores(bf(q), cb[:b], 0.5)
        assert got.tolist() == sc
        s, c, _, pairs = oracle.select(bf(q)[None], cb, t, 4, 2, 0.5)
        assert s[0].tolist() == sel, (t, s[0], sel)
        assert c[0] == sum(1 for v in sel if v >= 0)
        assert pairs == b


# ------------------------------------------------------------------------ O1
def test_compress_block_constants():
    # each block's 4 tokens hold the same distinct value -> block key = value
    L, d, r = 64, 8, 4
    vals = np.arange(L // r, dtype=np.float32) * 0.5 - 3.0
    keys = np.repeat(vals, r)[:, None] * np.ones((1, d), np.float32)
    out = oracle.compress(bf(keys), r)
    assert np.array_equal(widen(out)[:, 0], vals.astype(np.float64))


def test_compress_integer_mean_exact_and_tail_skipped():
    L, d, r = 4 * 50 + 3, 16, 4  # ragged tail of 3 tokens is not a block
    keys = gen.ints(7, 5, (L, d), -8, 8)
    out = oracle.compress(keys, r)
    assert out.shape == (50, d)
    ik = widen(keys)[:200].reshape(50, r, d).sum(1)  # exact integer sums
    assert np.array_equal(widen(out), ik / 4.0)  # multiples of 1/4 in [-8, 8]: exact in bf16


@pytest.mark.parametrize("r", [1, 2, 4, 8])
def test_compress_vs_double_mean(r):
    L, d = 4096, 64
    keys = gen.normal(11, 5, (L, d))
    out = oracle.compress(keys, r)
    if r == 1:
        assert np.array_equal(out, keys)
        return
    m = widen(keys).reshape(L // r, r, d).mean(1)
    ref = bf(m.astype(np.float32))  # fp32 of the exact mean, then bf16
    diff = np.abs(out.astype(np.int32) - ref.astype(np.int32))
    # the fp32 running sum can only move the result across a bf16 rounding
    # boundary: at most one bf16 step, and rarely
    assert diff.max() <= 1
    assert (diff == 0).mean() > 0.995


# ------------------------------------------------------------------------ O2
def test_scores_single_head_is_relu_dot():
    q = gen.normal(3, 4, (1, 64))
    c = gen.normal(3, 5, (300, 64))
    got = oracle.scores(q, c, 1.0)
    ref = np.maximum(widen(c) @ widen(q)[0], 0.0).astype(np.float32)
    assert np.array_equal(got, ref)


def test_scores_relu_identity_and_sign():
    # relu(x) - relu(-x) = x, so s(q) - s(-q) = w * sum_h q_h . c  (matmul)
    H, d, n, w = 8, 64, 500, 1.0 / 8
    q = gen.normal(5, 4, (H, d))
    c = gen.normal(5, 5, (n, d))
    neg = q ^ np.uint16(0x8000)
    lhs = oracle.scores(q, c, w).astype(np.float64) - oracle.scores(neg, c, w).astype(np.float64)
    rhs = w * (widen(c) @ widen(q).T).sum(1)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-5)
    # scores are non-negative and exactly 0 when every head is negative
    s = oracle.scores(q, c, w)
    assert (s >= 0).all()
    allneg = ((widen(c) @ widen(q).T) <= 0).all(1)
    assert (s[allneg] == 0).all()


def test_scores_head_permutation_and_scaling():
    H, d, n = 4, 64, 400
    q = gen.normal(9, 4, (H, d))
    c = gen.normal(9, 5, (n, d))
    s = oracle.scores(q, c, 0.25)
    perm = oracle.scores(q[[2, 0, 3, 1]], c, 0.25)
    assert np.allclose(s, perm, rtol=1e-6, atol=0)
    # doubling q (exact in bf16) doubles every score exactly; w scales linearly
    q2 = bf(widen(q) * 2.0)
    assert np.array_equal(oracle.scores(q2, c, 0.25), s * 2)
    assert np.array_equal(oracle.scores(q, c, 0.5), s * 2)


# ------------------------------------------------------------------------ O3
def _brute_kept(s, m):
    """The unique m-subset whose members all precede all non-members in
    (score desc, index asc) order, found by enumeration."""
    n = len(s)
    found = []
    for sub in itertools.combinations(range(n), m):
        ss = set(sub)
        ok = all((s[a] > s[x]) or (s[a] == s[x] and a < x) for a in ss for x in range(n) if x not in ss)
        if ok:
            found.append(sub)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("r", [1, 2, 4])
@pytest.mark.parametrize("kind", ["ints", "normal"])
def test_select_bruteforce(r, kind):
    L, d = 28, 8
    rng_seed = 100 + r
    for H in (1, 3):
        if kind == "ints":  # many exact ties, including zeros
            keys = gen.ints(rng_seed, 5, (L, d), -1, 1)
            q = gen.ints(rng_seed, 4, (L, H, d), -1, 1)
        else:
            keys = gen.normal(rng_seed, 5, (L, d))
            q = gen.normal(rng_seed, 4, (L, H, d))
        blocks = oracle.compress(keys, r)
        for k in range(1, 7):
            sel, cnt, band, pairs = oracle.select(q, blocks, 0, r, k, 1.0 / H)
            assert pairs == sum(t // r for t in range(L))
            for t in range(L):
                b = t // r
                s = oracle.scores(q[t], blocks[:b], 1.0 / H).tolist()
                m = min(k - 1, b)
                kept = _brute_kept(s, m) if b else []
                want = sorted(kept + [b])
                assert sel[t, :cnt[t]].tolist() == want, (r, H, k, t)
                assert (sel[t, cnt[t]:] == -1).all()
                assert cnt[t] == min(k, b + 1)


@pytest.mark.parametrize("name", ["c1"])
def test_select_invariants_config(name):
    W = CONFIGS[name]
    keys = gen.idx_keys(W.seed, 0, W.L, 0, W.L, W.di, W.needle_window, W.r)
    blocks = oracle.compress(keys, W.r)
    q = gen.normal(W.seed, gen.STREAM_IDX_Q, (W.n_q, W.Hi, W.di))
    sel, cnt, band, pairs = oracle.select(q, blocks, 0, W.r, W.k, W.w)
    t = np.arange(W.n_q)
    b = t // W.r
    N = W.L // W.r
    assert pairs == W.r * N * (N - 1) // 2  # sum_t floor(t / r), from position 0
    assert pairs / W.L ** 2 == pytest.approx(1.0 / (2 * W.r), rel=1e-3)  # the O(n^2 / r) claim
    assert (cnt == np.minimum(W.k, b + 1)).all()
    for i in range(W.n_q):
        row = sel[i, :cnt[i]]
        assert (np.diff(row) > 0).all()
        assert row[-1] == b[i]  # diagonal present, nothing after it (causal)
        ntok = sum(min(W.r, t[i] - j * W.r + 1) for j in row)
        assert ntok <= W.k * W.r
    # near-tie band bookkeeping: last kept >= first dropped
    has = ~np.isnan(band).any(1)
    assert (band[has, 0] >= band[has, 1]).all()


def test_select_budget_covers_context_keeps_everything():
    L, r = 64, 4
    keys = gen.normal(21, 5, (L, 64))
    q = gen.normal(21, 4, (L, 2, 64))
    blocks = oracle.compress(keys, r)
    sel, cnt, _, _ = oracle.select(q, blocks, 0, r, L // r, 0.5)
    for t in range(L):
        assert sel[t, :cnt[t]].tolist() == list(range(t // r + 1))


def test_select_ragged_start_and_length():
    # queries starting mid-block, context not a multiple of r
    L, r, k = 203, 4, 5
    keys = gen.normal(31, 5, (L, 64))
    q = gen.normal(31, 4, (L, 2, 64))
    blocks = oracle.compress(keys, r)
    t0 = 77
    sel, cnt, _, pairs = oracle.select(q[t0:], blocks, t0, r, k, 0.5)
    assert pairs == sum(t // r for t in range(t0, L))
    for i, t in enumerate(range(t0, L)):
        b = t // r
        s = oracle.scores(q[t], blocks[:b], 0.5).tolist()
        assert sel[i, :cnt[i]].tolist() == sorted(_brute_kept(s, min(k - 1, b)) + [b])


# -------------------------------------------------------------------- O5/O6
def _torch_dense(Q, K, V, t0, scale):
    q = torch.from_numpy(widen(Q)).permute(1, 0, 2)[None]  # [1, Hq, nq, D]
    G = Q.shape[1] // K.shape[1]
    L = t0 + Q.shape[0]
    k = torch.from_numpy(widen(K[:L])).repeat_interleave(G, 1).permute(1, 0, 2)[None]
    v = torch.from_numpy(widen(V[:L])).repeat_interleave(G, 1).permute(1, 0, 2)[None]
    # causal with an offset: query i sits at position t0 + i
    mask = torch.arange(L)[None, :] <= (t0 + torch.arange(Q.shape[0]))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_dense_vs_torch_sdpa_fp64():
    L, Hq, Hkv, D = 96, 8, 2, 128
    Q = gen.normal(41, 1, (L, Hq, D))
    K = gen.normal(41, 2, (L, Hkv, D))
    V = gen.normal(41, 3, (L, Hkv, D))
    t0 = 30
    o, lse = oracle.dense_attn(Q[t0:], K, V, t0)
    ref = _torch_dense(Q[t0:], K, V, t0, D ** -0.5)
    assert np.abs(o - ref).max() < 1e-12


def test_sparse_equals_dense_when_budget_covers_context():
    L, Hq, Hkv, D, r = 80, 4, 1, 128, 4
    Q = gen.normal(43, 1, (L, Hq, D))
    K = gen.normal(43, 2, (L, Hkv, D))
    V = gen.normal(43, 3, (L, Hkv, D))
    q = gen.normal(43, 4, (L, 2, 64))
    blocks = oracle.compress(gen.normal(43, 5, (L, 64)), r)
    sel, cnt, _, _ = oracle.select(q, blocks, 0, r, L // r, 0.5)
    o1, l1 = oracle.sparse_attn(Q, K, V, 0, r, sel, cnt)
    o2, l2 = oracle.dense_attn(Q, K, V, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_attend_closed_forms():
    L, Hq, Hkv, D = 40, 4, 2, 128
    K = gen.normal(47, 2, (L, Hkv, D))
    V = gen.normal(47, 3, (L, Hkv, D))
    q = gen.normal(47, 1, (Hq, D))
    # one kept token: output is that token's V row, lse is its logit
    o, lse = oracle.attend_tokens(q, K, V, [17])
    for h in range(Hq):
        g = h // (Hq // Hkv)
        assert np.array_equal(o[h], widen(V[17, g]))
        assert lse[h] == pytest.approx(widen(q[h]) @ widen(K[17, g]) / math.sqrt(D), abs=1e-12)
    # zero query: uniform weights -> mean of kept V rows, lse = ln |T|
    toks = [1, 5, 6, 30, 39]
    o, lse = oracle.attend_tokens(np.zeros((Hq, D), np.uint16), K, V, toks)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        assert np.allclose(o[h], widen(V[toks, g]).mean(0), atol=1e-14)
        assert lse[h] == pytest.approx(math.log(len(toks)), abs=1e-14)
    # constant V: output is that constant
    Vc = np.full_like(V, bf(1.5)[()])
    o, _ = oracle.attend_tokens(q, K, Vc, toks)
    assert np.allclose(o, 1.5, atol=1e-14)


def test_diagonal_block_is_causally_masked():
    # query at t = 4j + 1: its own block contributes tokens 4j and 4j + 1 only
    L, Hq, Hkv, D, r = 32, 2, 1, 128, 4
    Q = gen.normal(53, 1, (L, Hq, D))
    K = gen.normal(53, 2, (L, Hkv, D))
    V = gen.normal(53, 3, (L, Hkv, D))
    t = 4 * 5 + 1
    sel = np.array([[2, 5]], np.int32)
    cnt = np.array([2], np.int32)
    o, lse = oracle.sparse_attn(Q[t:t + 1], K, V, t, r, sel, cnt)
    o2, lse2 = oracle.attend_tokens(Q[t], K, V, [8, 9, 10, 11, 20, 21])
    assert np.array_equal(o[0], o2) and np.array_equal(lse[0], lse2)
    # and the same query through the library routine over those six tokens
    mask = np.zeros(L, bool)
    mask[[8, 9, 10, 11, 20, 21]] = True
    qq = torch.from_numpy(widen(Q[t]))[None, :, None, :]
    kk = torch.from_numpy(widen(K[:, 0]))[None, None].expand(1, Hq, L, D)
    vv = torch.from_numpy(widen(V[:, 0]))[None, None].expand(1, Hq, L, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=torch.from_numpy(mask)[None, None, None])
    assert np.abs(o[0] - ref[0, :, 0].numpy()).max() < 1e-12


# ------------------------------------------------------------------ O7 pins --
def _kl_inputs(seed, L, Hq, Hkv, Hi, r):
    Q = gen.normal(seed, 1, (L, Hq, 128))
    K = gen.normal(seed, 2, (L, Hkv, 128))
    iq = gen.normal(seed, 4, (L, Hi, 64))
    ik = gen.normal(seed, 5, (L, 64))
    return Q, K, iq, oracle.compress(ik, r)


def _lse(x):
    m = max(x)
    return m + math.log(sum(math.exp(v - m) for v in x))


def test_distill_kl_zero_queries_closed_form():
    # Q = 0: every head attends uniformly, every complete candidate block holds
    # r of the t + 1 tokens, so the target is uniform over the b_t candidates and
    # KL = lse(s) - mean(s) - ln b_t in terms of the (pinned) O2 scores alone
    L, Hq, Hkv, Hi, r = 120, 4, 2, 4, 4
    Q, K, iq, blocks = _kl_inputs(71, L, Hq, Hkv, Hi, r)
    Q0 = np.zeros_like(Q)
    t0 = 20
    kl = oracle.distill_kl(Q0[t0:], K, iq[t0:], blocks, t0, r, 1.0 / Hi)
    for i, t in enumerate(range(t0, L)):
        bt = t // r
        s = [float(v) for v in oracle.scores(iq[t], blocks[:bt], 1.0 / Hi)]
        want = _lse(s) - sum(s) / bt - math.log(bt)
        assert kl[i] == pytest.approx(want, abs=1e-12)


def test_distill_kl_zero_when_both_uniform_and_trivial_cases():
    L, Hq, Hkv, Hi, r = 64, 4, 1, 4, 4
    Q, K, iq, blocks = _kl_inputs(73, L, Hq, Hkv, Hi, r)
    # zero attention and zero indexer queries: both distributions uniform
    kl = oracle.distill_kl(np.zeros_like(Q), K, np.zeros_like(iq), blocks, 0, r, 1.0 / Hi)
    assert np.all(np.abs(kl) < 1e-13)
    # b_t = 0 (no candidate): 0; b_t = 1 (one candidate): both distributions are [1]
    kl = oracle.distill_kl(Q[:8], K, iq[:8], blocks, 0, r, 1.0 / Hi)
    assert np.all(kl[:4] == 0.0)
    assert np.all(np.abs(kl[4:8]) < 1e-13)


@pytest.mark.parametrize("peak", [1.0, 8.0])
def test_distill_kl_target_mass_vs_torch_softmax(peak):
    # The target built independently: torch's float64 softmax over the causal
    # prefix with the KV heads repeated per query-head group (head h reads KV
    # head h // G), the softmax scale 1/sqrt(D) applied to the logits, the
    # attention of every head summed per candidate block j < b_t and
    # renormalised; the indexer side as torch's log-softmax of the O2 scores.
    # Non-zero queries (and peaked ones, Q x 8) make the attention non-uniform,
    # so a wrong KV-head map, a missing scale or a block boundary off by a
    # token all change the loss.
    L, Hq, Hkv, Hi, r = 160, 8, 2, 8, 4
    Q, K, iq, blocks = _kl_inputs(83, L, Hq, Hkv, Hi, r)
    if peak != 1.0:
        Q = gen.f32_to_bf16(gen.bf16_to_f64(Q).astype(np.float32) * np.float32(peak))
    t0 = 9
    kl = oracle.distill_kl(Q[t0:], K, iq[t0:], blocks, t0, r, 1.0 / Hi)
    G = Hq // Hkv
    Kt = torch.from_numpy(widen(K)).repeat_interleave(G, dim=1)  # [L, Hq, D]
    scale = 1.0 / math.sqrt(128)
    for i, t in enumerate(range(t0, L)):
        bt = t // r
        q = torch.from_numpy(widen(Q[t]))  # [Hq, D]
        logits = torch.einsum("hd,shd->hs", q, Kt[: t + 1]) * scale
        a = torch.softmax(logits, dim=1)  # [Hq, t + 1]
        mass = a[:, : bt * r].sum(0).reshape(bt, r).sum(1)
        p = mass / mass.sum()
        s = torch.from_numpy(oracle.scores(iq[t], blocks[:bt], 1.0 / Hi).astype(np.float64))
        logq = torch.log_softmax(s, dim=0)
        want = float((p * (torch.log(p) - logq)).sum())
        assert kl[i] == pytest.approx(want, abs=1e-12, rel=1e-12), (t, kl[i], want)


def test_distill_kl_nonnegative_and_depends_on_scores():
    L, Hq, Hkv, Hi, r = 200, 8, 2, 8, 4
    Q, K, iq, blocks = _kl_inputs(79, L, Hq, Hkv, Hi, r)
    kl = oracle.distill_kl(Q[8:], K, iq[8:], blocks, 8, r, 1.0 / Hi)
    assert np.all(kl >= -1e-13) and np.all(np.isfinite(kl))
    # a larger indexer temperature-free logit scale changes the loss
    iq2 = gen.f32_to_bf16(gen.bf16_to_f64(iq).astype(np.float32) * 4)
    kl2 = oracle.distill_kl(Q[8:], K, iq2[8:], blocks, 8, r, 1.0 / Hi)
    assert not np.allclose(kl, kl2)


# ------------------------------------------------------------------ O8 pins --
def _gdn_small(seed, T, Hqk, Hv, dk, dv):
    q, k, v, g, beta = gen.gdn_inputs(seed, 1, T, Hqk, Hv, dk, dv)
    return q[0], k[0], v[0], g[0], beta[0]


def test_gdn_single_token_closed_form():
    # one token on a zero state: the error is v itself, S = b v k^T and
    # o = scale * b * (k . q) * v
    q, k, v, g, beta = _gdn_small(81, 1, 2, 4, 16, 8)
    o, S = oracle.gdn(q, k, v, g, beta, scale=0.3)
    for h in range(4):
        kk, qq, vv, b = widen(k[0, h // 2]), widen(q[0, h // 2]), widen(v[0, h]), float(beta[0, h])
        assert np.allclose(S[h], b * np.outer(vv, kk), rtol=1e-13, atol=1e-15)
        assert np.allclose(o[0, h], 0.3 * b * (kk @ qq) * vv, rtol=1e-12, atol=1e-15)


def test_gdn_no_write_only_decays():
    # write gate 0: the state only decays, S_t = exp(g_1 + .. + g_t) S0
    T, Hqk, Hv, dk, dv = 7, 1, 2, 8, 4
    q, k, v, g, beta = _gdn_small(82, T, Hqk, Hv, dk, dv)
    S0 = gen.gdn_state(82, 1, Hv, dv, dk)[0]
    o, S = oracle.gdn(q, k, v, g, np.zeros_like(beta), scale=0.5, S0=S0)
    G = np.cumsum(g.astype(np.float64), axis=0)
    for h in range(Hv):
        assert np.allclose(S[h], math.exp(G[-1, h]) * S0[h].astype(np.float64), rtol=1e-12)
        for t in range(T):
            ref = 0.5 * math.exp(G[t, h]) * (S0[h].astype(np.float64) @ widen(q[t, 0]))
            assert np.allclose(o[t, h], ref, rtol=1e-11, atol=1e-14)


def test_gdn_full_write_of_unit_keys_returns_the_value():
    # decay 1, write gate 1 and exactly unit keys: every token overwrites what
    # the memory returns for its key, so reading with q = k gives v back
    T, dk, dv = 40, 32, 8
    rng = np.random.default_rng(83)
    k = np.zeros((T, 1, dk), np.float32)
    for t in range(T):
        idx = rng.choice(dk, 16, replace=False)
        k[t, 0, idx] = rng.choice([-0.25, 0.25], 16)  # 16 * 1/16 = 1 exactly
    k = bf(k)
    v = gen.normal(83, 10, (T, 1, dv))
    o, _ = oracle.gdn(k, k, v, np.zeros((T, 1), np.float32), np.ones((T, 1), np.float32), scale=1.0)
    assert np.abs(o[:, 0] - widen(v[:, 0])).max() < 1e-12


def test_gdn_orthogonal_keys_closed_form():
    # distinct coordinate keys never interfere: from a zero state
    # S_T = sum_t b_t (prod_{s > t} a_s) v_t e_{p(t)}^T and
    # o_t = scale * sum_{s <= t} b_s (prod_{s < u <= t} a_u) q_t[p(s)] v_s
    T, dk, dv = 12, 16, 6
    rng = np.random.default_rng(84)
    perm = rng.permutation(dk)[:T]
    k = np.zeros((T, 1, dk), np.float32)
    k[np.arange(T), 0, perm] = 1.0
    k = bf(k)
    q = gen.normal(84, 8, (T, 1, dk))
    v = gen.normal(84, 10, (T, 1, dv))
    g = (-rng.uniform(0.01, 1.0, (T, 1))).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (T, 1)).astype(np.float32)
    o, S = oracle.gdn(q, k, v, g, beta, scale=0.7)
    a = np.exp(g[:, 0].astype(np.float64))
    b = beta[:, 0].astype(np.float64)
    V, Q = widen(v[:, 0]), widen(q[:, 0])
    ST = np.zeros((dv, dk))
    for t in range(T):
        ST[:, perm[t]] += b[t] * np.prod(a[t + 1:]) * V[t]
    assert np.allclose(S[0], ST, rtol=1e-12, atol=1e-15)
    for t in range(T):
        ref = sum(b[s] * np.prod(a[s + 1:t + 1]) * Q[t, perm[s]] * V[s] for s in range(t + 1))
        assert np.allclose(o[t, 0], 0.7 * ref, rtol=1e-11, atol=1e-14)


def test_gdn_matches_expanded_transition_products():
    # the recurrence unrolled: with A_t = a_t (I - b_t k_t k_t^T),
    # S_t = S0 A_1 .. A_t + sum_{s <= t} b_s v_s k_s^T A_{s+1} .. A_t
    T, Hqk, Hv, dk, dv = 10, 2, 4, 8, 5
    q, k, v, g, beta = _gdn_small(85, T, Hqk, Hv, dk, dv)
    S0 = gen.gdn_state(85, 1, Hv, dv, dk)[0]
    o, S = oracle.gdn(q, k, v, g, beta, scale=0.9, S0=S0)
    for h in range(Hv):
        K, Q, V = widen(k[:, h // 2]), widen(q[:, h // 2]), widen(v[:, h])
        a, b = np.exp(g[:, h].astype(np.float64)), beta[:, h].astype(np.float64)
        A = [a[t] * (np.eye(dk) - b[t] * np.outer(K[t], K[t])) for t in range(T)]
        for t in range(T):
            St = S0[h].astype(np.float64)
            for u in range(t + 1):
                St = St @ A[u]
            for s in range(t + 1):
                W = b[s] * np.outer(V[s], K[s])
                for u in range(s + 1, t + 1):
                    W = W @ A[u]
                St = St + W
            assert np.allclose(o[t, h], 0.9 * St @ Q[t], rtol=1e-10, atol=1e-13)
            if t == T - 1:
                assert np.allclose(S[h], St, rtol=1e-10, atol=1e-13)


def test_gdn_key_head_map_and_state_carry():
    # value head h reads key head h // (Hv / Hqk): the same as repeating the key
    # heads; and running [0, T1) then [T1, T) from the carried state is the same
    # as one run (up to the fp32 rounding of the carried state)
    T, T1, Hqk, Hv, dk, dv = 30, 13, 2, 6, 16, 8
    q, k, v, g, beta = _gdn_small(86, T, Hqk, Hv, dk, dv)
    o, S = oracle.gdn(q, k, v, g, beta)
    rep = np.repeat(np.arange(Hqk), Hv // Hqk)
    o2, S2 = oracle.gdn(q[:, rep], k[:, rep], v, g, beta)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    oa, Sa = oracle.gdn(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1])
    ob, Sb = oracle.gdn(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], S0=Sa.astype(np.float32))
    assert np.allclose(oa, o[:T1], rtol=0, atol=0)
    assert np.allclose(ob, o[T1:], rtol=1e-5, atol=1e-6)
    assert np.allclose(Sb, S, rtol=1e-5, atol=1e-6)


def test_gdn_heads_subset():
    T, Hqk, Hv, dk, dv = 9, 1, 3, 8, 4
    q, k, v, g, beta = _gdn_small(87, T, Hqk, Hv, dk, dv)
    o, S = oracle.gdn(q, k, v, g, beta)
    o1, S1 = oracle.gdn(q, k, v, g, beta, heads=[2])
    assert np.array_equal(o1[:, 2], o[:, 2]) and np.isnan(o1[:, :2]).all()
    assert np.array_equal(S1[2], S[2])
