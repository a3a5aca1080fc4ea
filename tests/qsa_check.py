"""Shared helpers of the GPU parity tests: upload of generated inputs and the
comparison rules (selection band, attention tolerances)."""
import numpy as np
import torch

import gen
import oracle

# Attention output tolerances (bf16 inputs, fp32 accumulation), plus an fp32
# check on the log-sum-exp that a single missing or extra token would break.
OUT_MAX_ABS = 2e-2
OUT_MEAN_ABS = 1e-3
LSE_MAX_ABS = 2e-4
# Selection: bit-exact except inside the oracle's near-tie band.
BAND_REL = 1e-4


def dev(a):
    """numpy uint16 bf16 bits -> torch bfloat16 on the GPU (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_selection(g_sel, g_cnt, o_sel, o_cnt, band, scores_of_row, rows=None):
    """Compare GPU and oracle selections row by row. Rows must agree exactly
    unless the oracle's last-kept and first-dropped scores are within BAND_REL;
    then the sets may differ only by candidates whose oracle score lies in the
    band around the last kept score. Returns the number of rows that differ
    (all inside the band)."""
    g_sel = np.asarray(g_sel)
    g_cnt = np.asarray(g_cnt)
    rows = range(len(o_cnt)) if rows is None else rows
    n_band = 0
    for i, gi in zip(range(len(o_cnt)), rows):
        oc, gc = int(o_cnt[i]), int(g_cnt[gi])
        assert oc == gc, f"row {gi}: count {gc} != oracle {oc}"
        if np.array_equal(g_sel[gi], o_sel[i]):
            continue
        a, b = float(band[i, 0]), float(band[i, 1])
        assert abs(a - b) <= BAND_REL * max(abs(a), abs(b)), \
            f"row {gi}: selections differ outside a near tie (a={a}, b={b})"
        assert (g_sel[gi, gc:] == -1).all()
        gs = set(g_sel[gi, :gc].tolist())
        os_ = set(o_sel[i, :oc].tolist())
        assert len(gs) == gc and max(gs) == max(os_), f"row {gi}: malformed GPU selection"
        s = scores_of_row(i)
        for j in gs ^ os_:
            assert abs(float(s[j]) - a) <= BAND_REL * abs(a), f"row {gi}: block {j} score {s[j]} outside band of {a}"
        n_band += 1
    return n_band


def check_attention(g_out, g_lse, o_out, o_lse, what=""):
    go = g_out.float().cpu().numpy().astype(np.float64)
    err = np.abs(go - o_out)
    assert err.max() <= OUT_MAX_ABS, f"{what} max abs {err.max()}"
    assert err.mean() <= OUT_MEAN_ABS, f"{what} mean abs {err.mean()}"
    if g_lse is not None:
        le = np.abs(g_lse.cpu().numpy().astype(np.float64) - o_lse)
        assert le.max() <= LSE_MAX_ABS, f"{what} lse max abs {le.max()}"
    return err.max(), err.mean()


def prefill_inputs(W, n_rows=None):
    """Host inputs of a prefill workload (bf16 bits)."""
    L = W.L
    n_q = W.n_q if n_rows is None else n_rows
    Q = gen.normal(W.seed, gen.STREAM_Q, (n_q, W.Hq, W.D))
    K = gen.normal(W.seed, gen.STREAM_K, (L, W.Hkv, W.D))
    V = gen.normal(W.seed, gen.STREAM_V, (L, W.Hkv, W.D))
    iq = gen.normal(W.seed, gen.STREAM_IDX_Q, (n_q, W.Hi, W.di))
    ik = gen.idx_keys(W.seed, 0, L, 0, L, W.di, W.needle_window, W.r)
    return Q, K, V, iq, ik


def oracle_rows_scores(iq_rows, blocks, t_rows, r, w):
    def f(i):
        return oracle.scores(iq_rows[i], blocks[: t_rows[i] // r], w)
    return f
