"""Guard bands and repeatability of every entry point.

Each output and each workspace is allocated with exactly the size the call
needs, between two 4 KiB bands filled with a known byte; after the call the
bands must be untouched (no write outside the buffer the caller handed in),
the inputs must be unchanged, and a second identical call must reproduce the
outputs bit for bit (no race, no order-dependent reduction). Shapes are small
and ragged (row counts and positions off the tile and block grid)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

BAND = 4096
PATTERN = 0xA5


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


class Guarded:
    """A tensor between two bands of PATTERN bytes."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((n + 2 * BAND,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[BAND:BAND + n].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def intact(self):
        lo = self.buf[:BAND]
        hi = self.buf[BAND + self.n:]
        return bool((lo == PATTERN).all()) and bool((hi == PATTERN).all())


def ws_guard(nbytes):
    return Guarded((max(int(nbytes), 1),), torch.uint8)


def rnd(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(dtype)


def snapshot(*ts):
    return [t.clone() for t in ts]


def unchanged(before, ts):
    return all(torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b) for a, b in zip(before, ts))


def run_twice(call, outs, guards, inputs):
    before = snapshot(*inputs)
    call()
    torch.cuda.synchronize()
    first = snapshot(*outs)
    for o in outs:
        o.zero_()
    call()
    torch.cuda.synchronize()
    for g in guards:
        assert g.intact(), "write outside a buffer"
    assert unchanged(before, inputs), "an input was modified"
    for a, b in zip(first, outs):
        assert torch.equal(a, b), "second call differs"


def test_guards_compress_and_index_prefill(qsa):
    L, Hi, r, k, n_q = 2999, 8, 4, 64, 413
    q0 = L - n_q
    ik = rnd((1, L, 64), 1)
    iq = rnd((n_q, Hi, 64), 2)
    cmp = Guarded((1, L // r, 64), torch.bfloat16)
    run_twice(lambda: qsa.qsa_compress_keys(ik, cmp.t, r, 0, L // r), [cmp.t], [cmp], [ik])
    d = qsa.index_desc(r, k, Hi)
    q_pos0 = torch.tensor([q0], dtype=torch.int32, device="cuda")
    sel = Guarded((1, n_q, k), torch.int32)
    cnt = Guarded((1, n_q), torch.int32)
    ws = ws_guard(qsa.qsa_index_topk_workspace_size(d, 1, n_q, L))
    run_twice(lambda: qsa.qsa_index_topk(d, iq[None], cmp.t, q_pos0, L, sel.t, cnt.t, ws.t),
              [sel.t, cnt.t], [sel, cnt, ws], [iq, cmp.t, q_pos0])


def test_guards_index_decode_and_varlen(qsa):
    B, N, Hi, r, k = 3, 2500, 8, 4, 128
    cmp = rnd((B, N, 64), 3)
    iq = rnd((B, 1, Hi, 64), 4)
    q_pos0 = torch.tensor([N * r - 1, 777, 5001], dtype=torch.int32, device="cuda")
    d = qsa.index_desc(r, k, Hi)
    sel = Guarded((B, 1, k), torch.int32)
    cnt = Guarded((B, 1), torch.int32)
    ws = ws_guard(qsa.qsa_index_topk_workspace_size(d, B, 1, N * r))
    run_twice(lambda: qsa.qsa_index_topk(d, iq, cmp, q_pos0, N * r, sel.t, cnt.t, ws.t),
              [sel.t, cnt.t], [sel, cnt, ws], [iq, cmp, q_pos0])
    # packed rows: 5, 1 and 130 rows appended to prefixes of 900, 4000 and 7000 tokens
    rows = [5, 1, 130]
    pos = [900, 4000, 7000]
    cu = torch.tensor(np.cumsum([0] + rows), dtype=torch.int32, device="cuda")
    qp = torch.tensor(pos, dtype=torch.int32, device="cuda")
    tq, mq, end = sum(rows), max(rows), max(p + n for p, n in zip(pos, rows))
    iqv = rnd((tq, Hi, 64), 5)
    cmpv = rnd((B, (end + r - 1) // r + 8, 64), 6)
    sel = Guarded((tq, k), torch.int32)
    cnt = Guarded((tq,), torch.int32)
    ws = ws_guard(qsa.qsa_index_topk_varlen_workspace_size(d, B, mq, end))
    run_twice(lambda: qsa.qsa_index_topk_varlen(d, iqv, cmpv, cu, qp, mq, end, sel.t, cnt.t, ws.t),
              [sel.t, cnt.t], [sel, cnt, ws], [iqv, cmpv, cu, qp])


def _selection(n_q, q0, r, k, seed):
    """Ascending valid block lists (own block last) for rows at q0 + i."""
    rng = np.random.default_rng(seed)
    sel = np.full((n_q, k), -1, np.int32)
    cnt = np.zeros(n_q, np.int32)
    for i in range(n_q):
        bt = (q0 + i) // r
        m = min(k - 1, bt)
        sel[i, :m] = np.sort(rng.choice(bt, m, replace=False)) if m else []
        sel[i, m] = bt
        cnt[i] = m + 1
    return torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda()


def test_guards_attention(qsa):
    Hq, Hkv, D, r, k, L, n_q = 16, 2, 128, 4, 96, 3001, 131
    q0 = L - n_q
    Q = rnd((n_q, Hq, D), 7)
    K = rnd((L, Hkv, D), 8)
    V = rnd((L, Hkv, D), 9)
    sel, cnt = _selection(n_q, q0, r, k, 10)
    a = qsa.attn_desc(Hq, Hkv, D)
    out = Guarded((n_q, Hq, D), torch.bfloat16)
    lse = Guarded((n_q, Hq), torch.float32)
    ws = ws_guard(qsa.qsa_sparse_attn_workspace_size(a, 1, n_q, k, r))
    run_twice(lambda: qsa.qsa_sparse_attn_prefill(a, r, Q, K, V, q0, sel, cnt, out.t, lse.t, ws.t),
              [out.t, lse.t], [out, lse, ws], [Q, K, V, sel, cnt])
    # decode: 3 sequences of ragged lengths in caches of 3001 rows
    B = 3
    lens = [3001, 17, 1234]
    Qd = rnd((B, Hq, D), 11)
    Kc = rnd((B, L, Hkv, D), 12)
    Vc = rnd((B, L, Hkv, D), 13)
    kv_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sl, cn = [], []
    for b, n in enumerate(lens):
        s_, c_ = _selection(1, n - 1, r, k, 20 + b)
        sl.append(s_)
        cn.append(c_)
    seld, cntd = torch.cat(sl), torch.cat(cn)
    out = Guarded((B, Hq, D), torch.bfloat16)
    lse = Guarded((B, Hq), torch.float32)
    ws = ws_guard(qsa.qsa_sparse_attn_workspace_size(a, B, 1, k, r))
    run_twice(lambda: qsa.qsa_sparse_attn_decode(a, r, Qd, Kc, Vc, kv_len, seld, cntd, out.t, lse.t, ws.t),
              [out.t, lse.t], [out, lse, ws], [Qd, Kc, Vc, kv_len, seld, cntd])
    # dense comparator, prefill and decode
    out = Guarded((n_q, Hq, D), torch.bfloat16)
    lse = Guarded((n_q, Hq), torch.float32)
    ws = ws_guard(qsa.qsa_dense_attn_workspace_size(a, 1, n_q, L))
    run_twice(lambda: qsa.qsa_dense_attn_prefill(a, Q, K, V, q0, out.t, lse.t, ws.t),
              [out.t, lse.t], [out, lse, ws], [Q, K, V])
    out = Guarded((B, Hq, D), torch.bfloat16)
    lse = Guarded((B, Hq), torch.float32)
    ws = ws_guard(qsa.qsa_dense_attn_workspace_size(a, B, 1, L))
    run_twice(lambda: qsa.qsa_dense_attn_decode(a, Qd, Kc, Vc, kv_len, out.t, lse.t, ws.t),
              [out.t, lse.t], [out, lse, ws], [Qd, Kc, Vc, kv_len])


def test_guards_paged_attention(qsa):
    Hq, Hkv, D, r, k, page = 32, 4, 128, 4, 64, 64
    rows, pos = [3, 70], [500, 1900]
    B = len(rows)
    tq = sum(rows)
    max_pages = (max(p + n for p, n in zip(pos, rows)) + page - 1) // page
    n_pages = B * max_pages + 3
    perm = np.random.default_rng(30).permutation(n_pages)[:B * max_pages].reshape(B, max_pages)
    table = torch.from_numpy(perm.astype(np.int32)).cuda()
    Kp = rnd((n_pages, page, Hkv, D), 31)
    Vp = rnd((n_pages, page, Hkv, D), 32)
    Q = rnd((tq, Hq, D), 33)
    cu = torch.tensor(np.cumsum([0] + rows), dtype=torch.int32, device="cuda")
    qp = torch.tensor(pos, dtype=torch.int32, device="cuda")
    sl, cn = [], []
    for b in range(B):
        s_, c_ = _selection(rows[b], pos[b], r, k, 40 + b)
        sl.append(s_)
        cn.append(c_)
    sel, cnt = torch.cat(sl), torch.cat(cn)
    a = qsa.attn_desc(Hq, Hkv, D)
    out = Guarded((tq, Hq, D), torch.bfloat16)
    lse = Guarded((tq, Hq), torch.float32)
    run_twice(lambda: qsa.qsa_sparse_attn_prefill_paged(a, r, Q, Kp, Vp, table, cu, qp, sel, cnt, out.t, lse.t),
              [out.t, lse.t], [out, lse], [Q, Kp, Vp, table, cu, qp, sel, cnt])


def test_guards_distill_kl(qsa):
    Hkv, r, L, n_q = 2, 4, 1500, 201
    Hq, Hi, D = 8 * Hkv, 8, 128
    q0 = L - n_q
    Q = rnd((n_q, Hq, D), 50)
    K = rnd((L, Hkv, D), 51)
    iq = rnd((n_q, Hi, 64), 52)
    cmp = rnd((L // r, 64), 53)
    a = qsa.attn_desc(Hq, Hkv, D)
    d = qsa.index_desc(r, 64, Hi)
    kl = Guarded((n_q,), torch.float32)
    ws = ws_guard(qsa.qsa_distill_kl_workspace_size(a, n_q))
    run_twice(lambda: qsa.qsa_distill_kl_prefill(a, d, Q, K, iq, cmp, q0, kl.t, ws.t), [kl.t], [kl, ws],
              [Q, K, iq, cmp])


def test_guards_gated_delta_rule(qsa):
    B, T, Hqk, Hv = 2, 333, 2, 4
    q = torch.nn.functional.normalize(rnd((B, T, Hqk, 128), 60, torch.float32), dim=-1).bfloat16()
    k = torch.nn.functional.normalize(rnd((B, T, Hqk, 128), 61, torch.float32), dim=-1).bfloat16()
    v = rnd((B, T, Hv, 128), 62)
    g = torch.nn.functional.logsigmoid(rnd((B, T, Hv), 63, torch.float32) + 3)
    beta = torch.sigmoid(rnd((B, T, Hv), 64, torch.float32))
    S0 = rnd((B, Hv, 128, 128), 65, torch.float32, 0.25)
    d = qsa.gdn_desc(Hqk, Hv)
    out = Guarded((B, T, Hv, 128), torch.bfloat16)
    Sf = Guarded((B, Hv, 128, 128), torch.float32)
    ws = ws_guard(qsa.qsa_gdn_prefill_workspace_size(d, B, T))
    run_twice(lambda: qsa.qsa_gdn_prefill(d, q, k, v, g, beta, out.t, initial_state=S0, final_state=Sf.t,
                                          workspace=ws.t),
              [out.t, Sf.t], [out, Sf, ws], [q, k, v, g, beta, S0])
    # decode updates the state in place: restore it before the second call
    state = Guarded((B, Hv, 128, 128), torch.float32, S0)
    dout = Guarded((B, Hv, 128), torch.bfloat16)
    args = (q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(), g[:, 0].contiguous(),
            beta[:, 0].contiguous())

    def call():
        state.t.copy_(S0)
        qsa.qsa_gdn_decode(d, *args, state.t, dout.t)
    run_twice(call, [dout.t, state.t], [state, dout], list(args))
