"""The allocation-free decode attention (library scratch instead of a caller
workspace) against the workspace call on the same inputs: two calls in a row,
the second smaller, outputs identical bit for bit; a size whose partial
results exceed the scratch is refused on the host; and a decode step using
it, captured as a HIP graph, replays to the eager step's bits."""
import numpy as np
import pytest
import torch

import gen
from qsa_check import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


def _case(qsa, seed, B, L, kv_len, Hq, Hkv, Hi, r, k):
    from block_sparse_long_09_amd.pipeline import DecodePath
    print("[case] noalloc decode", B, L, Hq, Hkv, r, k, flush=True)
    Kc = dev(gen.normal(seed, 2, (B, L, Hkv, 128)))
    Vc = dev(gen.normal(seed, 3, (B, L, Hkv, 128)))
    Q = dev(gen.normal(seed, 1, (B, Hq, 128)))
    iq = dev(gen.normal(seed, 4, (B, Hi, 64)))
    ik = torch.stack([dev(gen.idx_keys(seed, b, L, 0, L, 64, 4096, r)) for b in range(B)])
    cmp = torch.empty((B, L // r, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(ik, cmp, r, 0, L // r)
    kvl = torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    path = DecodePath(Hq, Hkv, Hi, B, L, r=r, k=k)
    path.select(iq, cmp, kvl - 1)
    sel = path.sel[:, 0].contiguous()
    cnt = path.cnt[:, 0].contiguous()
    desc = qsa.attn_desc(Hq, Hkv)
    ws = qsa.workspace(qsa.qsa_sparse_attn_workspace_size(desc, B, 1, k, r))
    out_ws = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse_ws = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out_na = torch.full((B, Hq, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_na = torch.full((B, Hq), 7.0, dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_decode(desc, r, Q, Kc, Vc, kvl, sel, cnt, out_ws, lse_ws, ws)
    qsa.qsa_sparse_attn_decode_noalloc(desc, r, Q, Kc, Vc, kvl, sel, cnt, out_na, lse_na)
    torch.cuda.synchronize()
    assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16))
    assert torch.equal(lse_ws, lse_na)
    assert torch.isfinite(out_na.float()).all()


def test_noalloc_decode_matches_workspace_call_twice(qsa):
    # the first call is the larger one: the second must not see its leftovers
    _case(qsa, 91, B=4, L=20000, kv_len=[20000, 19999, 7777, 4100], Hq=32, Hkv=4, Hi=8, r=4, k=512)
    _case(qsa, 92, B=2, L=3000, kv_len=[3000, 1234], Hq=16, Hkv=2, Hi=8, r=4, k=128)


def test_noalloc_decode_refuses_beyond_scratch(qsa):
    # 64 query heads over 4 sequences: the split partial results
    # (4 x 64 splits x 64 heads x 128 fp32, plus (m, l)) exceed 8 MiB
    desc = qsa.attn_desc(64, 4)
    need = qsa.qsa_sparse_attn_workspace_size(desc, 4, 1, 512, 4)
    assert need > 8 << 20
    B, L = 4, 4096
    Kc = torch.zeros((B, L, 4, 128), dtype=torch.bfloat16, device="cuda")
    Q = torch.zeros((B, 64, 128), dtype=torch.bfloat16, device="cuda")
    kvl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    sel = torch.zeros((B, 512), dtype=torch.int32, device="cuda")
    cnt = torch.ones((B,), dtype=torch.int32, device="cuda")
    out = torch.empty((B, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_sparse_attn_decode_noalloc(desc, 4, Q, Kc, Kc, kvl, sel, cnt, out)
    assert e.value.status == 2 and "scratch" in str(e.value)


def test_noalloc_decode_step_under_graph_capture(qsa):
    # the case the allocation-free call is for: a whole decode step (the
    # indexer on a caller workspace allocated beforehand, then the attention
    # on the library's scratch) captured once as a HIP graph and replayed;
    # every replay, with eager calls and synchronisations in between, gives
    # the eager step's bits
    from block_sparse_long_09_amd.pipeline import DecodePath
    B, L, Hq, Hkv, Hi, r, k, seed = 3, 9000, 32, 4, 8, 4, 256, 93
    print("[case] noalloc decode step under graph capture", flush=True)
    Kc = dev(gen.normal(seed, 2, (B, L, Hkv, 128)))
    Vc = dev(gen.normal(seed, 3, (B, L, Hkv, 128)))
    Q = dev(gen.normal(seed, 1, (B, Hq, 128)))
    iq = dev(gen.normal(seed, 4, (B, Hi, 64)))
    ik = torch.stack([dev(gen.idx_keys(seed, b, L, 0, L, 64, 4096, r)) for b in range(B)])
    cmp = torch.empty((B, L // r, 64), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(ik, cmp, r, 0, L // r)
    kvl = torch.tensor([L, 5001, 17], dtype=torch.int32, device="cuda")
    qpos = kvl - 1
    path = DecodePath(Hq, Hkv, Hi, B, L, r=r, k=k)
    desc = qsa.attn_desc(Hq, Hkv)
    sel = torch.empty((B, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def step():
        path.select(iq, cmp, qpos)
        sel.copy_(path.sel[:, 0])
        cnt.copy_(path.cnt[:, 0])
        qsa.qsa_sparse_attn_decode_noalloc(desc, r, Q, Kc, Vc, kvl, sel, cnt, out, lse)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_sel = out.clone(), lse.clone(), sel.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(4):
        out.fill_(7.0)
        lse.fill_(7.0)
        sel.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        step()  # eager work between the replays
        torch.cuda.synchronize()
