"""The C ABI on the host: the library loads, exports every declared entry
point, and rejects bad arguments before touching any device memory."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("qsa.h", "qsa_bench.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", src))
    return names


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    return q


def test_exports_every_declared_symbol(qsa):
    declared = _declared()
    assert len(declared) >= 12
    assert declared == set(qsa.EXPORTS)
    lib = ctypes.CDLL(qsa.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert qsa.abi_version() == 2


def _status(qsa, code):
    return qsa._lib.qsa_status_string(code).decode()


FAKE = 0x10000  # a 16-byte-aligned address never dereferenced by these calls


def test_compress_rejects_bad_arguments(qsa):
    L = qsa._lib
    assert L.qsa_compress_keys(FAKE, 0, 1, 32, 4, 0, 10, FAKE, 0, None) == 2  # d != 64
    assert L.qsa_compress_keys(FAKE, 0, 1, 64, 3, 0, 10, FAKE, 0, None) == 2  # r not a power of two
    assert L.qsa_compress_keys(None, 0, 1, 64, 4, 0, 10, FAKE, 0, None) == 1
    assert L.qsa_compress_keys(FAKE + 2, 0, 1, 64, 4, 0, 10, FAKE, 0, None) == 3
    assert L.qsa_compress_keys(FAKE, 100, 2, 64, 4, 0, 10, FAKE, 640, None) == 1  # stride too small
    assert L.qsa_compress_keys(FAKE, 0, 1, 64, 4, 0, 0, FAKE, 0, None) == 0  # nothing to do


def test_index_topk_rejects_bad_arguments(qsa):
    L = qsa._lib
    d = qsa.index_desc(4, 512, 8)
    ws = qsa.qsa_index_topk_workspace_size(d, 1, 4096, 1 << 20)
    assert ws > 0
    args = lambda **kw: dict(dict(desc=d, iq=FAKE, ck=FAKE, st=0, pos=FAKE, end=4096, b=1, nq=4096,
                                  sel=FAKE, cnt=FAKE, ws=FAKE, wsb=ws), **kw)

    def call(a):
        return L.qsa_index_topk(ctypes.byref(a["desc"]), a["iq"], a["ck"], a["st"], a["pos"], a["end"], a["b"],
                                a["nq"], a["sel"], a["cnt"], a["ws"], a["wsb"], None)
    small = qsa.qsa_index_topk_workspace_size(d, 1, 4096, 4096)
    assert call(args(wsb=small - 1)) == 4
    assert call(args(end=100)) == 1  # max_q_end < n_q
    assert call(args(iq=None)) == 1
    assert call(args(iq=FAKE + 8)) == 3
    assert call(args(desc=qsa.index_desc(4, 2048, 8))) == 2  # k > 1024
    assert call(args(desc=qsa.index_desc(4, 512, 3))) == 2
    assert call(args(desc=qsa.index_desc(4, 512, 8, 32))) == 2
    assert call(args(desc=qsa.index_desc(4, 512, 8, idx_head_weight=-1.0))) == 1
    assert call(args(b=2, st=64)) == 1  # batch stride does not cover the blocks
    assert call(args(nq=0)) == 0
    msg = L.qsa_last_error_message()
    assert isinstance(msg, bytes)


def test_attention_rejects_bad_arguments(qsa):
    L = qsa._lib
    a = qsa.attn_desc(32, 4)
    p = lambda desc, **kw: L.qsa_sparse_attn_prefill(ctypes.byref(desc), kw.get("r", 4), kw.get("k", 512), FAKE,
                                                     FAKE, FAKE, kw.get("q0", 0), kw.get("nq", 16),
                                                     kw.get("L", 16), FAKE, FAKE, FAKE, None, None, 0, None)
    assert p(qsa.attn_desc(32, 4, 64)) == 2
    assert p(qsa.attn_desc(32, 8)) == 2
    assert p(qsa.attn_desc(30, 4)) == 1
    assert p(qsa.attn_desc(128, 4)) == 2  # group of 32 heads
    assert p(a, r=5) == 2
    assert p(a, L=10) == 1  # q_pos0 + n_q > kv_len
    assert p(a, nq=0) == 0
    dec = qsa.qsa_sparse_attn_workspace_size(a, 64, 1, 512, 4)
    assert dec > 0
    r = L.qsa_sparse_attn_decode(ctypes.byref(a), 4, 512, FAKE, FAKE, FAKE, 1024, FAKE, 64, FAKE, FAKE, FAKE,
                                 None, FAKE, dec - 1, None)
    assert r == 4
    assert qsa.qsa_dense_attn_workspace_size(a, 4, 1, 1 << 20) > 0


def test_status_strings(qsa):
    names = [_status(qsa, i) for i in range(6)]
    assert names == ["QSA_OK", "QSA_ERR_INVALID_ARGUMENT", "QSA_ERR_UNSUPPORTED", "QSA_ERR_MISALIGNED",
                     "QSA_ERR_WORKSPACE_TOO_SMALL", "QSA_ERR_HIP"]


def test_workspace_sizes_grow_with_work(qsa):
    d = qsa.index_desc(4, 512, 8)
    a = qsa.qsa_index_topk_workspace_size(d, 1, 1024, 1 << 16)
    b = qsa.qsa_index_topk_workspace_size(d, 1, 4096, 1 << 16)
    c = qsa.qsa_index_topk_workspace_size(d, 4, 4096, 1 << 16)
    assert 0 < a <= b <= c
    assert qsa.qsa_index_topk_workspace_size(d, 1, 4096, 100) == 0  # max_q_end < n_q: invalid


def test_varlen_and_paged_reject_bad_arguments(qsa):
    L = qsa._lib
    d = qsa.index_desc(4, 512, 8)
    ws = qsa.qsa_index_topk_varlen_workspace_size(d, 8, 4096, 1 << 20)
    assert ws > 0

    def iv(**kw):
        a = dict(iq=FAKE, ck=FAKE, st=1 << 24, cu=FAKE, pos=FAKE, b=8, mq=4096, end=1 << 20, sel=FAKE, cnt=FAKE,
                 ws=FAKE, wsb=ws)
        a.update(kw)
        return L.qsa_index_topk_varlen(ctypes.byref(d), a["iq"], a["ck"], a["st"], a["cu"], a["pos"], a["b"],
                                       a["mq"], a["end"], a["sel"], a["cnt"], a["ws"], a["wsb"], None)
    assert iv(cu=None) == 1
    assert iv(wsb=ws - 1) == 4
    assert iv(end=100) == 1            # max_q_end < max_q
    assert iv(st=64) == 1              # per-sequence block keys do not fit the stride
    assert iv(cu=FAKE + 2) == 3
    assert iv(mq=0) == 0
    a = qsa.attn_desc(32, 4)

    def pg(**kw):
        x = dict(r=4, k=512, page=256, npages=100, tab=FAKE, maxp=16, cu=FAKE, pos=FAKE, b=2, tq=10)
        x.update(kw)
        return L.qsa_sparse_attn_prefill_paged(ctypes.byref(a), x["r"], x["k"], FAKE, FAKE, FAKE, x["page"],
                                               x["npages"], x["tab"], x["maxp"], x["cu"], x["pos"], x["b"],
                                               x["tq"], FAKE, FAKE, FAKE, None, None)
    assert pg(page=100) == 1           # not a power of two
    assert pg(page=2, r=4) == 1        # a block would straddle pages
    assert pg(npages=1 << 30) == 1     # pool beyond 2^31 tokens
    assert pg(tab=None) == 1
    assert pg(k=2048) == 2
    assert pg(tq=0) == 0


def test_gdn_rejects_bad_arguments(qsa):
    L = qsa._lib
    d = qsa.gdn_desc(16, 32)
    ws = qsa.qsa_gdn_prefill_workspace_size(d, 2, 1000)
    assert ws > 0 and qsa.qsa_gdn_prefill_workspace_size(d, 2, 2000) > ws

    def pf(desc=d, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, s0=None, B=2, T=1000, out=FAKE, sf=None, ws=FAKE, wsb=ws)
        a.update(kw)
        return L.qsa_gdn_prefill(ctypes.byref(desc), a["q"], a["k"], a["v"], a["g"], a["b"], a["s0"], a["B"], a["T"],
                                 a["out"], a["sf"], a["ws"], a["wsb"], None)
    assert pf(wsb=ws - 1) == 4
    assert pf(v=None) == 1
    assert pf(q=FAKE + 8) == 3
    assert pf(s0=FAKE + 2) == 3
    assert pf(T=-1) == 1
    assert pf(desc=qsa.gdn_desc(16, 24)) == 1      # value heads not a multiple of key heads
    assert pf(desc=qsa.gdn_desc(16, 32, 64, 64)) == 2
    assert pf(B=0) == 0
    assert pf(T=0, q=None, k=None, v=None, g=None, b=None, out=None, ws=None, wsb=0) == 0

    def dc(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, s=FAKE, B=4, out=FAKE)
        a.update(kw)
        return L.qsa_gdn_decode(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["s"], a["B"], a["out"],
                                None)
    assert dc(s=None) == 1
    assert dc(s=FAKE + 4) == 3
    assert dc(B=-1) == 1
    assert dc(B=0) == 0
