"""Launch plans of every benchmarked workload, checked on the host: each grid,
workgroup and LDS size within the device's limits, each value a kernel holds
in a 32-bit int below 2^31, each workspace offset far below 2^63, and the
workspace the plan lays out equal to what the size query returns.

A 32-bit per-(query, split) buffer offset is the kind of mistake these checks
are about: buffers of 32768 queries x several splits x 2048 entries x 8 B pass
2^31 bytes; the kernels form those offsets in 64 bits, and the plan reports the
largest one (checked below on a batch whose buffers pass 2^31 bytes)."""
import pytest

from gen.configs import CONFIGS, PAGED

MAX_GRID_X, MAX_GRID_YZ, MAX_LDS = 2 ** 31 - 1, 65535, 160 * 1024


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    return q


def _within_limits(info):
    assert info.fits == 1
    assert 1 <= info.n_launches <= 3
    for i in range(info.n_launches):
        x, y, z = info.grid[i]
        assert 1 <= x <= MAX_GRID_X and 1 <= y <= MAX_GRID_YZ and 1 <= z <= MAX_GRID_YZ, (i, x, y, z)
        assert 1 <= info.block[i] <= 1024
        assert info.lds[i] <= MAX_LDS, (i, info.lds[i])
    assert 0 <= info.max_int32_value < 2 ** 31
    assert 0 <= info.max_offset < 2 ** 62


def _index_cases():
    for name, W in CONFIGS.items():
        if W.mode == "prefill":
            chunk = W.chunk or W.n_q
            # every chunk of a chunked prefill: the last one has the most candidates
            yield name, W, 1, chunk, W.q_pos0 + W.n_q, W.Hi
        else:
            yield name, W, W.batch, 1, W.L, W.Hi


@pytest.mark.parametrize("name,W,batch,n_q,end,Hi", list(_index_cases()), ids=lambda v: v if isinstance(v, str) else "")
def test_index_plan_fits(qsa, name, W, batch, n_q, end, Hi):
    d = qsa.index_desc(W.r, W.k, Hi, W.di)
    info = qsa.qsa_index_topk_plan_info(d, batch, n_q, end)
    _within_limits(info)
    assert info.workspace_bytes == qsa.qsa_index_topk_workspace_size(d, batch, n_q, end)
    # the buffers of the many-query prefill indexer (or the decode score rows)
    # are addressed with 64-bit offsets: the largest must be what the sizes give
    if n_q > 1:
        assert info.max_offset == batch * n_q * info.splits * info.cap


def test_index_plan_buffers_past_2_31_bytes(qsa):
    # 16 sequences of the 32K prefill shape: the candidate buffers span more
    # than 2^31 bytes, which only 64-bit offsets address; the plan still fits
    W = CONFIGS["c2"]
    info = qsa.qsa_index_topk_plan_info(qsa.index_desc(W.r, W.k, W.Hi, W.di), 16, W.n_q, W.L)
    _within_limits(info)
    assert info.max_offset * 8 > 2 ** 31


def test_index_plan_paged_batch_fits(qsa):
    W = PAGED["c6"]
    d = qsa.index_desc(W.r, W.k, W.Hi, W.di)
    end = max(W.lengths)
    info = qsa.qsa_index_topk_plan_info(d, W.batch, max(W.new), end, packed=True)
    _within_limits(info)
    assert info.workspace_bytes == qsa.qsa_index_topk_varlen_workspace_size(d, W.batch, max(W.new), end)


@pytest.mark.parametrize("name", list(CONFIGS) + ["c6"])
def test_attention_plan_fits(qsa, name):
    if name == "c6":
        W = PAGED[name]
        rows, decode = sum(W.new), False
    else:
        W = CONFIGS[name]
        rows, decode = (W.chunk or W.n_q, False) if W.mode == "prefill" else (W.batch, True)
    d = qsa.attn_desc(W.Hq, W.Hkv, W.D)
    info = qsa.qsa_sparse_attn_plan_info(d, rows, W.k, W.r, decode)
    _within_limits(info)
    if decode:
        assert info.workspace_bytes == qsa.qsa_sparse_attn_workspace_size(d, rows, 1, W.k, W.r)


def test_plans_refuse_what_does_not_fit(qsa):
    # 65535 sequences x 2^31 - 1 positions: the decode list merge would stage
    # more than the device's LDS, so the indexer falls back to the prefill
    # kernels, whose query count then overflows nothing but whose select grid
    # is batch x n_q; a plan either fits or is reported as not fitting
    d = qsa.index_desc(4, 512, 8)
    info = qsa.qsa_index_topk_plan_info(d, 65535, 40000, 2 ** 31 - 1)
    assert info.fits in (0, 1)
    if info.fits == 0:
        assert info.max_int32_value >= 2 ** 31 or any(
            info.grid[i][0] > MAX_GRID_X or info.lds[i] > MAX_LDS for i in range(info.n_launches))


@pytest.mark.parametrize("k,expect", [(512, 16), (1024, 32), (309, 16), (308, 0), (256, 0), (64, 0)])
def test_index_plan_threshold_sample_stride(qsa, k, expect):
    # the many-query indexer seeds its thresholds from every rho-th key tile:
    # rho is the smallest power of two with 2.5 (k - 1) / rho <= 96 sample
    # scores to rank, and the sample is taken only when rho >= 16 (at most
    # 1/16 more scoring); so the seed's rank m = 2.5 (k - 1) / rho lies in
    # (48, 96] whenever it is used
    d = qsa.index_desc(4, k, 8, 64)
    info = qsa.qsa_index_topk_plan_info(d, 1, 16384, 1 << 20)
    assert info.sample_stride == expect
    if expect:
        assert 5 * (k - 1) <= 192 * expect and 5 * (k - 1) > 96 * expect
    # decode (one query per sequence), the few-query kernel and the
    # many-query kernel at one indexer head take no sample
    assert qsa.qsa_index_topk_plan_info(d, 4, 1, 1 << 20).sample_stride == 0
    assert qsa.qsa_index_topk_plan_info(d, 1, 32, 1 << 20).sample_stride == 0
    d1 = qsa.index_desc(4, k, 1, 64)
    assert qsa.qsa_index_topk_plan_info(d1, 1, 16384, 1 << 20).sample_stride == 0
