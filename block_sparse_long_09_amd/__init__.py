"""QSA (Qwen Sparse Attention) hot path on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libqsa.so`` (C ABI in ``include/qsa.h`` and
``include/qsa_bench.h``). Functions carry the C names and only marshal
arguments: torch tensors in device memory become raw pointers, the current
torch stream becomes the ``hipStream_t``, and a non-OK status raises
``QsaError``. Every step of the path runs in the library's HIP kernels; there
is no fallback: if the library is missing, importing this package fails.
"""
import ctypes
import math
import os

import torch  # loads the HIP runtime that libqsa.so then binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python block_sparse_long_09_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


class IndexDesc(ctypes.Structure):
    _fields_ = [("block_size", _i32), ("top_k_blocks", _i32), ("n_idx_heads", _i32),
                ("idx_head_dim", _i32), ("idx_head_weight", _f32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32), ("softmax_scale", _f32)]


class GdnDesc(ctypes.Structure):
    _fields_ = [("n_qk_heads", _i32), ("n_v_heads", _i32), ("key_dim", _i32), ("value_dim", _i32),
                ("scale", _f32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_launches", _i32), ("grid", (ctypes.c_uint32 * 3) * 3), ("block", ctypes.c_uint32 * 3),
                ("lds", ctypes.c_uint64 * 3), ("max_int32_value", _i64), ("max_offset", _i64),
                ("workspace_bytes", ctypes.c_uint64), ("splits", _i32), ("cap", _i32), ("fits", _i32),
                ("sample_stride", _i32)]


_PI, _PA, _PG = ctypes.POINTER(IndexDesc), ctypes.POINTER(AttnDesc), ctypes.POINTER(GdnDesc)


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("qsa_compress_keys", ctypes.c_int, [_vp, _i64, _i32, _i32, _i32, _i64, _i64, _vp, _i64, _vp])
_sig("qsa_index_topk_workspace_size", _sz, [_PI, _i32, _i32, _i64])
_sig("qsa_index_topk", ctypes.c_int, [_PI, _vp, _vp, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _sz, _vp])
_sig("qsa_sparse_attn_workspace_size", _sz, [_PA, _i32, _i32, _i32, _i32])
_sig("qsa_sparse_attn_prefill", ctypes.c_int,
     [_PA, _i32, _i32, _vp, _vp, _vp, _i64, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_sig("qsa_sparse_attn_decode", ctypes.c_int,
     [_PA, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_sig("qsa_sparse_attn_decode_noalloc", ctypes.c_int,
     [_PA, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp])
_sig("qsa_dense_attn_workspace_size", _sz, [_PA, _i32, _i32, _i64])
_sig("qsa_dense_attn_prefill", ctypes.c_int, [_PA, _vp, _vp, _vp, _i64, _i32, _i64, _vp, _vp, _vp, _sz, _vp])
_sig("qsa_dense_attn_decode", ctypes.c_int, [_PA, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _sz, _vp])
_sig("qsa_index_topk_varlen_workspace_size", _sz, [_PI, _i32, _i32, _i64])
_sig("qsa_index_topk_varlen", ctypes.c_int,
     [_PI, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i64, _vp, _vp, _vp, _sz, _vp])
_sig("qsa_sparse_attn_prefill_paged", ctypes.c_int,
     [_PA, _i32, _i32, _vp, _vp, _vp, _i32, _i64, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp])
_sig("qsa_distill_kl_workspace_size", _sz, [_PA, _i32])
_sig("qsa_distill_kl_prefill", ctypes.c_int, [_PA, _PI, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _vp, _vp, _sz, _vp])
_sig("qsa_gdn_prefill_workspace_size", _sz, [_PG, _i32, _i64])
_sig("qsa_gdn_prefill", ctypes.c_int, [_PG, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _sz, _vp])
_sig("qsa_gdn_decode", ctypes.c_int, [_PG, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp])
_sig("qsa_index_topk_plan_info", ctypes.c_int, [_PI, _i32, _i32, _i64, _i32, ctypes.POINTER(PlanInfo)])
_sig("qsa_sparse_attn_plan_info", ctypes.c_int, [_PA, _i32, _i32, _i32, _i32, ctypes.POINTER(PlanInfo)])
_sig("qsa_status_string", ctypes.c_char_p, [ctypes.c_int])
_sig("qsa_last_error_message", ctypes.c_char_p, [])
_sig("qsa_abi_version", ctypes.c_int, [])

#: every symbol the C headers declare
EXPORTS = (
    "qsa_compress_keys", "qsa_index_topk_workspace_size", "qsa_index_topk",
    "qsa_sparse_attn_workspace_size", "qsa_sparse_attn_prefill", "qsa_sparse_attn_decode",
    "qsa_sparse_attn_decode_noalloc",
    "qsa_status_string", "qsa_last_error_message", "qsa_abi_version",
    "qsa_dense_attn_workspace_size", "qsa_dense_attn_prefill", "qsa_dense_attn_decode",
    "qsa_index_topk_varlen_workspace_size", "qsa_index_topk_varlen", "qsa_sparse_attn_prefill_paged",
    "qsa_distill_kl_workspace_size", "qsa_distill_kl_prefill",
    "qsa_gdn_prefill_workspace_size", "qsa_gdn_prefill", "qsa_gdn_decode",
    "qsa_index_topk_plan_info", "qsa_sparse_attn_plan_info",
)


class QsaError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{_lib.qsa_status_string(status).decode()}: {message}")


def _check(status):
    if status != 0:
        raise QsaError(status, _lib.qsa_last_error_message().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else stream


def _bf16(t, name):
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")
    return _ptr(t)


def _i32t(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _ptr(t)


def index_desc(block_size, top_k_blocks, n_idx_heads, idx_head_dim=64, idx_head_weight=None):
    w = 1.0 / n_idx_heads if idx_head_weight is None else idx_head_weight
    return IndexDesc(block_size, top_k_blocks, n_idx_heads, idx_head_dim, w)


def attn_desc(n_q_heads, n_kv_heads, head_dim=128, softmax_scale=None):
    s = head_dim ** -0.5 if softmax_scale is None else softmax_scale
    return AttnDesc(n_q_heads, n_kv_heads, head_dim, s)


def abi_version():
    return _lib.qsa_abi_version()


# ----------------------------------------------------------------- method --
def qsa_compress_keys(idx_k, cmp_k, block_size, first_block, n_blocks, stream=None):
    """idx_k [B, L, 64] (or [L, 64]) -> cmp_k [B, N, 64] (or [N, 64]), blocks
    [first_block, first_block + n_blocks) of every row."""
    if idx_k.dim() == 2:
        idx_k, cmp_k = idx_k[None], cmp_k[None]
    B, _, d = idx_k.shape
    _check(_lib.qsa_compress_keys(_bf16(idx_k, "idx_k"), idx_k.stride(0), B, d, block_size, first_block,
                                  n_blocks, _bf16(cmp_k, "cmp_k"), cmp_k.stride(0), _stream(stream)))


def qsa_index_topk_workspace_size(desc, batch, n_q, max_q_end):
    return _lib.qsa_index_topk_workspace_size(ctypes.byref(desc), batch, n_q, max_q_end)


def qsa_index_topk(desc, idx_q, cmp_k, q_pos0, max_q_end, sel_blocks, sel_count, workspace, stream=None):
    """idx_q [B, n_q, H_i, 64]; cmp_k [B, N, 64]; q_pos0 int32 [B] (device);
    sel_blocks int32 [B, n_q, k]; sel_count int32 [B, n_q]; workspace uint8."""
    if idx_q.dim() == 3:
        idx_q = idx_q[None]
    if cmp_k.dim() == 2:
        cmp_k = cmp_k[None]
    B, n_q = idx_q.shape[0], idx_q.shape[1]
    ws = _ptr(workspace) if workspace is not None and workspace.numel() else None
    nbytes = workspace.numel() * workspace.element_size() if ws else 0
    _check(_lib.qsa_index_topk(ctypes.byref(desc), _bf16(idx_q, "idx_q"), _bf16(cmp_k, "cmp_k"), cmp_k.stride(0),
                               _i32t(q_pos0, "q_pos0"), max_q_end, B, n_q, _i32t(sel_blocks, "sel_blocks"),
                               _i32t(sel_count, "sel_count"), ws, nbytes, _stream(stream)))


def qsa_index_topk_varlen_workspace_size(desc, batch, max_q, max_q_end):
    return _lib.qsa_index_topk_varlen_workspace_size(ctypes.byref(desc), batch, max_q, max_q_end)


def qsa_index_topk_varlen(desc, idx_q, cmp_k, cu_q, q_pos0, max_q, max_q_end, sel_blocks, sel_count, workspace,
                          stream=None):
    """Packed rows: idx_q [total_q, H_i, 64]; cmp_k [B, N, 64]; cu_q int32 [B + 1] and q_pos0
    int32 [B] (device); sel_blocks int32 [total_q, k]; sel_count int32 [total_q]."""
    if cmp_k.dim() == 2:
        cmp_k = cmp_k[None]
    B = q_pos0.shape[0]
    ws = _ptr(workspace) if workspace is not None and workspace.numel() else None
    nbytes = workspace.numel() * workspace.element_size() if ws else 0
    _check(_lib.qsa_index_topk_varlen(ctypes.byref(desc), _bf16(idx_q, "idx_q"), _bf16(cmp_k, "cmp_k"),
                                      cmp_k.stride(0), _i32t(cu_q, "cu_q"), _i32t(q_pos0, "q_pos0"), B, max_q,
                                      max_q_end, _i32t(sel_blocks, "sel_blocks"), _i32t(sel_count, "sel_count"),
                                      ws, nbytes, _stream(stream)))


def qsa_sparse_attn_prefill_paged(desc, block_size, q, k_pages, v_pages, page_table, cu_q, q_pos0, sel_blocks,
                                  sel_count, out, lse=None, stream=None):
    """Packed rows over a paged pool: q, out [total_q, Hq, D]; k_pages, v_pages
    [n_pages, page_size, Hkv, D]; page_table int32 [B, max_pages]; cu_q int32 [B + 1];
    q_pos0 int32 [B]; sel_blocks [total_q, top_k]; lse [total_q, Hq] or None."""
    n_pages, page_size = k_pages.shape[0], k_pages.shape[1]
    B, max_pages = page_table.shape
    _check(_lib.qsa_sparse_attn_prefill_paged(
        ctypes.byref(desc), block_size, sel_blocks.shape[-1], _bf16(q, "q"), _bf16(k_pages, "k_pages"),
        _bf16(v_pages, "v_pages"), page_size, n_pages, _i32t(page_table, "page_table"), max_pages,
        _i32t(cu_q, "cu_q"), _i32t(q_pos0, "q_pos0"), B, q.shape[0], _i32t(sel_blocks, "sel_blocks"),
        _i32t(sel_count, "sel_count"), _bf16(out, "out"), _ptr(lse) if lse is not None else None,
        _stream(stream)))


def qsa_distill_kl_workspace_size(adesc, n_q):
    return _lib.qsa_distill_kl_workspace_size(ctypes.byref(adesc), n_q)


def qsa_distill_kl_prefill(adesc, idesc, q, k, idx_q, cmp_k, q_pos0, kl, workspace, stream=None):
    """q [n_q, Hq, D]; k [kv_len, Hkv, D]; idx_q [n_q, 8, 64]; cmp_k [blocks, 64]; kl float32 [n_q]."""
    n_q = q.shape[0]
    ws = _ptr(workspace)
    nbytes = workspace.numel() * workspace.element_size()
    if kl.dtype != torch.float32:
        raise TypeError("kl must be float32")
    _check(_lib.qsa_distill_kl_prefill(ctypes.byref(adesc), ctypes.byref(idesc), _bf16(q, "q"), _bf16(k, "k"),
                                       _bf16(idx_q, "idx_q"), _bf16(cmp_k, "cmp_k"), q_pos0, n_q, k.shape[0],
                                       _ptr(kl), ws, nbytes, _stream(stream)))


def qsa_sparse_attn_workspace_size(desc, batch, n_q, top_k_blocks, block_size):
    return _lib.qsa_sparse_attn_workspace_size(ctypes.byref(desc), batch, n_q, top_k_blocks, block_size)


def qsa_sparse_attn_prefill(desc, block_size, q, k, v, q_pos0, sel_blocks, sel_count, out, lse=None,
                            workspace=None, stream=None):
    """q [n_q, Hq, D]; k, v [kv_len, Hkv, D]; sel_blocks [n_q, top_k]; out [n_q, Hq, D]; lse [n_q, Hq]."""
    n_q = q.shape[0]
    top_k = sel_blocks.shape[-1]
    ws = _ptr(workspace) if workspace is not None and workspace.numel() else None
    nbytes = workspace.numel() * workspace.element_size() if ws else 0
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _check(_lib.qsa_sparse_attn_prefill(ctypes.byref(desc), block_size, top_k, _bf16(q, "q"), _bf16(k, "k"),
                                        _bf16(v, "v"), q_pos0, n_q, k.shape[0], _i32t(sel_blocks, "sel_blocks"),
                                        _i32t(sel_count, "sel_count"), _bf16(out, "out"), _ptr(lse), ws, nbytes,
                                        _stream(stream)))


def qsa_sparse_attn_decode(desc, block_size, q, k_cache, v_cache, kv_len, sel_blocks, sel_count, out, lse=None,
                           workspace=None, stream=None):
    """q [B, Hq, D]; caches [B, max_len, Hkv, D]; kv_len int32 [B] (device);
    sel_blocks [B, top_k]; out [B, Hq, D]; lse [B, Hq]."""
    B = q.shape[0]
    top_k = sel_blocks.shape[-1]
    ws = _ptr(workspace) if workspace is not None and workspace.numel() else None
    nbytes = workspace.numel() * workspace.element_size() if ws else 0
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _check(_lib.qsa_sparse_attn_decode(ctypes.byref(desc), block_size, top_k, _bf16(q, "q"),
                                       _bf16(k_cache, "k_cache"), _bf16(v_cache, "v_cache"), k_cache.shape[1],
                                       _i32t(kv_len, "kv_len"), B, _i32t(sel_blocks, "sel_blocks"),
                                       _i32t(sel_count, "sel_count"), _bf16(out, "out"), _ptr(lse), ws, nbytes,
                                       _stream(stream)))


def qsa_sparse_attn_decode_noalloc(desc, block_size, q, k_cache, v_cache, kv_len, sel_blocks, sel_count, out,
                                   lse=None, stream=None):
    """qsa_sparse_attn_decode without a workspace (the library's scratch on the
    device; calls that overlap on one device race)."""
    B = q.shape[0]
    top_k = sel_blocks.shape[-1]
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _check(_lib.qsa_sparse_attn_decode_noalloc(ctypes.byref(desc), block_size, top_k, _bf16(q, "q"),
                                               _bf16(k_cache, "k_cache"), _bf16(v_cache, "v_cache"),
                                               k_cache.shape[1], _i32t(kv_len, "kv_len"), B,
                                               _i32t(sel_blocks, "sel_blocks"), _i32t(sel_count, "sel_count"),
                                               _bf16(out, "out"), _ptr(lse), _stream(stream)))


# ------------------------------------------------------------- comparator --
def qsa_dense_attn_workspace_size(desc, batch, n_q, max_len):
    return _lib.qsa_dense_attn_workspace_size(ctypes.byref(desc), batch, n_q, max_len)


def qsa_dense_attn_prefill(desc, q, k, v, q_pos0, out, lse=None, workspace=None, stream=None):
    ws = _ptr(workspace) if workspace is not None and workspace.numel() else None
    nbytes = workspace.numel() * workspace.element_size() if ws else 0
    _check(_lib.qsa_dense_attn_prefill(ctypes.byref(desc), _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), q_pos0,
                                       q.shape[0], k.shape[0], _bf16(out, "out"), _ptr(lse), ws, nbytes,
                                       _stream(stream)))


def qsa_dense_attn_decode(desc, q, k_cache, v_cache, kv_len, out, lse=None, workspace=None, stream=None):
    ws = _ptr(workspace) if workspace is not None and workspace.numel() else None
    nbytes = workspace.numel() * workspace.element_size() if ws else 0
    _check(_lib.qsa_dense_attn_decode(ctypes.byref(desc), _bf16(q, "q"), _bf16(k_cache, "k_cache"),
                                      _bf16(v_cache, "v_cache"), k_cache.shape[1], _i32t(kv_len, "kv_len"),
                                      q.shape[0], _bf16(out, "out"), _ptr(lse), ws, nbytes, _stream(stream)))


# ------------------------------------------------- allocation conveniences --
def workspace(nbytes, device="cuda"):
    """A caller-owned scratch buffer (uint8) of at least nbytes."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def softmax_scale(head_dim=128):
    return 1.0 / math.sqrt(head_dim)


def gdn_desc(n_qk_heads, n_v_heads, key_dim=128, value_dim=128, scale=None):
    s = key_dim ** -0.5 if scale is None else scale
    return GdnDesc(n_qk_heads, n_v_heads, key_dim, value_dim, s)


def _f32t(t, name):
    if t is None:
        return None
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _ptr(t)


def qsa_gdn_prefill_workspace_size(desc, batch, seq_len):
    return _lib.qsa_gdn_prefill_workspace_size(ctypes.byref(desc), batch, seq_len)


def qsa_gdn_prefill(desc, q, k, v, g, beta, out, initial_state=None, final_state=None, workspace=None,
                    stream=None):
    """q, k [B, T, Hqk, dk]; v, out [B, T, Hv, dv] bf16; g, beta [B, T, Hv] fp32;
    states [B, Hv, dv, dk] fp32 (optional)."""
    B, T = v.shape[0], v.shape[1]
    ws = _ptr(workspace) if workspace is not None and workspace.numel() else None
    nbytes = workspace.numel() * workspace.element_size() if ws else 0
    _check(_lib.qsa_gdn_prefill(ctypes.byref(desc), _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _f32t(g, "g"),
                                _f32t(beta, "beta"), _f32t(initial_state, "initial_state"), B, T,
                                _bf16(out, "out"), _f32t(final_state, "final_state"), ws, nbytes, _stream(stream)))


def qsa_gdn_decode(desc, q, k, v, g, beta, state, out, stream=None):
    """q, k [B, Hqk, dk]; v, out [B, Hv, dv] bf16; g, beta [B, Hv] fp32; state [B, Hv, dv, dk] fp32 (in place)."""
    _check(_lib.qsa_gdn_decode(ctypes.byref(desc), _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _f32t(g, "g"),
                               _f32t(beta, "beta"), _f32t(state, "state"), v.shape[0], _bf16(out, "out"),
                               _stream(stream)))


def qsa_index_topk_plan_info(desc, batch, n_q, max_q_end, packed=False):
    """The launch plan qsa_index_topk (or, packed, qsa_index_topk_varlen) would
    use for these sizes (host only)."""
    info = PlanInfo()
    _check(_lib.qsa_index_topk_plan_info(ctypes.byref(desc), batch, n_q, max_q_end, int(bool(packed)),
                                         ctypes.byref(info)))
    return info


def qsa_sparse_attn_plan_info(desc, rows, top_k_blocks, block_size, decode=False):
    """The launch plan of the sparse attention calls for these sizes (host only)."""
    info = PlanInfo()
    _check(_lib.qsa_sparse_attn_plan_info(ctypes.byref(desc), rows, top_k_blocks, block_size, int(bool(decode)),
                                          ctypes.byref(info)))
    return info
