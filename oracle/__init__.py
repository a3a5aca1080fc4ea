"""CPU oracle for QSA — TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``qsa_oracle.c`` (plain C, double precision, OpenMP
over queries). Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU library never does, and the
two share no code. See ``qsa_oracle.c`` for the method, its sources and the
readings taken where the sources are silent.
"""
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build():
    """Compile the oracle library in place (gcc; no -ffast-math, no FMA contraction)."""
    subprocess.check_call(["gcc", *CFLAGS, "-o", _SO + ".tmp", _SRC, "-lm"])
    os.replace(_SO + ".tmp", _SO)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.qsa_ref_compress.argtypes = [vp, i64, i32, i32, vp]
        L.qsa_ref_scores.argtypes = [vp, vp, i64, i32, i32, f64, vp]
        L.qsa_ref_select.argtypes = [vp, vp, i64, i32, i32, i32, i32, i32, f64, vp, vp, vp]
        L.qsa_ref_select.restype = i64
        L.qsa_ref_attend_tokens.argtypes = [vp, vp, vp, i32, i32, i32, f64, vp, i64, vp, vp]
        L.qsa_ref_sparse_attn.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, f64, i32, i32, vp, vp, vp, vp]
        L.qsa_ref_dense_attn.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, f64, vp, vp]
        L.qsa_ref_distill_kl.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, f64, i32, i32, f64, i32, vp]
        L.qsa_ref_gdn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, f64, vp, i32, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def compress(keys, r):
    """O1. keys: [L, d] bf16 bits -> [L // r, d] bf16 bits."""
    keys = _u16(keys)
    L, d = keys.shape
    out = np.empty((L // r, d), np.uint16)
    lib().qsa_ref_compress(_p(keys), L, d, r, _p(out))
    return out


def scores(q, blocks, w):
    """O2. q: [H, d]; blocks: [n, d] -> fp32 [n]."""
    q, blocks = _u16(q), _u16(blocks)
    H, d = q.shape
    n = blocks.shape[0]
    out = np.empty(n, np.float32)
    lib().qsa_ref_scores(_p(q), _p(blocks), n, H, d, float(w), _p(out))
    return out


def select(idx_q, blocks, t0, r, k, w):
    """O2 + O3 for queries t0 .. t0 + nq - 1.

    Returns (sel [nq, k] int32 ascending with -1 pad, cnt [nq] int32,
    band [nq, 2] fp32 = (last kept, first dropped) scores, scored pair count).
    """
    idx_q, blocks = _u16(idx_q), _u16(blocks)
    nq, H, d = idx_q.shape
    need = (t0 + nq - 1) // r
    assert blocks.shape[0] >= need and blocks.shape[1] == d
    sel = np.empty((nq, k), np.int32)
    cnt = np.empty(nq, np.int32)
    band = np.empty((nq, 2), np.float32)
    pairs = lib().qsa_ref_select(_p(idx_q), _p(blocks), t0, nq, H, d, r, k, float(w), _p(sel), _p(cnt), _p(band))
    return sel, cnt, band, pairs


def attend_tokens(q, K, V, tokens, scale=None):
    """O5 for one query over an explicit token list. q: [Hq, D]; K, V: [L, Hkv, D]."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    Hq, D = q.shape
    Hkv = K.shape[1]
    tok = np.ascontiguousarray(tokens, np.int64)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.empty((Hq, D), np.float64)
    lse = np.empty(Hq, np.float64)
    lib().qsa_ref_attend_tokens(_p(q), _p(K), _p(V), Hq, Hkv, D, scale, _p(tok), len(tok), _p(out), _p(lse))
    return out, lse


def sparse_attn(Q, K, V, t0, r, sel, cnt, scale=None):
    """O4 + O5 for queries t0 .. t0 + nq - 1. Q: [nq, Hq, D]; K, V: [L, Hkv, D]."""
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    nq, Hq, D = Q.shape
    Hkv = K.shape[1]
    assert K.shape[0] >= t0 + nq
    sel = np.ascontiguousarray(sel, np.int32)
    cnt = np.ascontiguousarray(cnt, np.int32)
    k = sel.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.empty((nq, Hq, D), np.float64)
    lse = np.empty((nq, Hq), np.float64)
    lib().qsa_ref_sparse_attn(_p(Q), _p(K), _p(V), t0, nq, Hq, Hkv, D, scale, r, k, _p(sel), _p(cnt), _p(out), _p(lse))
    return out, lse


def dense_attn(Q, K, V, t0, scale=None):
    """O6: causal attention over every token 0 .. t."""
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    nq, Hq, D = Q.shape
    Hkv = K.shape[1]
    assert K.shape[0] >= t0 + nq
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.empty((nq, Hq, D), np.float64)
    lse = np.empty((nq, Hq), np.float64)
    lib().qsa_ref_dense_attn(_p(Q), _p(K), _p(V), t0, nq, Hq, Hkv, D, scale, _p(out), _p(lse))
    return out, lse


def distill_kl(Q, K, idx_q, blocks, t0, r, w, scale=None):
    """O7: per-query KL(attention-mass target || indexer softmax) over the candidate
    blocks, for queries t0 .. t0 + nq - 1. Q [nq, Hq, D]; K [L, Hkv, D];
    idx_q [nq, Hi, di]; blocks [*, di] -> float64 [nq]."""
    Q, K, idx_q, blocks = _u16(Q), _u16(K), _u16(idx_q), _u16(blocks)
    nq, Hq, D = Q.shape
    Hkv = K.shape[1]
    Hi, di = idx_q.shape[1], idx_q.shape[2]
    assert K.shape[0] >= t0 + nq
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.empty(nq, np.float64)
    lib().qsa_ref_distill_kl(_p(Q), _p(K), _p(idx_q), _p(blocks), t0, nq, Hq, Hkv, D, scale, Hi, di, float(w), r,
                             _p(out))
    return out


def gdn(q, k, v, g, beta, scale=None, S0=None, heads=None):
    """O8: gated delta rule over one sequence, token by token.

    q, k [T, Hqk, dk] and v [T, Hv, dv] bf16 bits; g (log decay), beta [T, Hv]
    fp32; S0 [Hv, dv, dk] fp32 or None (zero state). Returns (o [T, Hv, dv],
    S_T [Hv, dv, dk]) in float64; with ``heads`` only those value heads are
    computed (the other entries are NaN).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    T, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T and Hv % Hqk == 0
    g = np.ascontiguousarray(g, np.float32)
    beta = np.ascontiguousarray(beta, np.float32)
    assert g.shape == (T, Hv) and beta.shape == (T, Hv)
    scale = 1.0 / math.sqrt(dk) if scale is None else scale
    heads = np.arange(Hv, dtype=np.int32) if heads is None else np.ascontiguousarray(heads, np.int32)
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(S0, np.float32)
        assert s0.shape == (Hv, dv, dk)
    o = np.full((T, Hv, dv), np.nan)
    S = np.full((Hv, dv, dk), np.nan)
    lib().qsa_ref_gdn(_p(q), _p(k), _p(v), _p(g), _p(beta), None if s0 is None else _p(s0), T, Hqk, Hv, dk, dv,
                      float(scale), _p(heads), len(heads), _p(o), _p(S))
    return o, S
