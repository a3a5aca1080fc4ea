"""Seeded, counter-based synthetic inputs for the sparse-attention harness.

The arithmetic lives in ``qsa_gen.c`` (see its header for the definition).
Everything here returns bf16 *bit patterns* as ``numpy.uint16`` arrays; the
oracle widens them exactly and the GPU side uploads the same bytes. Nothing in
this package computes any step of the method.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_gen.c")
_SO = os.path.join(_HERE, "libqsagen.so")
_lib = None

# Stream ids of the tensors of one workload.
STREAM_Q, STREAM_K, STREAM_V, STREAM_IDX_Q, STREAM_IDX_K = 1, 2, 3, 4, 5
# Streams of the recurrent-layer (gated delta rule) inputs.
STREAM_GDN_Q, STREAM_GDN_K, STREAM_GDN_V, STREAM_GDN_A, STREAM_GDN_B, STREAM_GDN_S = 8, 9, 10, 11, 12, 13


def build():
    """Compile the generator library in place (gcc, OpenMP)."""
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", _SO + ".tmp", _SRC, "-lm"])
    os.replace(_SO + ".tmp", _SO)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, u32, i64, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        L.qsa_gen_init.argtypes = []
        L.qsa_gen_ntab.argtypes = [vp]
        L.qsa_gen_normal_bf16.argtypes = [u64, u32, u64, u64, ctypes.c_float, vp]
        L.qsa_gen_int_bf16.argtypes = [u64, u32, u64, u64, i32, i32, vp]
        L.qsa_gen_needle_dir.argtypes = [u64, i32, vp]
        L.qsa_gen_needle_offset.argtypes = [u64, i64, i64, i64, i32]
        L.qsa_gen_needle_offset.restype = i64
        L.qsa_gen_idx_keys_bf16.argtypes = [u64, i64, i64, i64, i64, i32, i64, i32, vp]
        L.qsa_gen_init()
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def ntab():
    out = np.empty(65536, np.float32)
    lib().qsa_gen_ntab(_ptr(out))
    return out


def normal(seed, stream, shape, e0=0, scale=1.0, out=None):
    """Elements [e0, e0 + prod(shape)) of a normal stream, as bf16 bits."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, np.uint16)
    lib().qsa_gen_normal_bf16(seed, stream, e0, n, scale, _ptr(out))
    return out


def ints(seed, stream, shape, lo, hi, e0=0):
    """Integer-valued bf16 elements uniform in [lo, hi]."""
    out = np.empty(shape, np.uint16)
    lib().qsa_gen_int_bf16(seed, stream, e0, int(np.prod(shape)), lo, hi, _ptr(out))
    return out


def needle_dir(seed, d=64):
    u = np.empty(d, np.float64)
    lib().qsa_gen_needle_dir(seed, d, _ptr(u))
    return u


def needle_offset(seed, b, w, window, r):
    return lib().qsa_gen_needle_offset(seed, b, w, window, r)


def idx_keys(seed, b, L, s0, ns, d=64, window=0, r=4, out=None):
    """Indexer keys of batch row b, tokens [s0, s0 + ns) of a [B, L, d] tensor."""
    if out is None:
        out = np.empty((ns, d), np.uint16)
    lib().qsa_gen_idx_keys_bf16(seed, b, L, s0, ns, d, window, r, _ptr(out))
    return out


def bf16_to_f64(a):
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16(x):
    """Round-to-nearest-even fp32 -> bf16 bits (harness helper for building inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _unit_rows(bits):
    """Rows of bf16 bits scaled to unit L2 norm (in double), rounded back to bf16."""
    x = bf16_to_f64(bits)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return f32_to_bf16(x.astype(np.float32))


def gdn_inputs(seed, B, T, Hqk, Hv, dk=128, dv=128, decay_shift=3.0):
    """Inputs of the gated delta rule for B sequences of T tokens.

    q, k [B, T, Hqk, dk]: normal rows scaled to unit norm (the layer normalises
    them before the mixing), bf16 bits. v [B, T, Hv, dv]: N(0, 1) bf16 bits.
    g [B, T, Hv] fp32: log of the decay gate sigmoid(x + decay_shift), x
    normal (mean decay about 0.95 at the default shift). beta [B, T, Hv] fp32:
    the write gate sigmoid(y), y normal.
    """
    q = _unit_rows(normal(seed, STREAM_GDN_Q, (B, T, Hqk, dk)))
    k = _unit_rows(normal(seed, STREAM_GDN_K, (B, T, Hqk, dk)))
    v = normal(seed, STREAM_GDN_V, (B, T, Hv, dv))
    x = bf16_to_f64(normal(seed, STREAM_GDN_A, (B, T, Hv))) + decay_shift
    g = (-np.logaddexp(0.0, -x)).astype(np.float32)
    y = bf16_to_f64(normal(seed, STREAM_GDN_B, (B, T, Hv)))
    beta = (1.0 / (1.0 + np.exp(-y))).astype(np.float32)
    return q, k, v, g, beta


def gdn_state(seed, B, Hv, dv=128, dk=128, scale=0.25):
    """An initial recurrent state [B, Hv, dv, dk] fp32: scaled normal values."""
    return (bf16_to_f64(normal(seed, STREAM_GDN_S, (B, Hv, dv, dk))) * scale).astype(np.float32)
