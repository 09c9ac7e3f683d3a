"""ctypes binding of the fp64 C oracle, plus a numpy brute force used to pin it.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_ref.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile attention_ref.c into liboracle.so with gcc + OpenMP (host code only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_paged_prefill.restype = ctypes.c_int
        lib.oracle_paged_prefill.argtypes = [i32, i32, i32, i32, i32, i32, f64, f64, f64,
                                             p, p, p, p, p, p, p, i64, p, i64, i64, p, p]
        lib.oracle_merge_states.restype = None
        lib.oracle_merge_states.argtypes = [i64, i32, i32, i32, p, p, p, p]
        lib.oracle_e4m3_to_double.restype = f64
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_bf16_to_double.restype = f64
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits16(x) -> np.ndarray:
    """bf16 tensor/array -> contiguous uint16 bit pattern (no arithmetic)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy()
                                        .view(np.uint16))
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    assert a.dtype == np.uint16, a.dtype
    return a


def _bits8(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.uint8).numpy())
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    assert a.dtype == np.uint8, a.dtype
    return a


def paged_prefill(*, q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                  num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                  kv_dtype: str = "bf16", sm_scale: float | None = None,
                  k_scale: float = 1.0, v_scale: float = 1.0, rows=None,
                  key_range: tuple[int, int] | None = None):
    """Attention rows, fp64. Returns (o [n, Hq, d], lse [n, Hq]) as numpy float64.

    ``q`` is bf16 ``[Nq, Hq, d]``; pools are ``[num_pages, page_size, Hkv, d]`` bf16 or
    E4M3 codes (uint8 / float8_e4m3fn). ``rows`` selects global query tokens (default: all).
    ``key_range=(lo, hi)`` keeps only keys in [lo, hi) -- one KV split's partial state.
    """
    lib = _load()
    qb = _bits16(q)
    if kv_dtype == "bf16":
        kb, vb, dt = _bits16(k_pool), _bits16(v_pool), 0
    elif kv_dtype == "fp8_e4m3":
        kb, vb, dt = _bits8(k_pool), _bits8(v_pool), 1
    else:
        raise ValueError(f"unknown kv_dtype {kv_dtype}")
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    kvp = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    kvi = np.ascontiguousarray(kv_indices, dtype=np.int32)
    lpl = np.ascontiguousarray(kv_last_page_len, dtype=np.int32)
    batch = len(qo) - 1
    nq = int(qo[-1])
    if qb.size != nq * num_qo_heads * head_dim:
        raise ValueError("q does not hold qo_indptr[-1] rows")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    if rows is None:
        sel, n = None, nq
    else:
        sel = np.ascontiguousarray(rows, dtype=np.int64)
        n = sel.size
    o = np.zeros((n, num_qo_heads, head_dim), dtype=np.float64)
    lse = np.zeros((n, num_qo_heads), dtype=np.float64)
    lo, hi = (0, -1) if key_range is None else key_range
    if n == 0:
        return o, lse
    rc = lib.oracle_paged_prefill(batch, num_qo_heads, num_kv_heads, head_dim, page_size, dt,
                                  float(sm_scale), float(k_scale), float(v_scale),
                                  _ptr(qo), _ptr(kvp), _ptr(kvi), _ptr(lpl), _ptr(qb),
                                  _ptr(kb), _ptr(vb), n,
                                  None if sel is None else _ptr(sel), int(lo), int(hi),
                                  _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle rejected the batch (qo_len > kv_len or malformed tables)")
    return o, lse


def merge_states(o_part: np.ndarray, lse_part: np.ndarray):
    """Combine softmax partials: o_part [R, S, H, d], lse_part [R, S, H] (natural log)."""
    lib = _load()
    op = np.ascontiguousarray(o_part, dtype=np.float64)
    lp = np.ascontiguousarray(lse_part, dtype=np.float64)
    R, S, H, d = op.shape
    assert lp.shape == (R, S, H)
    o = np.zeros((R, H, d), dtype=np.float64)
    lse = np.zeros((R, H), dtype=np.float64)
    lib.oracle_merge_states(R, S, H, d, _ptr(op), _ptr(lp), _ptr(o), _ptr(lse))
    return o, lse


def e4m3_decode_table() -> np.ndarray:
    """Value of every E4M3 code 0..255 (NaN for the two NaN codes), fp64."""
    lib = _load()
    return np.array([lib.oracle_e4m3_to_double(c) for c in range(256)], dtype=np.float64)


def dense_attention_np(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                       sm_scale: float):
    """Brute-force masked softmax attention, fp64, dense K/V, one request.

    q [n, Hq, d], k/v [L, Hkv, d] (float arrays), q_pos [n] absolute positions.
    Key j is visible to a query at position p iff j <= p. Builds the full score matrix,
    masks it with an explicit boolean matrix and normalises with numpy's exp/sum.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    k_rep = np.repeat(k, g, axis=1)  # [L, Hq, d]; q head h reads kv head h // g
    v_rep = np.repeat(v, g, axis=1)
    scores = np.einsum("nhd,lhd->hnl", q, k_rep) * sm_scale  # [Hq, n, L]
    visible = np.arange(L)[None, :] <= np.asarray(q_pos)[:, None]  # [n, L]
    scores = np.where(visible[None], scores, -np.inf)
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    denom = e.sum(axis=-1, keepdims=True)
    o = np.einsum("hnl,lhd->nhd", e / denom, v_rep)
    lse = (m[..., 0] + np.log(denom[..., 0])).T  # [n, Hq]
    return o, lse
