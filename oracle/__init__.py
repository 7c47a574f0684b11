"""fp64 CPU oracle for one paged-KV decode step (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline may import this package.  The product library never does, and this
package never imports the product library.

The C source states what is computed and which passages it follows.  This
wrapper only marshals numpy arrays (the storage-dtype buffers drawn by
``workloads``) into the C calls.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_decode.argtypes = [ctypes.c_int, P, P, I64]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_kv_append.argtypes = [ctypes.c_int, P, P, I64, P, P, P, I32, P, I32, I32, I32, I32, I32]
        lib.oracle_kv_append.restype = ctypes.c_int
        lib.oracle_paged_decode_attention.argtypes = [ctypes.c_int, P, P, P, I64, P, P, P, I32, P,
                                                      I32, I32, I32, I32, I32, I32, ctypes.c_float, I32]
        lib.oracle_paged_decode_attention.restype = ctypes.c_int
        lib.oracle_threads.argtypes = [I32]
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [P, P, I64]
        lib.oracle_e4m3_decode.restype = ctypes.c_int
        lib.oracle_e4m3_quantize_row.argtypes = [ctypes.c_int, P, I32, P, P]
        lib.oracle_e4m3_quantize_row.restype = ctypes.c_int
        lib.oracle_kv_append_fp8.argtypes = [ctypes.c_int, P, P, I64, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32]
        lib.oracle_kv_append_fp8.restype = ctypes.c_int
        lib.oracle_e4m3_dequantize_rows.argtypes = [P, P, I64, I32, P]
        lib.oracle_e4m3_dequantize_rows.restype = ctypes.c_int
        lib.oracle_e2m1_decode.argtypes = [P, P, I64]
        lib.oracle_e2m1_decode.restype = ctypes.c_int
        lib.oracle_mxfp4_quantize_row.argtypes = [ctypes.c_int, P, I32, P, P]
        lib.oracle_mxfp4_quantize_row.restype = ctypes.c_int
        lib.oracle_kv_append_mxfp4.argtypes = [ctypes.c_int, P, P, I64, P, P, P, P, P, I32, P, I32, I32, I32, I32,
                                               I32]
        lib.oracle_kv_append_mxfp4.restype = ctypes.c_int
        lib.oracle_mxfp4_dequantize_rows.argtypes = [P, P, I64, I32, P]
        lib.oracle_mxfp4_dequantize_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def decode(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Storage-dtype elements -> float64, using the oracle's own decoders."""
    src = np.ascontiguousarray(bits)
    dst = np.empty(src.size, dtype=np.float64)
    _check(_load().oracle_decode(_DTYPE_CODE[dtype], _ptr(src), _ptr(dst), src.size), "decode")
    return dst.reshape(src.shape)


def kv_append(dtype: str, k_new, v_new, k_pool, v_pool, block_tables, positions, block_size: int):
    """Copy the new token's K/V bits into its (block, slot), in place on k_pool / v_pool."""
    B, H_kv, D = k_new.shape
    for a in (k_new, v_new, k_pool, v_pool, block_tables, positions):
        assert a.flags.c_contiguous
    rc = _load().oracle_kv_append(_DTYPE_CODE[dtype], _ptr(k_new), _ptr(v_new), H_kv * D,
                                  _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
                                  _ptr(positions), B, H_kv, D, block_size, k_pool.shape[0])
    _check(rc, "oracle_kv_append")


def paged_decode_attention(dtype: str, q, k_pool, v_pool, block_tables, context_lens, scale,
                           *, with_lse: bool = False, nthreads: int = 0):
    """fp64 attention output [B, H_q, D] (and optionally lse [B, H_q])."""
    B, H_q, D = q.shape
    n_blocks, H_kv, bs, D2 = k_pool.shape
    assert D == D2 and v_pool.shape == k_pool.shape
    q = np.ascontiguousarray(q)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    for a in (k_pool, v_pool):
        assert a.flags.c_contiguous
    out = np.zeros((B, H_q, D), dtype=np.float64)
    lse = np.zeros((B, H_q), dtype=np.float64) if with_lse else None
    rc = _load().oracle_paged_decode_attention(
        _DTYPE_CODE[dtype], _ptr(out), _ptr(lse), _ptr(q), H_q * D, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), max(block_tables.shape[1], 1), _ptr(context_lens),
        B, H_q, H_kv, D, bs, n_blocks, float(scale), int(nthreads))
    _check(rc, "oracle_paged_decode_attention")
    return (out, lse) if with_lse else out


def threads(nthreads: int = 0) -> int:
    """How many OpenMP threads the oracle runs with for this request (0 = default)."""
    return int(_load().oracle_threads(int(nthreads)))


def run_step(w, nthreads: int = 0):
    """One whole decode step on a ``workloads.Workload``: append (if any), then attention.

    Returns (out fp64 [B,H_q,D], k_pool_after, v_pool_after) -- for an FP8 or
    MXFP4 workload each pool is a (codes, scales) pair; the workload's own pools
    are left untouched.
    """
    k_pool, v_pool = w.k_pool.copy(), w.v_pool.copy()
    if getattr(w.cfg, "kv_dtype", "") == "mxfp4":
        k_scale, v_scale = w.k_scale.copy(), w.v_scale.copy()
        if w.positions is not None:
            kv_append_mxfp4(w.cfg.dtype, w.k_new, w.v_new, k_pool, v_pool, k_scale, v_scale, w.block_tables,
                            w.positions, w.cfg.block_size)
        out = paged_decode_attention_mxfp4(w.cfg.dtype, w.q, k_pool, v_pool, k_scale, v_scale, w.block_tables,
                                           w.context_lens, w.scale, nthreads=nthreads)
        return out, (k_pool, k_scale), (v_pool, v_scale)
    if getattr(w.cfg, "fp8", False):
        k_scale, v_scale = w.k_scale.copy(), w.v_scale.copy()
        if w.positions is not None:
            kv_append_fp8(w.cfg.dtype, w.k_new, w.v_new, k_pool, v_pool, k_scale, v_scale, w.block_tables,
                          w.positions, w.cfg.block_size)
        out = paged_decode_attention_fp8(w.cfg.dtype, w.q, k_pool, v_pool, k_scale, v_scale, w.block_tables,
                                         w.context_lens, w.scale, nthreads=nthreads)
        return out, (k_pool, k_scale), (v_pool, v_scale)
    if w.positions is not None:
        kv_append(w.cfg.dtype, w.k_new, w.v_new, k_pool, v_pool, w.block_tables, w.positions,
                  w.cfg.block_size)
    out = paged_decode_attention(w.cfg.dtype, w.q, k_pool, v_pool, w.block_tables, w.context_lens,
                                 w.scale, nthreads=nthreads)
    return out, k_pool, v_pool


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) K/V cache with one power-of-two scale per token row and head
# ---------------------------------------------------------------------------

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for S.1111.111)."""
    src = np.ascontiguousarray(codes, dtype=np.uint8)
    dst = np.empty(src.size, dtype=np.float64)
    _check(_load().oracle_e4m3_decode(_ptr(src), _ptr(dst), src.size), "e4m3_decode")
    return dst.reshape(src.shape)


def e4m3_quantize_row(dtype: str, row: np.ndarray):
    """One row of source-dtype storage elements -> (uint8 codes, float32 power-of-two scale)."""
    src = np.ascontiguousarray(row)
    codes = np.empty(src.size, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.float32)
    _check(_load().oracle_e4m3_quantize_row(_DTYPE_CODE[dtype], _ptr(src), src.size, _ptr(codes), _ptr(scale)),
           "e4m3_quantize_row")
    return codes, np.float32(scale[0])


def kv_append_fp8(dtype: str, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions,
                  block_size: int):
    """Quantize the new K/V rows (source dtype) into their slots, in place on the code and scale pools."""
    B, H_kv, D = k_new.shape
    for a in (k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions):
        assert a.flags.c_contiguous
    assert k_pool.dtype == np.uint8 and k_scale.dtype == np.float32
    rc = _load().oracle_kv_append_fp8(_DTYPE_CODE[dtype], _ptr(k_new), _ptr(v_new), H_kv * D, _ptr(k_pool),
                                      _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                      block_tables.shape[1], _ptr(positions), B, H_kv, D, block_size,
                                      k_pool.shape[0])
    _check(rc, "oracle_kv_append_fp8")


def e4m3_dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Pools of codes [..., D] and scales [...] -> float32 values (exact)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    assert c.shape[:-1] == s.shape
    D = c.shape[-1]
    out = np.empty(c.shape, dtype=np.float32)
    _check(_load().oracle_e4m3_dequantize_rows(_ptr(c), _ptr(s), s.size, D, _ptr(out)), "e4m3_dequantize")
    return out


def paged_decode_attention_fp8(q_dtype: str, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens,
                               scale, *, with_lse: bool = False, nthreads: int = 0):
    """fp64 attention over FP8 pools: the float32 attention on the exactly dequantized pools, q exactly widened."""
    qf = decode(q_dtype, q).astype(np.float32) if q_dtype != "f32" else np.ascontiguousarray(q)
    kf = e4m3_dequantize(k_pool, k_scale)
    vf = e4m3_dequantize(v_pool, v_scale)
    return paged_decode_attention("f32", qf, kf, vf, block_tables, context_lens, scale, with_lse=with_lse,
                                  nthreads=nthreads)


# ---------------------------------------------------------------------------
# MXFP4 K/V cache: E2M1 codes two per byte, one E8M0 scale per 32 elements
# ---------------------------------------------------------------------------

def e2m1_decode(packed: np.ndarray) -> np.ndarray:
    """Packed E2M1 codes (uint8, two per byte, element 2k in the low nibble) -> float64 values, unscaled."""
    src = np.ascontiguousarray(packed, dtype=np.uint8)
    dst = np.empty(src.size * 2, dtype=np.float64)
    _check(_load().oracle_e2m1_decode(_ptr(src), _ptr(dst), dst.size), "e2m1_decode")
    return dst.reshape(src.shape[:-1] + (src.shape[-1] * 2,)) if src.ndim else dst


def mxfp4_quantize_row(dtype: str, row: np.ndarray):
    """One row of D source-dtype storage elements -> (uint8 codes [D/2], uint8 E8M0 scales [D/32])."""
    src = np.ascontiguousarray(row)
    D = src.size
    codes = np.zeros(D // 2, dtype=np.uint8)
    scales = np.zeros(D // 32, dtype=np.uint8)
    _check(_load().oracle_mxfp4_quantize_row(_DTYPE_CODE[dtype], _ptr(src), D, _ptr(codes), _ptr(scales)),
           "mxfp4_quantize_row")
    return codes, scales


def kv_append_mxfp4(dtype: str, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions,
                    block_size: int):
    """Quantize the new K/V rows (source dtype) into their slots, in place on the code and scale pools."""
    B, H_kv, D = k_new.shape
    for a in (k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions):
        assert a.flags.c_contiguous
    assert k_pool.dtype == np.uint8 and k_scale.dtype == np.uint8
    rc = _load().oracle_kv_append_mxfp4(_DTYPE_CODE[dtype], _ptr(k_new), _ptr(v_new), H_kv * D, _ptr(k_pool),
                                        _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                        block_tables.shape[1], _ptr(positions), B, H_kv, D, block_size,
                                        k_pool.shape[0])
    _check(rc, "oracle_kv_append_mxfp4")


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Pools of codes [..., D/2] and scales [..., D/32] -> float32 values [..., D] (exact)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    D = c.shape[-1] * 2
    assert c.shape[:-1] == s.shape[:-1] and s.shape[-1] * 32 == D
    n_rows = int(np.prod(c.shape[:-1]))
    out = np.empty(c.shape[:-1] + (D,), dtype=np.float32)
    _check(_load().oracle_mxfp4_dequantize_rows(_ptr(c), _ptr(s), n_rows, D, _ptr(out)), "mxfp4_dequantize")
    return out


def paged_decode_attention_mxfp4(q_dtype: str, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens,
                                 scale, *, with_lse: bool = False, nthreads: int = 0):
    """fp64 attention over MXFP4 pools: the float32 attention on the exactly dequantized pools, q exactly widened."""
    qf = decode(q_dtype, q).astype(np.float32) if q_dtype != "f32" else np.ascontiguousarray(q)
    kf = mxfp4_dequantize(k_pool, k_scale)
    vf = mxfp4_dequantize(v_pool, v_scale)
    return paged_decode_attention("f32", qf, kf, vf, block_tables, context_lens, scale, with_lse=with_lse,
                                  nthreads=nthreads)
