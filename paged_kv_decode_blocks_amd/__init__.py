"""paged_kv_decode_blocks_amd -- paged-KV decode attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libpkv.so``, whose C ABI is declared in
``include/pkv.h``.  This module only marshals arguments: it turns torch tensors
into device pointers, element strides and the current HIP stream, and raises
on a non-OK status.  Every step of the computation runs in the library's HIP
kernels; there is no CPU or PyTorch fallback, and a missing library is an error.

Entry points (same names as the C ABI without the ``pkv_`` prefix):
  kv_append                 write each request's new K/V token into its slot
  paged_decode_attention    attention of one query per head over the paged history
  append_decode_attention   both, as one decode step (single attention launch)
  decode_workspace_bytes    workspace size of a split-KV call
  copy_blocks               copy whole physical blocks (copy-on-write of shared blocks)
  kv_append_fp8, paged_decode_attention_fp8, append_decode_attention_fp8
                            the same calls over an FP8 (OCP E4M3) cache with per-row scales
  BlockManager              host-side block allocation, sharing and reclaim (pkv_bm_*)
  StepGraphs                the fused step captured per (batch, context) bucket (pkv_step_graphs_*)
  Decoder                   one call per decode step: manager, staged metadata, graph or eager launch
  cu_mask, CuMaskedStream   streams whose kernels run on a chosen subset of compute units
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "PkvError", "LIB_PATH", "load_library", "library_loaded", "kv_append", "paged_decode_attention",
    "append_decode_attention", "decode_workspace_bytes", "last_launch", "version", "probe_stream_read",
    "PKV_F32", "PKV_F16", "PKV_BF16", "EXPORTED_SYMBOLS", "copy_blocks", "BlockManager", "StepGraphs", "DualStepGraphs", "Decoder", "cu_mask", "CuMaskedStream",
    "kv_append_fp8", "paged_decode_attention_fp8", "append_decode_attention_fp8", "copy_blocks_fp8",
    "device_cu_count", "append_decode_attention_persistent", "append_decode_attention_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "kv_append_mxfp4", "paged_decode_attention_mxfp4", "append_decode_attention_mxfp4", "copy_blocks_mxfp4",
    "PKV_ERR_OUT_OF_BLOCKS", "PKV_ERR_SEQUENCE", "PKV_ERR_ALIASED_APPEND", "PKV_ERR_HIP", "check_step_metadata",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
PKV_ERR_INVALID_ARG, PKV_ERR_ALIASED_APPEND, PKV_ERR_HIP, PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_SEQUENCE = -2, -5, -6, -7, -8
BLOCK_SIZE = 16

EXPORTED_SYMBOLS = (
    "pkv_version", "pkv_status_string", "pkv_last_error", "pkv_last_launch", "pkv_kv_append",
    "pkv_decode_workspace_bytes", "pkv_paged_decode_attention", "pkv_append_decode_attention",
    "pkv_append_decode_attention_persistent", "pkv_append_decode_attention_noalloc", "pkv_check_step_metadata",
    "pkv_probe_mfma_burn", "pkv_probe_gemm_bf16", "pkv_dual_step_graphs_create", "pkv_dual_step_graphs_launch",
    "pkv_dual_step_graphs_destroy",
    "pkv_probe_stream_read", "pkv_probe_tile_read", "pkv_copy_blocks", "pkv_copy_blocks_fp8", "pkv_kv_append_fp8", "pkv_paged_decode_attention_fp8",
    "pkv_append_decode_attention_fp8", "pkv_kv_append_mxfp4", "pkv_paged_decode_attention_mxfp4",
    "pkv_append_decode_attention_mxfp4", "pkv_copy_blocks_mxfp4",
    "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_add_sequence", "pkv_bm_add_sequence_shared", "pkv_bm_fork",
    "pkv_bm_append_token", "pkv_bm_append_batch", "pkv_bm_free_sequence", "pkv_bm_num_free_blocks",
    "pkv_bm_num_sequences", "pkv_bm_sequence_length", "pkv_bm_block_refcount", "pkv_bm_block_table",
    "pkv_bm_batch_tables", "pkv_step_graphs_create", "pkv_step_graphs_launch", "pkv_step_graphs_destroy",
    "pkv_decoder_create", "pkv_decoder_destroy", "pkv_decoder_block_manager", "pkv_decoder_step",
    "pkv_device_cu_count", "pkv_cu_mask", "pkv_stream_create_cu_masked", "pkv_stream_destroy",
)

_lib = None


class StepDesc(ctypes.Structure):
    """Mirror of ``pkv_step_desc`` in include/pkv.h (same field order and types)."""
    _fields_ = [
        ("dtype", ctypes.c_int), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("scale", ctypes.c_float),
        ("partition_size", ctypes.c_int32), ("out", ctypes.c_void_p), ("q", ctypes.c_void_p),
        ("q_row_stride", ctypes.c_int64), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("new_row_stride", ctypes.c_int64), ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("bt_stride", ctypes.c_int32), ("positions", ctypes.c_void_p),
        ("cow_src", ctypes.c_void_p), ("cow_dst", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("k_mx_scale", ctypes.c_void_p), ("v_mx_scale", ctypes.c_void_p),
    ]


class DecoderDesc(ctypes.Structure):
    """Mirror of ``pkv_decoder_desc`` in include/pkv.h (same field order and types)."""
    _fields_ = [
        ("dtype", ctypes.c_int), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("scale", ctypes.c_float),
        ("partition_size", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("bt_stride", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("q", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("new_row_stride", ctypes.c_int64),
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("shuffle_seed", ctypes.c_uint64),
        ("batch_caps", ctypes.c_void_p), ("n_batch_caps", ctypes.c_int32),
        ("ctx_caps", ctypes.c_void_p), ("n_ctx_caps", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("k_mx_scale", ctypes.c_void_p), ("v_mx_scale", ctypes.c_void_p),
    ]


class PkvError(RuntimeError):
    """A libpkv call returned a non-OK status (or the library is missing)."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: Optional[str] = None):
    """Load libpkv.so (built in-tree by ``build.py``) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise PkvError(-100, f"libpkv.so not found at {p}; build it with paged_kv_decode_blocks_amd.build.build()")
    lib = ctypes.CDLL(p)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_launch.argtypes = []
    lib.pkv_last_launch.restype = ctypes.c_char_p
    lib.pkv_kv_append.argtypes = [ctypes.c_int, P, P, I64, P, P, P, I32, P, I32, I32, I32, I32, I32, P]
    lib.pkv_kv_append.restype = ctypes.c_int
    lib.pkv_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.pkv_decode_workspace_bytes.restype = SZ
    lib.pkv_paged_decode_attention.argtypes = [ctypes.c_int, P, P, I64, P, P, P, I32, P,
                                               I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32,
                                               P, SZ, P]
    lib.pkv_paged_decode_attention.restype = ctypes.c_int
    lib.pkv_append_decode_attention.argtypes = [ctypes.c_int, P, P, I64, P, P, I64, P, P, P, I32, P,
                                                I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32,
                                                P, SZ, P]
    lib.pkv_append_decode_attention.restype = ctypes.c_int
    lib.pkv_check_step_metadata.argtypes = [P, I32, P, P, I32, I32, I32, I32, P]
    lib.pkv_check_step_metadata.restype = ctypes.c_int
    lib.pkv_append_decode_attention_noalloc.argtypes = [ctypes.c_int, P, P, I64, P, P, I64, P, P, P, I32, P,
                                                        I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32, P]
    lib.pkv_append_decode_attention_noalloc.restype = ctypes.c_int
    lib.pkv_append_decode_attention_persistent.argtypes = [ctypes.c_int, P, P, I64, P, P, I64, P, P, P, I32, P,
                                                           I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32,
                                                           P, SZ, I32, P]
    lib.pkv_append_decode_attention_persistent.restype = ctypes.c_int
    lib.pkv_probe_mfma_burn.argtypes = [I32, I32, P, P]
    lib.pkv_probe_mfma_burn.restype = ctypes.c_int
    lib.pkv_probe_gemm_bf16.argtypes = [I32, P, P, P, I32, I32, I32, P]
    lib.pkv_probe_gemm_bf16.restype = ctypes.c_int
    lib.pkv_probe_stream_read.argtypes = [P, SZ, P, I32, P]
    lib.pkv_probe_stream_read.restype = ctypes.c_int
    lib.pkv_probe_tile_read.argtypes = [P, P, P, P, I32, I32, I32, P, I32, I32, I32, I32, P, I32, P]
    lib.pkv_probe_tile_read.restype = ctypes.c_int
    lib.pkv_kv_append_fp8.argtypes = [ctypes.c_int, P, P, I64, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, P]
    lib.pkv_kv_append_fp8.restype = ctypes.c_int
    lib.pkv_paged_decode_attention_fp8.argtypes = [ctypes.c_int, P, P, I64, P, P, P, P, P, I32, P,
                                                   I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32,
                                                   P, SZ, P]
    lib.pkv_paged_decode_attention_fp8.restype = ctypes.c_int
    lib.pkv_append_decode_attention_fp8.argtypes = [ctypes.c_int, P, P, I64, P, P, I64, P, P, P, P, P, I32, P,
                                                    I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32,
                                                    P, SZ, P]
    lib.pkv_append_decode_attention_fp8.restype = ctypes.c_int
    lib.pkv_kv_append_mxfp4.argtypes = [ctypes.c_int, P, P, I64, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, P]
    lib.pkv_kv_append_mxfp4.restype = ctypes.c_int
    lib.pkv_paged_decode_attention_mxfp4.argtypes = [ctypes.c_int, P, P, I64, P, P, P, P, P, I32, P,
                                                     I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32,
                                                     P, SZ, P]
    lib.pkv_paged_decode_attention_mxfp4.restype = ctypes.c_int
    lib.pkv_append_decode_attention_mxfp4.argtypes = [ctypes.c_int, P, P, I64, P, P, I64, P, P, P, P, P, I32, P,
                                                      I32, I32, I32, I32, I32, I32, I32, ctypes.c_float, I32,
                                                      P, SZ, P]
    lib.pkv_append_decode_attention_mxfp4.restype = ctypes.c_int
    lib.pkv_copy_blocks_fp8.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, P]
    lib.pkv_copy_blocks_fp8.restype = ctypes.c_int
    lib.pkv_copy_blocks_mxfp4.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, P]
    lib.pkv_copy_blocks_mxfp4.restype = ctypes.c_int
    lib.pkv_copy_blocks.argtypes = [ctypes.c_int, P, P, P, P, I32, I32, I32, I32, I32, P]
    lib.pkv_copy_blocks.restype = ctypes.c_int
    U64, C = ctypes.c_uint64, ctypes.c_int
    lib.pkv_bm_create.argtypes = [I32, I32, U64]
    lib.pkv_bm_create.restype = P
    lib.pkv_bm_destroy.argtypes = [P]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_add_sequence.argtypes = [P, I64, I32]
    lib.pkv_bm_add_sequence_shared.argtypes = [P, I64, I32, I64, I32, P]
    lib.pkv_bm_fork.argtypes = [P, I64, I64]
    lib.pkv_bm_append_token.argtypes = [P, I64, P, P, P]
    lib.pkv_bm_append_batch.argtypes = [P, P, I32, P, I32, P, P, P, P]
    lib.pkv_bm_free_sequence.argtypes = [P, I64]
    lib.pkv_bm_num_free_blocks.argtypes = [P]
    lib.pkv_bm_num_sequences.argtypes = [P]
    lib.pkv_bm_sequence_length.argtypes = [P, I64]
    lib.pkv_bm_block_refcount.argtypes = [P, I32]
    lib.pkv_bm_block_table.argtypes = [P, I64, P, I32, P]
    lib.pkv_bm_batch_tables.argtypes = [P, P, I32, P, I32, P]
    for name in ("add_sequence", "add_sequence_shared", "fork", "append_token", "append_batch", "free_sequence",
                 "block_table", "batch_tables"):
        getattr(lib, "pkv_bm_" + name).restype = C
    for name in ("num_free_blocks", "num_sequences", "sequence_length", "block_refcount"):
        getattr(lib, "pkv_bm_" + name).restype = I32
    lib.pkv_step_graphs_create.argtypes = [ctypes.POINTER(StepDesc), P, I32, P, I32]
    lib.pkv_step_graphs_create.restype = P
    lib.pkv_step_graphs_launch.argtypes = [P, I32, I32, I32, P]
    lib.pkv_step_graphs_launch.restype = C
    lib.pkv_step_graphs_destroy.argtypes = [P]
    lib.pkv_step_graphs_destroy.restype = None
    lib.pkv_dual_step_graphs_create.argtypes = [ctypes.POINTER(StepDesc), ctypes.POINTER(StepDesc), P, I32, P, I32,
                                                I32, ctypes.c_int]
    lib.pkv_dual_step_graphs_create.restype = P
    lib.pkv_dual_step_graphs_launch.argtypes = [P, I32, I32, P]
    lib.pkv_dual_step_graphs_launch.restype = ctypes.c_int
    lib.pkv_dual_step_graphs_destroy.argtypes = [P]
    lib.pkv_dual_step_graphs_destroy.restype = None
    lib.pkv_decoder_create.argtypes = [ctypes.POINTER(DecoderDesc)]
    lib.pkv_decoder_create.restype = P
    lib.pkv_decoder_destroy.argtypes = [P]
    lib.pkv_decoder_destroy.restype = None
    lib.pkv_decoder_block_manager.argtypes = [P]
    lib.pkv_decoder_block_manager.restype = P
    lib.pkv_decoder_step.argtypes = [P, P, I32, P, P]
    lib.pkv_decoder_step.restype = C
    lib.pkv_device_cu_count.argtypes = []
    lib.pkv_device_cu_count.restype = C
    lib.pkv_cu_mask.argtypes = [I32, I32, C, P, I32]
    lib.pkv_cu_mask.restype = C
    lib.pkv_stream_create_cu_masked.argtypes = [P, I32, ctypes.POINTER(ctypes.c_void_p)]
    lib.pkv_stream_create_cu_masked.restype = C
    lib.pkv_stream_destroy.argtypes = [P]
    lib.pkv_stream_destroy.restype = C
    if path is None:
        _lib = lib
    return lib


def library_loaded() -> bool:
    return _lib is not None


def _check(rc: int, what: str):
    if rc != 0:
        lib = load_library()
        raise PkvError(rc, f"{what}: {lib.pkv_status_string(rc).decode()}: {lib.pkv_last_error().decode()}")


def version() -> int:
    return int(load_library().pkv_version())


def last_launch() -> str:
    return load_library().pkv_last_launch().decode()


def probe_stream_read(buf, sink, grid: int = 16384, *, nbytes: Optional[int] = None, stream=None):
    """Launch the streaming-read measurement kernel over the first `nbytes` bytes of `buf`
    (a device tensor; all of it by default)."""
    total = buf.numel() * buf.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    _require(0 <= nbytes <= total, "nbytes exceeds the buffer")
    _check(load_library().pkv_probe_stream_read(_ptr(buf), nbytes, _ptr(sink), int(grid), _stream(stream)),
           "probe_stream_read")


def probe_tile_read(k_pool, v_pool, block_ids, sink, *, heads: int, tile_bytes: int, team: int = 1,
                    paths: int = 0, depth: int = 4, k_scale=None, v_scale=None, n_items: Optional[int] = None,
                    grid: int = 1024, stream=None):
    """Launch the tile-read measurement kernel: item t reads `team` neighbouring heads of block
    block_ids[t] from K/V pools viewed as [n_blocks][heads][tile_bytes] (and 64-byte scale tiles
    if k_scale / v_scale are given); `paths` bit 1 / 2 / 4 moves K / V / scale tiles by DMA into
    LDS; each wave keeps `depth` items in flight.  Returns the bytes read."""
    torch = _torch()
    nbytes = lambda t: t.numel() * t.element_size()
    _require(block_ids.dtype == torch.int32 and block_ids.is_contiguous(), "block_ids int32, contiguous")
    _require((k_scale is None) == (v_scale is None), "k_scale and v_scale: both or neither")
    n_blocks = min(nbytes(k_pool), nbytes(v_pool)) // (int(heads) * int(tile_bytes))
    if k_scale is not None:
        n_blocks = min(n_blocks, min(nbytes(k_scale), nbytes(v_scale)) // (int(heads) * 64))
    n_items = block_ids.numel() if n_items is None else int(n_items)
    _require(0 <= n_items <= block_ids.numel(), "n_items exceeds block_ids")
    _check(load_library().pkv_probe_tile_read(_ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), n_blocks,
                                              int(heads), int(tile_bytes), _ptr(block_ids), n_items, int(team),
                                              int(paths), int(depth), _ptr(sink), int(grid), _stream(stream)),
           "probe_tile_read")
    return n_items * int(team) * (2 * int(tile_bytes) + (128 if k_scale is not None else 0))


def probe_gemm_bf16(a, b_t, c, n_workgroups: int, *, stream=None):
    """Launch the GEMM neighbour: c[M][N] (float32) = a[M][K] . b_t[N][K]^T (bf16) on n_workgroups CUs."""
    torch = _torch()
    M, K = a.shape
    N = b_t.shape[0]
    _require(a.dtype == torch.bfloat16 and b_t.dtype == torch.bfloat16 and c.dtype == torch.float32,
             "a, b_t bf16 and c float32")
    _require(a.is_contiguous() and b_t.is_contiguous() and c.is_contiguous(), "contiguous operands")
    _require(tuple(b_t.shape) == (N, K) and tuple(c.shape) == (M, N), "shapes a [M][K], b_t [N][K], c [M][N]")
    _check(load_library().pkv_probe_gemm_bf16(int(n_workgroups), _ptr(a), _ptr(b_t), _ptr(c), M, N, K,
                                              _stream(stream)), "probe_gemm_bf16")


def decode_workspace_bytes(B: int, H_q: int, D: int, max_context_len: int, partition_size: int) -> int:
    return int(load_library().pkv_decode_workspace_bytes(B, H_q, D, max_context_len, partition_size))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}
    if t.dtype not in m:
        raise PkvError(-3, f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(cond: bool, msg: str):
    if not cond:
        raise PkvError(-2, msg)


def _rows(t, name: str, heads: int, D: int):
    """Row stride (elements) of a [B, heads, D] view whose heads are D apart and elements contiguous."""
    _require(t.dim() == 3 and t.shape[1] == heads and t.shape[2] == D, f"{name} must be [B, {heads}, {D}]")
    _require(t.stride(2) == 1 and (heads == 1 or t.stride(1) == D), f"{name}: heads must be contiguous rows of D")
    return t.stride(0) if t.shape[0] > 1 else heads * D


def _pool_dims(k_pool, v_pool):
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "k_pool/v_pool must be [n_blocks, H_kv, 16, D]")
    _require(k_pool.is_contiguous() and v_pool.is_contiguous(), "pools must be contiguous")
    _require(k_pool.dtype == v_pool.dtype, "k_pool and v_pool dtypes differ")
    n_blocks, H_kv, bs, D = k_pool.shape
    return n_blocks, H_kv, bs, D


def _int32_2d(t, name):
    torch = _torch()
    _require(t.dtype == torch.int32 and t.dim() == 2 and t.stride(1) == 1, f"{name} must be int32 [B, W] rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _int32_1d(t, name, B):
    torch = _torch()
    _require(t.dtype == torch.int32 and t.dim() == 1 and t.shape[0] == B and (B <= 1 or t.stride(0) == 1),
             f"{name} must be contiguous int32 [B]")


def kv_append(k_new, v_new, k_pool, v_pool, block_tables, positions, *, stream=None):
    """Write k_new/v_new [B, H_kv, D] into slot positions[b] of each request's block (bit copy)."""
    n_blocks, H_kv, bs, D = _pool_dims(k_pool, v_pool)
    B = k_new.shape[0]
    _require(k_new.dtype == k_pool.dtype and v_new.dtype == k_pool.dtype, "k_new/v_new dtype must match the pools")
    rs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == rs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    rc = load_library().pkv_kv_append(_dtype_code(k_pool), _ptr(k_new), _ptr(v_new), rs, _ptr(k_pool), _ptr(v_pool),
                                      _ptr(block_tables), bts, _ptr(positions), B, H_kv, D, bs, n_blocks,
                                      _stream(stream))
    _check(rc, "kv_append")


def _workspace(B, H_q, D, max_context_len, partition_size, workspace, device):
    need = decode_workspace_bytes(B, H_q, D, max_context_len, partition_size)
    if need == 0:
        return None, 0
    if workspace is None:
        torch = _torch()
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def paged_decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale: float, max_context_len: int,
                           *, partition_size: int = 0, out=None, workspace=None, stream=None):
    """out[b, h, :] = softmax(scale * q[b, h] . K_t) V over the request's context_lens[b] paged tokens (float32).

    ``max_context_len`` is a host-known bound on context_lens.  With
    ``partition_size`` > 0 the context is split and merged by log-sum-exp; a
    workspace is allocated here unless one is passed (pass one to keep the
    call allocation-free).
    """
    torch = _torch()
    n_blocks, H_kv, bs, D = _pool_dims(k_pool, v_pool)
    B, H_q = q.shape[0], q.shape[1]
    _require(q.dtype == k_pool.dtype, "q dtype must match the pools")
    qrs = _rows(q, "q", H_q, D)
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(context_lens, "context_lens", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    ws, ws_bytes = _workspace(B, H_q, D, max_context_len, partition_size, workspace, q.device)
    rc = load_library().pkv_paged_decode_attention(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), bts,
        _ptr(context_lens), B, H_q, H_kv, D, bs, n_blocks, int(max_context_len), float(scale),
        int(partition_size), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "paged_decode_attention")
    return out


def append_decode_attention(q, k_new, v_new, k_pool, v_pool, block_tables, positions, scale: float,
                            max_context_len: int, *, partition_size: int = 0, out=None, workspace=None,
                            stream=None):
    """One decode step: write the new token at positions[b], attend over positions[b] + 1 tokens."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _pool_dims(k_pool, v_pool)
    B, H_q = q.shape[0], q.shape[1]
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _require(t.dtype == k_pool.dtype, f"{nm} dtype must match the pools")
    qrs = _rows(q, "q", H_q, D)
    nrs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == nrs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    ws, ws_bytes = _workspace(B, H_q, D, max_context_len, partition_size, workspace, q.device)
    rc = load_library().pkv_append_decode_attention(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_new), _ptr(v_new), nrs, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), bts, _ptr(positions), B, H_q, H_kv, D, bs, n_blocks, int(max_context_len),
        float(scale), int(partition_size), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "append_decode_attention")
    return out


def check_step_metadata(block_tables, *, context_lens=None, positions=None, n_blocks: int,
                        max_context_len: int = 0, block_size: int = BLOCK_SIZE, stream=None) -> int:
    """The step's device metadata against the kernels' contract (synchronous debugging aid).

    Returns PKV_OK (0), PKV_ERR_INVALID_ARG (a length or block id out of range) or
    PKV_ERR_ALIASED_APPEND (two appends of the step target one (block, slot)); the
    detail of a violation is in last_error()."""
    _require((context_lens is None) != (positions is None), "pass exactly one of context_lens and positions")
    lens = positions if positions is not None else context_lens
    B = int(lens.shape[0])
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(lens, "positions" if positions is not None else "context_lens", B)
    return int(load_library().pkv_check_step_metadata(
        _ptr(block_tables), bts, _ptr(context_lens), _ptr(positions), B, int(block_size), int(n_blocks),
        int(max_context_len), _stream(stream)))


def last_error() -> str:
    """Detail of the calling thread's last non-OK status."""
    return load_library().pkv_last_error().decode()


NOALLOC_SCRATCH_BYTES = 32 << 20     # PKV_NOALLOC_SCRATCH_BYTES


def append_decode_attention_noalloc(q, k_new, v_new, k_pool, v_pool, block_tables, positions, scale: float,
                                    max_context_len: int, *, partition_size: int = 0, out=None, stream=None):
    """append_decode_attention whose split partials live in the library's own device array
    (at most NOALLOC_SCRATCH_BYTES): the C call allocates nothing.  Pass ``out`` to keep the
    Python call allocation-free too.  Calls that overlap on one GPU race on that array."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _pool_dims(k_pool, v_pool)
    B, H_q = q.shape[0], q.shape[1]
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _require(t.dtype == k_pool.dtype, f"{nm} dtype must match the pools")
    qrs = _rows(q, "q", H_q, D)
    nrs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == nrs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    rc = load_library().pkv_append_decode_attention_noalloc(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_new), _ptr(v_new), nrs, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), bts, _ptr(positions), B, H_q, H_kv, D, bs, n_blocks, int(max_context_len),
        float(scale), int(partition_size), _stream(stream))
    _check(rc, "append_decode_attention_noalloc")
    return out


def append_decode_attention_persistent(q, k_new, v_new, k_pool, v_pool, block_tables, positions, scale: float,
                                       max_context_len: int, n_workgroups: int, *, partition_size: int = 0,
                                       out=None, workspace=None, stream=None):
    """The fused step as ``n_workgroups`` persistent 16-wave workgroups, one per CU (f16/bf16, H_q == H_kv)."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _pool_dims(k_pool, v_pool)
    B, H_q = q.shape[0], q.shape[1]
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _require(t.dtype == k_pool.dtype, f"{nm} dtype must match the pools")
    qrs = _rows(q, "q", H_q, D)
    nrs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == nrs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    ws, ws_bytes = _workspace(B, H_q, D, max_context_len, partition_size, workspace, q.device)
    rc = load_library().pkv_append_decode_attention_persistent(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_new), _ptr(v_new), nrs, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), bts, _ptr(positions), B, H_q, H_kv, D, bs, n_blocks, int(max_context_len),
        float(scale), int(partition_size), _ptr(ws), ws_bytes, int(n_workgroups), _stream(stream))
    _check(rc, "append_decode_attention_persistent")
    return out


def copy_blocks(k_pool, v_pool, src, dst, *, stream=None):
    """pool[dst[i]] = pool[src[i]] for both pools; src/dst are device int32 [n] tensors."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _pool_dims(k_pool, v_pool)
    n = src.shape[0]
    for t, nm in ((src, "src"), (dst, "dst")):
        _require(t.dtype == torch.int32 and t.dim() == 1 and t.shape[0] == n and (n <= 1 or t.stride(0) == 1),
                 f"{nm} must be contiguous int32 [n]")
    rc = load_library().pkv_copy_blocks(_dtype_code(k_pool), _ptr(k_pool), _ptr(v_pool), _ptr(src), _ptr(dst), n,
                                        H_kv, D, bs, n_blocks, _stream(stream))
    _check(rc, "copy_blocks")


# ---------------------------------------------------------------------------
# Host block manager (numpy arrays in and out; no device memory involved)
# ---------------------------------------------------------------------------

class BlockManager:
    """Owns a ``pkv_block_manager``: which physical blocks each sequence maps.

    Method names follow the C ABI (``pkv_bm_<name>``); a failing call raises
    PkvError with the C status and changes nothing.
    """

    def __init__(self, n_blocks: int, block_size: int = BLOCK_SIZE, shuffle_seed: int = 0, *, _borrow=None):
        lib = load_library()
        if _borrow is not None:            # a manager owned by a Decoder; never destroyed here
            h, self._owner = _borrow
        else:
            h = lib.pkv_bm_create(int(n_blocks), int(block_size), int(shuffle_seed) & ((1 << 64) - 1))
            self._owner = None
        if not h:
            raise PkvError(-2, "pkv_bm_create: " + lib.pkv_last_error().decode())
        self._h = ctypes.c_void_p(h)
        self._lib = lib
        self.n_blocks = int(n_blocks)
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None) is not None:
            if self._owner is None:
                self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def add_sequence(self, seq_id: int, num_tokens: int) -> None:
        _check(self._lib.pkv_bm_add_sequence(self._h, int(seq_id), int(num_tokens)), "bm_add_sequence")

    def add_sequence_shared(self, seq_id: int, num_tokens: int, prefix_id: int, prefix_tokens: int) -> int:
        """Returns the number of leading tokens mapped from prefix_id (whole blocks)."""
        shared = ctypes.c_int32(0)
        _check(self._lib.pkv_bm_add_sequence_shared(self._h, int(seq_id), int(num_tokens), int(prefix_id),
                                                    int(prefix_tokens), ctypes.byref(shared)),
               "bm_add_sequence_shared")
        return shared.value

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(self._lib.pkv_bm_fork(self._h, int(parent_id), int(child_id)), "bm_fork")

    def append_token(self, seq_id: int):
        """Returns (position, cow_src, cow_dst); (-1, -1) when no block must be copied."""
        pos, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pkv_bm_append_token(self._h, int(seq_id), ctypes.byref(pos), ctypes.byref(src),
                                             ctypes.byref(dst)), "bm_append_token")
        return pos.value, src.value, dst.value

    def append_batch(self, seq_ids, bt_stride: int, *, out_tables=None, out_positions=None):
        """One decode step's metadata.  Returns (tables int32 [B, bt_stride], positions int32 [B],
        cow int32 [n_cow, 2] of (src, dst) pairs)."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        B = ids.shape[0]
        tables = out_tables if out_tables is not None else np.empty((B, bt_stride), dtype=np.int32)
        positions = out_positions if out_positions is not None else np.empty(B, dtype=np.int32)
        _require(tables.dtype == np.int32 and tables.shape == (B, bt_stride) and tables.flags.c_contiguous,
                 "out_tables must be C-contiguous int32 [B, bt_stride]")
        _require(positions.dtype == np.int32 and positions.shape == (B,) and positions.flags.c_contiguous,
                 "out_positions must be contiguous int32 [B]")
        cow = np.empty((2, max(B, 1)), dtype=np.int32)
        n_cow = ctypes.c_int32(0)
        _check(self._lib.pkv_bm_append_batch(self._h, _np_ptr(ids), B, _np_ptr(tables), int(bt_stride),
                                             _np_ptr(positions), _np_ptr(cow[0]), _np_ptr(cow[1]),
                                             ctypes.byref(n_cow)), "bm_append_batch")
        return tables, positions, np.ascontiguousarray(cow[:, :n_cow.value].T)

    def free_sequence(self, seq_id: int) -> None:
        _check(self._lib.pkv_bm_free_sequence(self._h, int(seq_id)), "bm_free_sequence")

    def num_free_blocks(self) -> int:
        return int(self._lib.pkv_bm_num_free_blocks(self._h))

    def num_sequences(self) -> int:
        return int(self._lib.pkv_bm_num_sequences(self._h))

    def sequence_length(self, seq_id: int) -> int:
        return int(self._lib.pkv_bm_sequence_length(self._h, int(seq_id)))

    def block_refcount(self, block: int) -> int:
        return int(self._lib.pkv_bm_block_refcount(self._h, int(block)))

    def block_table(self, seq_id: int):
        import numpy as np
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_bm_block_table(self._h, int(seq_id), None, 0, ctypes.byref(n)), "bm_block_table")
        table = np.empty(max(n.value, 1), dtype=np.int32)
        _check(self._lib.pkv_bm_block_table(self._h, int(seq_id), _np_ptr(table), n.value, ctypes.byref(n)),
               "bm_block_table")
        return table[:n.value]

    def batch_tables(self, seq_ids, bt_stride: int):
        """Returns (tables int32 [B, bt_stride], context_lens int32 [B]) without changing anything."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        B = ids.shape[0]
        tables = np.empty((B, bt_stride), dtype=np.int32)
        lens = np.empty(B, dtype=np.int32)
        _check(self._lib.pkv_bm_batch_tables(self._h, _np_ptr(ids), B, _np_ptr(tables), int(bt_stride),
                                             _np_ptr(lens)), "bm_batch_tables")
        return tables, lens


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------------------
# Step graphs (device tensors held for the object's lifetime)
# ---------------------------------------------------------------------------

def _step_desc(q, k_new, v_new, k_pool, v_pool, block_tables, positions, out, scale, max_batch, max_ctx,
               partition_size, cow_src, cow_dst, workspace, k_scale, v_scale):
    """A ``StepDesc`` over torch buffers sized for max_batch rows (checked), and the tensors it points into."""
    torch = _torch()
    lowp = k_scale is not None                  # FP8 (float32 scales) or MXFP4 (uint8 scales)
    mx4 = lowp and k_scale.dtype == torch.uint8
    fp8 = lowp and not mx4
    n_blocks, H_kv, bs, D = (_mx4_pools(k_pool, v_pool, k_scale, v_scale) if mx4
                             else _fp8_pools(k_pool, v_pool, k_scale, v_scale) if fp8
                             else _pool_dims(k_pool, v_pool))
    Bmax, H_q = q.shape[0], q.shape[1]
    _require(max_batch <= Bmax, "batch capacities must fit the buffers' rows")
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _require(t.dtype == (q.dtype if lowp else k_pool.dtype),
                 f"{nm} dtype must match the pools (q's for FP8 / MXFP4)")
    qrs = _rows(q, "q", H_q, D)
    nrs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == nrs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _require(block_tables.shape[0] >= max_batch, "block_tables needs a row per batch slot")
    _int32_1d(positions, "positions", positions.shape[0])
    _require(positions.shape[0] >= max_batch, "positions needs an entry per batch slot")
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape[1:]) == (H_q, D)
             and out.shape[0] >= max_batch, "out must be contiguous float32 [>= max batch cap, H_q, D]")
    if (cow_src is None) != (cow_dst is None):
        raise PkvError(-2, "cow_src and cow_dst go together")
    if cow_src is not None:
        for t, nm in ((cow_src, "cow_src"), (cow_dst, "cow_dst")):
            _int32_1d(t, nm, t.shape[0])
            _require(t.shape[0] >= max_batch, f"{nm} needs an entry per batch slot")
    need = decode_workspace_bytes(max_batch, H_q, D, max_ctx, partition_size) if partition_size and max_batch else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    keep = (q, k_new, v_new, k_pool, v_pool, block_tables, positions, out, cow_src, cow_dst, workspace, k_scale,
            v_scale)
    d = StepDesc()
    d.dtype, d.H_q, d.H_kv, d.D, d.block_size, d.n_blocks = _dtype_code(q), H_q, H_kv, D, bs, n_blocks
    d.scale, d.partition_size = float(scale), int(partition_size)
    d.out, d.q, d.q_row_stride = out.data_ptr(), q.data_ptr(), qrs
    d.k_new, d.v_new, d.new_row_stride = k_new.data_ptr(), v_new.data_ptr(), nrs
    d.k_pool, d.v_pool = k_pool.data_ptr(), v_pool.data_ptr()
    d.block_tables, d.bt_stride, d.positions = block_tables.data_ptr(), bts, positions.data_ptr()
    d.cow_src = cow_src.data_ptr() if cow_src is not None else None
    d.cow_dst = cow_dst.data_ptr() if cow_dst is not None else None
    d.workspace = workspace.data_ptr() if workspace is not None else None
    d.workspace_bytes = workspace.numel() if workspace is not None else 0
    d.k_scale = k_scale.data_ptr() if fp8 else None
    d.v_scale = v_scale.data_ptr() if fp8 else None
    d.k_mx_scale = k_scale.data_ptr() if mx4 else None
    d.v_mx_scale = v_scale.data_ptr() if mx4 else None
    return d, keep


class StepGraphs:
    """The fused decode step captured once per (batch capacity, context capacity).

    Buffers are torch device tensors sized for the largest capacities; this
    object keeps references to them so their addresses stay valid.  Before each
    ``launch(B, max_context_len)`` the caller writes the step's rows into them;
    ``positions`` rows from B up to the chosen batch capacity must be -1, and
    unused copy pairs -1.
    """

    def __init__(self, q, k_new, v_new, k_pool, v_pool, block_tables, positions, out, scale: float,
                 batch_caps, ctx_caps, *, partition_size: int = 0, cow_src=None, cow_dst=None, workspace=None,
                 k_scale=None, v_scale=None):
        bcaps = [int(x) for x in batch_caps]
        ccaps = [int(x) for x in ctx_caps]
        _require(bcaps and ccaps, "capacity lists must not be empty")
        d, keep = _step_desc(q, k_new, v_new, k_pool, v_pool, block_tables, positions, out, scale, bcaps[-1],
                             ccaps[-1], partition_size, cow_src, cow_dst, workspace, k_scale, v_scale)
        self._keep, self._desc = keep, d
        lib = load_library()
        bc = (ctypes.c_int32 * len(bcaps))(*bcaps)
        cc = (ctypes.c_int32 * len(ccaps))(*ccaps)
        h = lib.pkv_step_graphs_create(ctypes.byref(d), ctypes.cast(bc, ctypes.c_void_p), len(bcaps),
                                       ctypes.cast(cc, ctypes.c_void_p), len(ccaps))
        if not h:
            raise PkvError(PKV_ERR_HIP, "pkv_step_graphs_create: " + lib.pkv_last_error().decode())
        self._lib, self._h = lib, ctypes.c_void_p(h)
        self.batch_caps, self.ctx_caps = bcaps, ccaps

    def launch(self, B: int, max_context_len: int, n_copies: int = 0, *, stream=None):
        _check(self._lib.pkv_step_graphs_launch(self._h, int(B), int(max_context_len), int(n_copies),
                                                _stream(stream)), "step_graphs_launch")

    def close(self):
        if getattr(self, "_h", None) is not None:
            self._lib.pkv_step_graphs_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


class DualStepGraphs:
    """A local and an offloaded attention batch per step, captured once per (local capacity,
    offloaded capacity) pair as two parallel graph branches (``parallel=False``: one after the
    other).  Each batch is a dict of the buffers ``StepGraphs`` takes (q, k_new, v_new, k_pool,
    v_pool, block_tables, positions, out, optional workspace / k_scale / v_scale), sized for
    its largest capacity, and optionally its own ``partition_size`` (else the keyword's); a
    capacity of 0 leaves that branch out."""

    def __init__(self, local: dict, offloaded: dict, scale: float, local_caps, off_caps, ctx_cap: int, *,
                 partition_size: int = 0, parallel: bool = True):
        lcaps = [int(x) for x in local_caps]
        ocaps = [int(x) for x in off_caps]
        _require(lcaps and ocaps, "capacity lists must not be empty")
        descs, keeps = [], []
        for bufs, caps in ((local, lcaps), (offloaded, ocaps)):
            d, keep = _step_desc(bufs["q"], bufs["k_new"], bufs["v_new"], bufs["k_pool"], bufs["v_pool"],
                                 bufs["block_tables"], bufs["positions"], bufs["out"], scale, caps[-1], ctx_cap,
                                 int(bufs.get("partition_size", partition_size)), None, None, bufs.get("workspace"),
                                 bufs.get("k_scale"), bufs.get("v_scale"))
            descs.append(d)
            keeps.append(keep)
        self._keep, self._descs = keeps, descs
        lib = load_library()
        lc = (ctypes.c_int32 * len(lcaps))(*lcaps)
        oc = (ctypes.c_int32 * len(ocaps))(*ocaps)
        h = lib.pkv_dual_step_graphs_create(ctypes.byref(descs[0]), ctypes.byref(descs[1]),
                                            ctypes.cast(lc, ctypes.c_void_p), len(lcaps),
                                            ctypes.cast(oc, ctypes.c_void_p), len(ocaps), int(ctx_cap),
                                            1 if parallel else 0)
        if not h:
            raise PkvError(PKV_ERR_HIP, "pkv_dual_step_graphs_create: " + lib.pkv_last_error().decode())
        self._lib, self._h = lib, ctypes.c_void_p(h)
        self.local_caps, self.off_caps, self.ctx_cap = lcaps, ocaps, int(ctx_cap)

    def launch(self, B_local: int, B_off: int, *, stream=None):
        _check(self._lib.pkv_dual_step_graphs_launch(self._h, int(B_local), int(B_off), _stream(stream)),
               "dual_step_graphs_launch")

    def close(self):
        if getattr(self, "_h", None) is not None:
            self._lib.pkv_dual_step_graphs_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


class Decoder:
    """One call per decode step (``pkv_decoder_*``): the library's block manager
    reserves the batch's slots, the metadata is staged to the device on a side
    stream, and the step runs as a graph replay (when capacity lists are given)
    or call by call.  ``block_manager`` registers, forks and frees sequences.

    q, k_new, v_new and out are device tensors with ``max_batch`` rows; before
    each step the caller writes row b for seq_ids[b].
    """

    def __init__(self, q, k_new, v_new, k_pool, v_pool, out, scale: float, bt_stride: int, *,
                 partition_size: int = 0, workspace=None, shuffle_seed: int = 0, batch_caps=None, ctx_caps=None,
                 k_scale=None, v_scale=None):
        torch = _torch()
        lowp = k_scale is not None                  # FP8 (float32 scales) or MXFP4 (uint8 scales)
        mx4 = lowp and k_scale.dtype == torch.uint8
        fp8 = lowp and not mx4
        n_blocks, H_kv, bs, D = (_mx4_pools(k_pool, v_pool, k_scale, v_scale) if mx4
                                 else _fp8_pools(k_pool, v_pool, k_scale, v_scale) if fp8
                                 else _pool_dims(k_pool, v_pool))
        max_batch, H_q = q.shape[0], q.shape[1]
        for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
            _require(t.dtype == (q.dtype if lowp else k_pool.dtype) and t.shape[0] == max_batch,
                     f"{nm}: pool dtype (q's for FP8 / MXFP4), max_batch rows")
        qrs = _rows(q, "q", H_q, D)
        nrs = _rows(k_new, "k_new", H_kv, D)
        _require(_rows(v_new, "v_new", H_kv, D) == nrs, "k_new and v_new must share a row stride")
        _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (max_batch, H_q, D),
                 "out must be contiguous float32 [max_batch, H_q, D]")
        if partition_size and workspace is None:
            need = decode_workspace_bytes(max_batch, H_q, D, bt_stride * bs, partition_size)
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        self._keep = (q, k_new, v_new, k_pool, v_pool, out, workspace, k_scale, v_scale)
        d = DecoderDesc()
        d.dtype, d.H_q, d.H_kv, d.D, d.block_size, d.n_blocks = _dtype_code(q), H_q, H_kv, D, bs, n_blocks
        d.scale, d.partition_size, d.max_batch, d.bt_stride = float(scale), int(partition_size), max_batch, bt_stride
        d.out, d.q, d.q_row_stride = out.data_ptr(), q.data_ptr(), qrs
        d.k_new, d.v_new, d.new_row_stride = k_new.data_ptr(), v_new.data_ptr(), nrs
        d.k_pool, d.v_pool = k_pool.data_ptr(), v_pool.data_ptr()
        d.workspace = workspace.data_ptr() if workspace is not None else None
        d.workspace_bytes = workspace.numel() if workspace is not None else 0
        d.shuffle_seed = int(shuffle_seed) & ((1 << 64) - 1)
        d.k_scale = k_scale.data_ptr() if fp8 else None
        d.v_scale = v_scale.data_ptr() if fp8 else None
        d.k_mx_scale = k_scale.data_ptr() if mx4 else None
        d.v_mx_scale = v_scale.data_ptr() if mx4 else None
        self._caps = None
        if batch_caps is not None:
            bc = (ctypes.c_int32 * len(batch_caps))(*[int(x) for x in batch_caps])
            cc = (ctypes.c_int32 * len(ctx_caps))(*[int(x) for x in ctx_caps])
            self._caps = (bc, cc)
            d.batch_caps, d.n_batch_caps = ctypes.cast(bc, ctypes.c_void_p), len(batch_caps)
            d.ctx_caps, d.n_ctx_caps = ctypes.cast(cc, ctypes.c_void_p), len(ctx_caps)
        lib = load_library()
        h = lib.pkv_decoder_create(ctypes.byref(d))
        if not h:
            raise PkvError(PKV_ERR_HIP, "pkv_decoder_create: " + lib.pkv_last_error().decode())
        self._lib, self._h = lib, ctypes.c_void_p(h)
        self.max_batch, self.bt_stride = max_batch, bt_stride
        self.block_manager = BlockManager(n_blocks, bs, _borrow=(lib.pkv_decoder_block_manager(self._h), self))
        self._ids = None

    def step(self, seq_ids, *, stream=None) -> int:
        """Enqueue one decode step for seq_ids; returns the number of copy-on-write block copies."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_decoder_step(self._h, _np_ptr(ids), ids.shape[0], _stream(stream), ctypes.byref(n)),
               "decoder_step")
        return n.value

    def close(self):
        if getattr(self, "_h", None) is not None:
            self.block_manager.close()
            self._lib.pkv_decoder_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


# ---------------------------------------------------------------------------
# CU-limited streams
# ---------------------------------------------------------------------------

def device_cu_count() -> int:
    n = int(load_library().pkv_device_cu_count())
    if n < 0:
        _check(n, "device_cu_count")
    return n


def cu_mask(n_cus: int, count: int, layout: str = "spread"):
    """uint32 words selecting `count` of `n_cus` CUs: 'first' = CUs 0..count-1, 'spread' = evenly strided."""
    import numpy as np
    words = (n_cus + 31) // 32
    mask = np.zeros(words, dtype=np.uint32)
    _check(load_library().pkv_cu_mask(int(n_cus), int(count), {"first": 0, "spread": 1}[layout], _np_ptr(mask),
                                      words), "cu_mask")
    return mask


class CuMaskedStream:
    """A HIP stream restricted to the CUs of ``mask``; ``.torch`` is the same stream as a torch.cuda.ExternalStream
    (for torch work on it), ``.ptr`` the raw hipStream_t for the library's ``stream=`` arguments."""

    def __init__(self, mask):
        import numpy as np
        m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint32))
        out = ctypes.c_void_p()
        lib = load_library()
        _check(lib.pkv_stream_create_cu_masked(_np_ptr(m), m.shape[0], ctypes.byref(out)), "stream_create_cu_masked")
        self._lib, self.ptr = lib, out.value
        self.mask = m
        self.torch = _torch().cuda.ExternalStream(self.ptr)

    @property
    def cuda_stream(self):
        return self.ptr

    def close(self):
        if getattr(self, "ptr", None):
            _torch().cuda.synchronize()
            self._lib.pkv_stream_destroy(ctypes.c_void_p(self.ptr))
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) K/V cache: uint8 code pools plus float32 per-row scales
# ---------------------------------------------------------------------------

def _fp8_pools(k_pool, v_pool, k_scale, v_scale):
    torch = _torch()
    _require(k_pool.dtype == torch.uint8 and v_pool.dtype == torch.uint8, "FP8 pools are uint8 codes")
    n_blocks, H_kv, bs, D = _pool_dims(k_pool, v_pool)
    for t, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _require(t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == (n_blocks, H_kv, bs),
                 f"{nm} must be contiguous float32 [n_blocks, H_kv, block_size]")
    return n_blocks, H_kv, bs, D


def kv_append_fp8(k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions, *, stream=None):
    """Quantize k_new/v_new [B, H_kv, D] (f32/f16/bf16) into slot positions[b] of each request's block."""
    n_blocks, H_kv, bs, D = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    B = k_new.shape[0]
    _require(v_new.dtype == k_new.dtype, "k_new and v_new dtypes differ")
    rs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == rs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    rc = load_library().pkv_kv_append_fp8(_dtype_code(k_new), _ptr(k_new), _ptr(v_new), rs, _ptr(k_pool),
                                          _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), bts,
                                          _ptr(positions), B, H_kv, D, bs, n_blocks, _stream(stream))
    _check(rc, "kv_append_fp8")


def paged_decode_attention_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, scale: float,
                               max_context_len: int, *, partition_size: int = 0, out=None, workspace=None,
                               stream=None):
    """paged_decode_attention over FP8 pools; q in f32/f16/bf16, output float32."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    B, H_q = q.shape[0], q.shape[1]
    qrs = _rows(q, "q", H_q, D)
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(context_lens, "context_lens", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    ws, ws_bytes = _workspace(B, H_q, D, max_context_len, partition_size, workspace, q.device)
    rc = load_library().pkv_paged_decode_attention_fp8(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), bts, _ptr(context_lens), B, H_q, H_kv, D, bs, n_blocks, int(max_context_len),
        float(scale), int(partition_size), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "paged_decode_attention_fp8")
    return out


def append_decode_attention_fp8(q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions,
                                scale: float, max_context_len: int, *, partition_size: int = 0, out=None,
                                workspace=None, stream=None):
    """One decode step over FP8 pools: quantize and write the new rows, attend over positions[b] + 1 tokens."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    B, H_q = q.shape[0], q.shape[1]
    _require(k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new/v_new dtype must match q")
    qrs = _rows(q, "q", H_q, D)
    nrs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == nrs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    ws, ws_bytes = _workspace(B, H_q, D, max_context_len, partition_size, workspace, q.device)
    rc = load_library().pkv_append_decode_attention_fp8(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_new), _ptr(v_new), nrs, _ptr(k_pool), _ptr(v_pool),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), bts, _ptr(positions), B, H_q, H_kv, D, bs, n_blocks,
        int(max_context_len), float(scale), int(partition_size), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "append_decode_attention_fp8")
    return out


def copy_blocks_fp8(k_pool, v_pool, k_scale, v_scale, src, dst, *, stream=None):
    """copy_blocks for an FP8 cache: codes and row scales of blocks src[i] -> dst[i]."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    n = src.shape[0]
    for t, nm in ((src, "src"), (dst, "dst")):
        _require(t.dtype == torch.int32 and t.dim() == 1 and t.shape[0] == n and (n <= 1 or t.stride(0) == 1),
                 f"{nm} must be contiguous int32 [n]")
    rc = load_library().pkv_copy_blocks_fp8(_ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(src),
                                            _ptr(dst), n, H_kv, D, bs, n_blocks, _stream(stream))
    _check(rc, "copy_blocks_fp8")


# ---------------------------------------------------------------------------
# MXFP4 K/V cache: E2M1 codes two per byte plus one E8M0 scale byte per 32 elements
# ---------------------------------------------------------------------------

def _mx4_pools(k_pool, v_pool, k_scale, v_scale):
    """(n_blocks, H_kv, block_size, D) of MXFP4 pools: codes [.., D/2] and scales [.., D/32], all uint8."""
    torch = _torch()
    _require(k_pool.dtype == torch.uint8 and v_pool.dtype == torch.uint8, "MXFP4 pools are uint8 code bytes")
    n_blocks, H_kv, bs, half = _pool_dims(k_pool, v_pool)
    D = 2 * half
    for t, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _require(t.dtype == torch.uint8 and t.is_contiguous() and tuple(t.shape) == (n_blocks, H_kv, bs, D // 32),
                 f"{nm} must be contiguous uint8 [n_blocks, H_kv, block_size, D/32]")
    return n_blocks, H_kv, bs, D


def copy_blocks_mxfp4(k_pool, v_pool, k_scale, v_scale, src, dst, *, stream=None):
    """copy_blocks for an MXFP4 cache: code and scale bytes of blocks src[i] -> dst[i]."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _mx4_pools(k_pool, v_pool, k_scale, v_scale)
    n = src.shape[0]
    for t, nm in ((src, "src"), (dst, "dst")):
        _require(t.dtype == torch.int32 and t.dim() == 1 and t.shape[0] == n and (n <= 1 or t.stride(0) == 1),
                 f"{nm} must be contiguous int32 [n]")
    rc = load_library().pkv_copy_blocks_mxfp4(_ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(src),
                                              _ptr(dst), n, H_kv, D, bs, n_blocks, _stream(stream))
    _check(rc, "copy_blocks_mxfp4")


def kv_append_mxfp4(k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions, *, stream=None):
    """Quantize k_new/v_new [B, H_kv, D] (f32/f16/bf16) to MXFP4 into slot positions[b] of each request's block."""
    n_blocks, H_kv, bs, D = _mx4_pools(k_pool, v_pool, k_scale, v_scale)
    B = k_new.shape[0]
    _require(v_new.dtype == k_new.dtype, "k_new and v_new dtypes differ")
    rs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == rs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    rc = load_library().pkv_kv_append_mxfp4(_dtype_code(k_new), _ptr(k_new), _ptr(v_new), rs, _ptr(k_pool),
                                            _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), bts,
                                            _ptr(positions), B, H_kv, D, bs, n_blocks, _stream(stream))
    _check(rc, "kv_append_mxfp4")


def paged_decode_attention_mxfp4(q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, scale: float,
                                 max_context_len: int, *, partition_size: int = 0, out=None, workspace=None,
                                 stream=None):
    """paged_decode_attention over MXFP4 pools; q in f32/f16/bf16, output float32."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _mx4_pools(k_pool, v_pool, k_scale, v_scale)
    B, H_q = q.shape[0], q.shape[1]
    qrs = _rows(q, "q", H_q, D)
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(context_lens, "context_lens", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    ws, ws_bytes = _workspace(B, H_q, D, max_context_len, partition_size, workspace, q.device)
    rc = load_library().pkv_paged_decode_attention_mxfp4(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), bts, _ptr(context_lens), B, H_q, H_kv, D, bs, n_blocks, int(max_context_len),
        float(scale), int(partition_size), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "paged_decode_attention_mxfp4")
    return out


def append_decode_attention_mxfp4(q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables, positions,
                                  scale: float, max_context_len: int, *, partition_size: int = 0, out=None,
                                  workspace=None, stream=None):
    """One decode step over MXFP4 pools: quantize and write the new rows, attend over positions[b] + 1 tokens."""
    torch = _torch()
    n_blocks, H_kv, bs, D = _mx4_pools(k_pool, v_pool, k_scale, v_scale)
    B, H_q = q.shape[0], q.shape[1]
    _require(k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new/v_new dtype must match q")
    qrs = _rows(q, "q", H_q, D)
    nrs = _rows(k_new, "k_new", H_kv, D)
    _require(_rows(v_new, "v_new", H_kv, D) == nrs, "k_new and v_new must share a row stride")
    bts = _int32_2d(block_tables, "block_tables")
    _int32_1d(positions, "positions", B)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, H_q, D),
             "out must be contiguous float32 [B, H_q, D]")
    ws, ws_bytes = _workspace(B, H_q, D, max_context_len, partition_size, workspace, q.device)
    rc = load_library().pkv_append_decode_attention_mxfp4(
        _dtype_code(q), _ptr(out), _ptr(q), qrs, _ptr(k_new), _ptr(v_new), nrs, _ptr(k_pool), _ptr(v_pool),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), bts, _ptr(positions), B, H_q, H_kv, D, bs, n_blocks,
        int(max_context_len), float(scale), int(partition_size), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "append_decode_attention_mxfp4")
    return out
