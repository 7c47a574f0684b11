"""Seeded synthetic decode-step inputs for paged-KV decode attention.

This module is shared by the fp64 oracle (``oracle/``) and the HIP path
(``paged_kv_decode_blocks_amd``).  It holds no part of the method's arithmetic:
it only draws random values and lays them out as a paged KV pool with
per-request block tables, the structure described by
"从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2 (fixed-size
physical blocks, one page table per request, blocks placed anywhere in the
pool).  Whatever scores, softmax, weighted sums or appends are done with these
buffers happens in ``oracle/`` or in the HIP kernels.

Storage dtypes on the host:
  f32  -> numpy.float32
  f16  -> numpy.float16
  bf16 -> numpy.uint16 (raw bfloat16 bit patterns)

Every slot of the pool that holds no valid token (unassigned blocks, slots at
or past a request's history length, the slot the step's append will fill) is a
quiet NaN, so any stray read shows up in the output.

FP8 K/V workloads (``kv_dtype="fp8"``) hold OCP E4M3 codes (uint8) and one
float32 scale per (block, KV head, slot).  The generator draws codes and scales
directly -- codes with exponent fields concentrated around 12.5 (spread 1.6),
uniform mantissas and signs, so a row looks like a quantized Gaussian whose
largest values sit near the top of the E4M3 range; scales 2^k with k uniform in
[-12, -8] -- and never quantizes anything.  Their poison is the NaN code 0x7F
with a NaN scale.  q, k_new and v_new keep ``dtype``.

MXFP4 K/V workloads (``kv_dtype="mxfp4"``) hold E2M1 codes two per byte
(element 2k in the low nibble of byte k) and one E8M0 scale byte per 32
elements of a row ([n_blocks][H_kv][slot][D/2] and [n_blocks][H_kv][slot][D/32]
uint8).  The generator draws code bytes uniformly (every 4-bit code is finite)
and scale bytes 2^k with k uniform in [-5, -1], and never quantizes anything.
Their poison is a NaN scale byte (0xFF) over code bytes 0x77.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Config", "Workload", "CONFIGS", "get_config", "make_workload", "draw_lengths",
    "DTYPE_BYTES", "NAN_BITS", "to_storage", "storage_dtype",
    "kv_bytes_per_token", "step_bytes", "draw_e4m3_codes", "make_peaked_workload",
]

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# quiet-NaN bit patterns used as poison in each storage dtype
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


def storage_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values once to the storage dtype (RNE)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32.copy()
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return _f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def _poison(dtype: str):
    if dtype == "f32":
        return np.uint32(NAN_BITS["f32"]).view(np.float32)
    if dtype == "f16":
        return np.uint16(NAN_BITS["f16"]).view(np.float16)
    return np.uint16(NAN_BITS["bf16"])


@dataclass(frozen=True)
class Config:
    """One synthetic decode workload (a single attention layer's decode step)."""
    name: str
    title: str
    B: int
    H_q: int
    H_kv: int
    D: int
    dtype: str
    block_size: int
    lengths: Tuple            # ("fixed", (..)) | ("const", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    pool: Tuple               # ("blocks", N) | ("factor", f)
    q_std: float = 1.0
    kv_std: float = 1.0
    append: bool = False      # the step appends one new token per request before attention
    partition_size: int = 0   # split-KV partition length in tokens (0 = whole context per workgroup)
    kv_dtype: str = ""        # "" = same as dtype; "fp8" = OCP E4M3 codes with per-row scales;
                              # "mxfp4" = E2M1 codes with an E8M0 scale per 32 elements

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def fp8(self) -> bool:
        return self.kv_dtype == "fp8"

    @property
    def mxfp4(self) -> bool:
        return self.kv_dtype == "mxfp4"


# The five workloads.  Shapes, dtypes, length mixes and pool sizes follow the
# decode batches the Adrenaline review profiles (Llama-2 7B/13B-shaped layers,
# batches of 8 to 80) plus a grouped-query long-context case.
CONFIGS = {
    "c1": Config("c1", "tiny paged decode (B2, 2 heads MHA, D64, f32, ctx {5,37}, 8-block pool, append)",
                 B=2, H_q=2, H_kv=2, D=64, dtype="f32", block_size=16,
                 lengths=("fixed", (5, 37)), pool=("blocks", 8), append=True),
    "c2": Config("c2", "Llama-2-7B-shaped layer decode (B8, 32 heads MHA, D128, f16, ctx 1024)",
                 B=8, H_q=32, H_kv=32, D=128, dtype="f16", block_size=16,
                 lengths=("const", 1024), pool=("factor", 2.0)),
    "c3": Config("c3", "large decode batch (B80, 32 heads MHA, D128, f16, ctx U[128,2048], append)",
                 B=80, H_q=32, H_kv=32, D=128, dtype="f16", block_size=16,
                 lengths=("uniform", 128, 2048), pool=("factor", 1.5), append=True),
    "c4": Config("c4", "Llama-2-13B-shaped (B64, 40 heads MHA, D128, bf16, ctx logU[512,4096], split 512)",
                 B=64, H_q=40, H_kv=40, D=128, dtype="bf16", block_size=16,
                 lengths=("loguniform", 512, 4096), pool=("factor", 1.5), kv_std=0.5,
                 partition_size=512),
    "c5": Config("c5", "GQA long context (B32, 64 q / 8 kv heads, D128, bf16, ctx U[4096,16384], split 1024)",
                 B=32, H_q=64, H_kv=8, D=128, dtype="bf16", block_size=16,
                 lengths=("uniform", 4096, 16384), pool=("factor", 1.2), partition_size=1024),
}
# the same decode batches with an FP8 K/V cache (q, new rows and output keep their dtype)
CONFIGS["c3f8"] = replace(CONFIGS["c3"], name="c3f8", kv_dtype="fp8",
                          title="large decode batch, FP8 E4M3 K/V (B80, 32 heads MHA, D128, f16 q, ctx U[128,2048], "
                                "append)")
CONFIGS["c5f8"] = replace(CONFIGS["c5"], name="c5f8", kv_dtype="fp8",
                          title="GQA long context, FP8 E4M3 K/V (B32, 64 q / 8 kv heads, D128, bf16 q, "
                                "ctx U[4096,16384], split 1024)")
# and with an MXFP4 K/V cache
CONFIGS["c3f4"] = replace(CONFIGS["c3"], name="c3f4", kv_dtype="mxfp4",
                          title="large decode batch, MXFP4 K/V (B80, 32 heads MHA, D128, f16 q, ctx U[128,2048], "
                                "append)")
CONFIGS["c5f4"] = replace(CONFIGS["c5"], name="c5f4", kv_dtype="mxfp4",
                          title="GQA long context, MXFP4 K/V (B32, 64 q / 8 kv heads, D128, bf16 q, "
                                "ctx U[4096,16384], split 1024)")


def draw_e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """E4M3 codes shaped like a quantized Gaussian row (never the NaN code)."""
    ex = np.clip(np.rint(rng.normal(12.5, 1.6, shape)), 0, 15).astype(np.uint8)
    man = rng.integers(0, 8, shape).astype(np.uint8)
    man = np.where((ex == 15) & (man == 7), 6, man).astype(np.uint8)
    sign = rng.integers(0, 2, shape).astype(np.uint8)
    return ((sign << 7) | (ex << 3) | man).astype(np.uint8)


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


@dataclass
class Workload:
    cfg: Config
    seed: int
    context_lens: np.ndarray          # int32 [B]: tokens attention reads (after the append, if any)
    positions: Optional[np.ndarray]   # int32 [B]: slot index of the appended token (= context_lens-1), or None
    block_tables: np.ndarray          # int32 [B, W], -1 padding
    n_blocks: int
    q: np.ndarray                     # [B, H_q, D] storage dtype
    k_pool: np.ndarray                # [n_blocks, H_kv, bs, D] storage dtype
    v_pool: np.ndarray
    k_new: Optional[np.ndarray]       # [B, H_kv, D] storage dtype (append only)
    v_new: Optional[np.ndarray]
    scale: np.float32
    meta: dict = field(default_factory=dict)
    k_scale: Optional[np.ndarray] = None   # FP8 pools only: [n_blocks, H_kv, bs] float32
    v_scale: Optional[np.ndarray] = None

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def history_lens(self) -> np.ndarray:
        """Tokens already in the pool before the step (context_lens-1 with append)."""
        return self.context_lens - 1 if self.positions is not None else self.context_lens


def draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Context lengths of one batch (the first draw make_workload takes from its generator)."""
    kind = cfg.lengths[0]
    if kind == "fixed":
        n = np.array(cfg.lengths[1], dtype=np.int64)
        assert n.size == cfg.B
    elif kind == "const":
        n = np.full(cfg.B, cfg.lengths[1], dtype=np.int64)
    elif kind == "uniform":
        lo, hi = cfg.lengths[1], cfg.lengths[2]
        n = rng.integers(lo, hi + 1, size=cfg.B, dtype=np.int64)
    elif kind == "loguniform":
        lo, hi = cfg.lengths[1], cfg.lengths[2]
        u = rng.uniform(math.log(lo), math.log(hi + 1), size=cfg.B)
        n = np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int64)
    else:
        raise ValueError(kind)
    return n.astype(np.int32)


def make_workload(cfg: Config, seed: Optional[int] = None, *, append: Optional[bool] = None,
                  lengths: Optional[np.ndarray] = None) -> Workload:
    """Draw one decode step's inputs.

    Draw order: lengths -> block permutation -> q -> K history -> V history ->
    k_new -> v_new.  ``context_lens`` is what attention reads; with
    ``append`` the last of those tokens is the one the step appends (its pool
    slot is poison until the append writes it).
    """
    if seed is None:
        seed = int(cfg.name[1:]) if cfg.name[1:].isdigit() else 0
    if append is None:
        append = cfg.append
    rng = np.random.default_rng(seed)
    bs, H_kv, D = cfg.block_size, cfg.H_kv, cfg.D

    ctx = draw_lengths(cfg, rng) if lengths is None else np.asarray(lengths, dtype=np.int32)
    B = ctx.size
    hist = ctx - 1 if append else ctx.copy()
    if append and np.any(ctx < 1):
        raise ValueError("append needs context_lens >= 1")
    nb = (ctx.astype(np.int64) + bs - 1) // bs      # blocks each request holds for this step
    required = int(nb.sum())
    if cfg.pool[0] == "blocks":
        n_blocks = int(cfg.pool[1])
    else:
        n_blocks = int(math.ceil(cfg.pool[1] * required))
    n_blocks = max(n_blocks, required, 1)
    W = max(int(nb.max()) if B else 0, 1)

    perm = rng.permutation(n_blocks).astype(np.int32)
    bt = np.full((B, W), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :nb[b]] = perm[off:off + nb[b]]
        off += int(nb[b])

    sdt = storage_dtype(cfg.dtype)
    q = to_storage(cfg.q_std * rng.standard_normal((B, cfg.H_q, D), dtype=np.float32), cfg.dtype)

    poison = _poison(cfg.dtype)
    pools, scales = [], []
    for _ in range(2):  # K then V (FP8, MXFP4: codes then scales for each)
        if cfg.fp8:
            pool = np.full((n_blocks, H_kv, bs, D), 0x7F, dtype=np.uint8)
            sc = np.full((n_blocks, H_kv, bs), np.nan, dtype=np.float32)
        elif cfg.mxfp4:
            pool = np.full((n_blocks, H_kv, bs, D // 2), 0x77, dtype=np.uint8)
            sc = np.full((n_blocks, H_kv, bs, D // 32), 0xFF, dtype=np.uint8)
        else:
            pool = np.full((n_blocks, H_kv, bs, D), poison, dtype=sdt)
        for b in range(B):
            h = int(hist[b])
            full, rem = divmod(h, bs)
            nfill = full + (1 if rem else 0)
            if nfill == 0:
                continue
            ids = bt[b, :nfill]
            if cfg.fp8:
                vals = draw_e4m3_codes(rng, (nfill, H_kv, bs, D))
                svals = (2.0 ** rng.integers(-12, -7, (nfill, H_kv, bs))).astype(np.float32)
                if rem:
                    vals[-1, :, rem:, :] = 0x7F
                    svals[-1, :, rem:] = np.nan
                pool[ids] = vals
                sc[ids] = svals
            elif cfg.mxfp4:
                vals = rng.integers(0, 256, (nfill, H_kv, bs, D // 2), dtype=np.uint8)
                svals = rng.integers(127 - 5, 127, (nfill, H_kv, bs, D // 32), dtype=np.uint8)
                if rem:
                    vals[-1, :, rem:, :] = 0x77
                    svals[-1, :, rem:, :] = 0xFF
                pool[ids] = vals
                sc[ids] = svals
            else:
                vals = cfg.kv_std * rng.standard_normal((nfill, H_kv, bs, D), dtype=np.float32)
                vals = to_storage(vals, cfg.dtype)
                if rem:
                    vals[-1, :, rem:, :] = poison
                pool[ids] = vals
        pools.append(pool)
        if cfg.fp8 or cfg.mxfp4:
            scales.append(sc)
    k_pool, v_pool = pools
    k_scale, v_scale = scales if (cfg.fp8 or cfg.mxfp4) else (None, None)

    k_new = v_new = positions = None
    if append:
        positions = (ctx - 1).astype(np.int32)
        k_new = to_storage(cfg.kv_std * rng.standard_normal((B, H_kv, D), dtype=np.float32), cfg.dtype)
        v_new = to_storage(cfg.kv_std * rng.standard_normal((B, H_kv, D), dtype=np.float32), cfg.dtype)

    scale = np.float32(1.0 / math.sqrt(D))
    return Workload(cfg=cfg, seed=seed, context_lens=ctx, positions=positions, block_tables=bt,
                    n_blocks=n_blocks, q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
                    scale=scale, meta={"required_blocks": required}, k_scale=k_scale, v_scale=v_scale)


def make_peaked_workload(cfg: Config, seed: int, *, period: int = 512, rise_log2: float = 64.0,
                         dominant_first=(), dominant_last=(), dominant_log2: float = 96.0) -> Workload:
    """Decode-step inputs whose scores climb steeply along each context.

    Built for the online softmax's rescaling: where the running maximum of a
    head's scores grows by many binary orders within a pass, every weight and
    partial sum already accumulated must be scaled down.  The layout (lengths,
    tables, poison, draw of the first values) is ``make_workload``'s; then, from
    a second generator seeded with (seed, 0x5EA4), per request b and KV head g:

      u ~ N(0, 1)^D                                a direction
      q_h = u + 0.3 n_h  for even h in the group   "climbing" heads
      q_h = n_h          for odd h                  heads that see only noise
      k_t = z_t + a(t) u / |u|,   z_t ~ N(0, 1)^D
      a(t) = ln2 * rise_log2 * ((t mod period) / period) / (scale |u|)

    so a climbing head's score of token t is about ln2 * rise_log2 * (t mod
    period) / period plus unit noise: in binary orders, a sawtooth that rises by
    ``rise_log2`` over each ``period`` tokens.  Token 0 of each request in
    ``dominant_first`` and the last token (the appended one, with append) of
    each in ``dominant_last`` instead get a(t) for rise_log2 + dominant_log2
    orders: they outweigh every other token of a climbing head by about
    2^dominant_log2.  V rows (and v_new) ~ N(0, 1)^D.  Values are drawn in
    float32 and rounded once to ``cfg.dtype``.

    FP8 or MXFP4 configs get the same rows in ``cfg.dtype`` storage (this module
    never quantizes): the returned workload's config has ``kv_dtype=""``.
    """
    base = replace(cfg, kv_dtype="")
    w = make_workload(base, seed)
    rng = np.random.default_rng([seed, 0x5EA4])
    bs, H_kv, D, G = cfg.block_size, cfg.H_kv, cfg.D, cfg.G
    B = w.context_lens.size
    scale = float(w.scale)
    ln2 = math.log(2.0)
    q = np.empty((B, cfg.H_q, D), dtype=np.float32)
    kp = w.k_pool.copy()
    vp = w.v_pool.copy()
    k_new = np.empty((B, H_kv, D), dtype=np.float32)
    v_new = np.empty((B, H_kv, D), dtype=np.float32)
    first, last = set(int(b) for b in dominant_first), set(int(b) for b in dominant_last)
    for b in range(B):
        n = int(w.context_lens[b])
        hist = n - 1 if w.positions is not None else n
        t = np.arange(n)
        for g in range(H_kv):
            u = rng.standard_normal(D).astype(np.float64)
            un = float(np.sqrt(u @ u))
            for hh in range(G):
                nh = rng.standard_normal(D)
                q[b, g * G + hh] = (u + 0.3 * nh) if hh % 2 == 0 else nh
            orders = rise_log2 * (t % period) / period
            if b in first and n > 0:
                orders[0] = rise_log2 + dominant_log2
            if b in last and n > 0:
                orders[n - 1] = rise_log2 + dominant_log2
            a = ln2 * orders / (scale * un)
            krows = rng.standard_normal((n, D)) + a[:, None] * (u / un)[None, :]
            vrows = rng.standard_normal((n, D))
            if hist > 0:
                x = np.arange(hist)
                blk, slot = w.block_tables[b, x // bs], x % bs
                kp[blk, g, slot] = to_storage(krows[:hist], cfg.dtype)
                vp[blk, g, slot] = to_storage(vrows[:hist], cfg.dtype)
            if w.positions is not None:
                k_new[b, g] = krows[n - 1]
                v_new[b, g] = vrows[n - 1]
    w.q = to_storage(q, cfg.dtype)
    w.k_pool, w.v_pool = kp, vp
    if w.positions is not None:
        w.k_new, w.v_new = to_storage(k_new, cfg.dtype), to_storage(v_new, cfg.dtype)
    w.meta.update(peaked=dict(period=period, rise_log2=rise_log2, dominant_first=sorted(first),
                              dominant_last=sorted(last), dominant_log2=dominant_log2))
    return w


# ---------------------------------------------------------------------------
# Byte accounting for the bandwidth roofline (measurement, not the method).
# ---------------------------------------------------------------------------

def kv_bytes_per_token(H_kv: int, D: int, elem_bytes: float, layers: int = 1) -> float:
    """Bytes of K plus V that one token occupies: 2 * layers * H_kv * D * elem_bytes."""
    return 2.0 * layers * H_kv * D * elem_bytes


def step_bytes(cfg: Config, context_lens: np.ndarray, append: bool) -> dict:
    """Algorithmic HBM bytes of one decode step: what the step must move at minimum.

    History K/V read once, the new token's K/V read and written once (append),
    q read, the f32 output written, one block-table entry per block touched and
    one length word per request.  Split-KV partials, padding and re-reads are
    not algorithmic bytes.
    """
    e = DTYPE_BYTES[cfg.dtype]
    # an FP8 row is D one-byte codes plus its 4-byte scale; an MXFP4 row D/2 code bytes plus D/32 scale bytes
    if cfg.fp8:
        row = 2.0 * cfg.H_kv * (cfg.D + 4)
    elif cfg.mxfp4:
        row = 2.0 * cfg.H_kv * (cfg.D // 2 + cfg.D // 32)
    else:
        row = kv_bytes_per_token(cfg.H_kv, cfg.D, e)
    ctx = np.asarray(context_lens, dtype=np.int64)
    B = ctx.size
    hist = ctx - 1 if append else ctx
    out = {
        "kv_history": float(hist.sum() * row),
        # the new rows are read in q's dtype and written as stored
        "append": float(B * (2.0 * cfg.H_kv * cfg.D * e + row)) if append else 0.0,
        "q": float(B * cfg.H_q * cfg.D * e),
        "out": float(B * cfg.H_q * cfg.D * 4),
        "block_tables": float(((ctx + cfg.block_size - 1) // cfg.block_size).sum() * 4),
        "lengths": float(B * 4),          # context_lens, or positions in a fused step
    }
    out["total"] = sum(out.values())
    # attention alone reads every context token from the pool
    out["attention_only"] = float(ctx.sum() * row) + out["q"] + out["out"] + out["block_tables"] + B * 4
    return out
