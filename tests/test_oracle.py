"""Pins for the fp64 oracle (CPU only).

None of these re-type the oracle's formula.  They tie it to things fixed
outside it: torch's scaled_dot_product_attention in float64 on contiguous
inputs, the IEEE/bfloat16 decoders of numpy and torch, closed forms of softmax
attention, invariances that the paging definition implies (blocks may sit
anywhere and may be shared), the log-sum-exp merge identity, and a set of
planted mistakes that must each be caught.
"""
import math
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from workloads import get_config, make_workload, to_storage, NAN_BITS

DTYPES = ["f32", "f16", "bf16"]


def f64_of(dtype, bits):
    """Library decoding (numpy/torch), independent of the oracle's own decoders."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        a = np.asarray(bits)
        return (a.view(np.float16) if a.dtype == np.uint16 else a.astype(np.float16)).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def contiguous_case(rng, dtype, B, H_q, H_kv, D, lens, bs=16, extra_blocks=3):
    """Per-request contiguous K/V [n, H_kv, D] and the paged pool built from them by reshaping.

    Request b's tokens fill blocks off_b .. off_b+nb-1 in order: padding the
    [n, H_kv, D] array to nb*bs tokens, reshaping to [nb, bs, H_kv, D] and
    moving the head axis in front of the slot axis gives the pool's
    [block][head][slot][d] order without any hand-written index arithmetic.
    """
    nbs = [max(1, -(-n // bs)) for n in lens]
    n_blocks = sum(nbs) + extra_blocks
    sdt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    nan = {"f32": np.uint32(NAN_BITS["f32"]).view(np.float32), "f16": np.uint16(NAN_BITS["f16"]).view(np.float16),
           "bf16": np.uint16(NAN_BITS["bf16"])}[dtype]
    kp = np.full((n_blocks, H_kv, bs, D), nan, dtype=sdt)
    vp = np.full((n_blocks, H_kv, bs, D), nan, dtype=sdt)
    bt = np.full((B, max(nbs)), -1, dtype=np.int32)
    Ks, Vs = [], []
    off = 0
    for b, n in enumerate(lens):
        K = to_storage(rng.standard_normal((n, H_kv, D)), dtype)
        V = to_storage(rng.standard_normal((n, H_kv, D)), dtype)
        Ks.append(K)
        Vs.append(V)
        nb = nbs[b]
        for src, dst in ((K, kp), (V, vp)):
            pad = np.full((nb * bs, H_kv, D), nan, dtype=sdt)
            pad[:n] = src
            dst[off:off + nb] = pad.reshape(nb, bs, H_kv, D).transpose(0, 2, 1, 3)
        bt[b, :nb] = np.arange(off, off + nb, dtype=np.int32)
        off += nb
    q = to_storage(rng.standard_normal((B, H_q, D)), dtype)
    return q, kp, vp, bt, np.array(lens, dtype=np.int32), Ks, Vs


def sdpa_reference(dtype, q, Ks, Vs, scale, H_q, H_kv):
    """torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, request by request."""
    outs = []
    for b in range(q.shape[0]):
        n = Ks[b].shape[0]
        if n == 0:
            outs.append(np.zeros((H_q, q.shape[2])))
            continue
        qt = torch.from_numpy(f64_of(dtype, q[b]))[None, :, None, :]                     # [1,H_q,1,D]
        kt = torch.from_numpy(f64_of(dtype, Ks[b])).permute(1, 0, 2)[None].contiguous()  # [1,H_kv,n,D]
        vt = torch.from_numpy(f64_of(dtype, Vs[b])).permute(1, 0, 2)[None].contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(scale),
                                                             enable_gqa=(H_q != H_kv))
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


# ---------------------------------------------------------------------------
# decoders
# ---------------------------------------------------------------------------

def test_decode_f16_exhaustive(oracle_lib):
    bits = np.arange(1 << 16, dtype=np.uint16)
    mine = oracle.decode("f16", bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_exhaustive(oracle_lib):
    bits = np.arange(1 << 16, dtype=np.uint16)
    mine = oracle.decode("bf16", bits)
    ref = f64_of("bf16", bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_decode_f32_random_bits(oracle_lib):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    mine = oracle.decode("f32", vals)
    with np.errstate(invalid="ignore"):
        ref = vals.astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


# ---------------------------------------------------------------------------
# attention against a library routine on contiguous inputs
# ---------------------------------------------------------------------------

SHAPES = [
    # B, H_q, H_kv, D, lens
    (1, 1, 1, 8, [1]),
    (2, 2, 2, 8, [5, 37]),
    (3, 4, 4, 64, [16, 17, 40]),
    (2, 8, 2, 64, [31, 33]),       # GQA, G = 4
    (3, 4, 1, 8, [3, 16, 32]),     # MQA, G = 4
    (2, 6, 3, 16, [15, 48]),       # G = 2
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES)
def test_matches_sdpa_on_contiguous(oracle_lib, dtype, shape):
    B, H_q, H_kv, D, lens = shape
    rng = np.random.default_rng(hash((dtype, B, H_q, H_kv, D)) % (1 << 32))
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, dtype, B, H_q, H_kv, D, lens)
    scale = np.float32(1.0 / math.sqrt(D))
    got = oracle.paged_decode_attention(dtype, q, kp, vp, bt, ctx, scale)
    ref = sdpa_reference(dtype, q, Ks, Vs, scale, H_q, H_kv)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_matches_sdpa_on_generated_workload(oracle_lib):
    """c1's generated pool (random block placement) against SDPA on the gathered history."""
    w = make_workload(get_config("c1"), append=False)
    got = oracle.paged_decode_attention("f32", w.q, w.k_pool, w.v_pool, w.block_tables,
                                        w.context_lens, w.scale)
    # gather through the table with numpy reshapes: each request's blocks, in table order
    Ks, Vs = [], []
    for b in range(w.cfg.B):
        n = int(w.context_lens[b])
        nb = -(-n // 16)
        for pool, lst in ((w.k_pool, Ks), (w.v_pool, Vs)):
            blocks = pool[w.block_tables[b, :nb]]                 # [nb, H, bs, D]
            lst.append(blocks.transpose(0, 2, 1, 3).reshape(nb * 16, w.cfg.H_kv, w.cfg.D)[:n])
    ref = sdpa_reference("f32", w.q, Ks, Vs, w.scale, w.cfg.H_q, w.cfg.H_kv)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_one_token_returns_v0_exactly(oracle_lib, dtype):
    rng = np.random.default_rng(1)
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, dtype, 3, 4, 4, 64, [1, 1, 1])
    got = oracle.paged_decode_attention(dtype, q, kp, vp, bt, ctx, np.float32(0.125))
    for b in range(3):
        assert np.array_equal(got[b], f64_of(dtype, Vs[b][0]))


def set_request_rows(pool, ids, n_tokens, rows_by_token):
    """Write [n_tokens, H, D] rows into a request's blocks through the reshape route."""
    nb = len(ids)
    H, bs, D = pool.shape[1], pool.shape[2], pool.shape[3]
    seq = pool[ids].transpose(0, 2, 1, 3).reshape(nb * bs, H, D).copy()
    seq[:n_tokens] = rows_by_token
    pool[ids] = seq.reshape(nb, bs, H, D).transpose(0, 2, 1, 3)


@pytest.mark.parametrize("dtype", DTYPES)
def test_identical_v_rows_return_that_row(oracle_lib, dtype):
    rng = np.random.default_rng(2)
    lens = [23, 40]
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, dtype, 2, 2, 2, 64, lens)
    rows = to_storage(rng.standard_normal((2, 2, 64)), dtype)     # one row per (request, head)
    for b, n in enumerate(lens):
        set_request_rows(vp, bt[b, :-(-n // 16)], n, np.repeat(rows[b][None], n, axis=0))
    got = oracle.paged_decode_attention(dtype, q, kp, vp, bt, ctx, np.float32(0.125))
    for b in range(2):
        ref = f64_of(dtype, rows[b])
        assert np.max(np.abs(got[b] - ref)) <= 1e-14 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("dtype", DTYPES)
def test_zero_query_gives_mean_of_v(oracle_lib, dtype):
    rng = np.random.default_rng(3)
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, dtype, 2, 2, 2, 16, [7, 33])
    q[:] = to_storage(np.zeros(q.shape), dtype)
    got = oracle.paged_decode_attention(dtype, q, kp, vp, bt, ctx, np.float32(0.25))
    for b in range(2):
        ref = f64_of(dtype, Vs[b]).mean(axis=0)     # [H, D]
        assert np.max(np.abs(got[b] - ref)) <= 1e-13
    # scale = 0 is the same uniform average with any query
    q2 = to_storage(rng.standard_normal(q.shape), dtype)
    got0 = oracle.paged_decode_attention(dtype, q2, kp, vp, bt, ctx, np.float32(0.0))
    assert np.max(np.abs(got0 - got)) <= 1e-13


def test_dominant_logit_selects_argmax_row(oracle_lib):
    rng = np.random.default_rng(4)
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, "f32", 1, 1, 1, 64, [40])
    # make the query equal to key row 17 times a large factor
    kvals = f64_of("f32", Ks[0][:, 0, :])
    q[0, 0] = (kvals[17] * 1000.0).astype(np.float32)
    got = oracle.paged_decode_attention("f32", q, kp, vp, bt, ctx, np.float32(1.0))
    assert np.all(np.isfinite(got))
    s = kvals @ f64_of("f32", q[0, 0])
    assert int(np.argmax(s)) == 17
    assert np.max(np.abs(got[0, 0] - f64_of("f32", Vs[0][17, 0]))) <= 1e-12


def test_empty_context_gives_zero_row(oracle_lib):
    rng = np.random.default_rng(5)
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, "f16", 2, 2, 2, 8, [0, 9])
    got, lse = oracle.paged_decode_attention("f16", q, kp, vp, bt, ctx, np.float32(0.3), with_lse=True)
    assert np.array_equal(got[0], np.zeros((2, 8)))
    assert np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(got[1]))


# ---------------------------------------------------------------------------
# invariances implied by paging (blocks anywhere; blocks may be shared)
# ---------------------------------------------------------------------------

def relocate(w_k, w_v, bt, rng):
    """Move every physical block to a new random place and rewrite the tables to match."""
    n = w_k.shape[0]
    sigma = rng.permutation(n).astype(np.int32)
    k2 = np.empty_like(w_k)
    v2 = np.empty_like(w_v)
    k2[sigma] = w_k
    v2[sigma] = w_v
    bt2 = np.where(bt >= 0, sigma[np.maximum(bt, 0)], -1).astype(np.int32)
    return k2, v2, bt2


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_block_relocation_invariance(oracle_lib, name):
    cfg = get_config(name)
    w = make_workload(cfg, seed=11, append=False,
                      lengths=None if name == "c1" else np.array([1024, 300, 17, 1, 64, 999, 513, 2]))
    ref = oracle.paged_decode_attention(cfg.dtype, w.q, w.k_pool, w.v_pool, w.block_tables,
                                        w.context_lens, w.scale)
    k2, v2, bt2 = relocate(w.k_pool, w.v_pool, w.block_tables, np.random.default_rng(12))
    got = oracle.paged_decode_attention(cfg.dtype, w.q, k2, v2, bt2, w.context_lens, w.scale)
    assert np.array_equal(got, ref)


def test_batch_permutation_equivariance(oracle_lib):
    cfg = get_config("c3", B=6)
    w = make_workload(cfg, seed=5, append=False)
    ref = oracle.paged_decode_attention(cfg.dtype, w.q, w.k_pool, w.v_pool, w.block_tables,
                                        w.context_lens, w.scale)
    p = np.random.default_rng(3).permutation(cfg.B)
    got = oracle.paged_decode_attention(cfg.dtype, w.q[p].copy(), w.k_pool, w.v_pool,
                                        w.block_tables[p].copy(), w.context_lens[p].copy(), w.scale)
    assert np.array_equal(got, ref[p])


def test_shared_prefix_blocks(oracle_lib):
    """Two requests whose tables point at the same physical blocks see the same history."""
    rng = np.random.default_rng(8)
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, "bf16", 1, 4, 4, 64, [40])
    bt2 = np.repeat(bt, 3, axis=0)
    q2 = np.repeat(q, 3, axis=0)
    ctx2 = np.array([40, 40, 32], dtype=np.int32)     # third: a shorter view of the same blocks
    got = oracle.paged_decode_attention("bf16", q2, kp, vp, bt2, ctx2, np.float32(0.125))
    assert np.array_equal(got[0], got[1])
    ref_short = sdpa_reference("bf16", q, [Ks[0][:32]], [Vs[0][:32]], np.float32(0.125), 4, 4)
    assert np.max(np.abs(got[2] - ref_short[0])) <= 1e-12


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gqa_equals_mha_with_repeated_kv_heads(oracle_lib, dtype):
    cfg = get_config("c5", B=2, lengths=("fixed", (37, 70)), pool=("factor", 1.2), dtype=dtype)
    w = make_workload(cfg, seed=21)
    got = oracle.paged_decode_attention(dtype, w.q, w.k_pool, w.v_pool, w.block_tables,
                                        w.context_lens, w.scale)
    G = cfg.G
    k_rep = np.ascontiguousarray(np.repeat(w.k_pool, G, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(w.v_pool, G, axis=1))
    ref = oracle.paged_decode_attention(dtype, w.q, k_rep, v_rep, w.block_tables, w.context_lens, w.scale)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("P", [16, 64, 512])
def test_lse_merge_of_subranges_equals_whole(oracle_lib, P):
    """Attention over token ranges [iP, (i+1)P) merged by log-sum-exp equals attention over all tokens."""
    cfg = get_config("c4", B=3, lengths=("fixed", (1, 700, 1100)))
    w = make_workload(cfg, seed=4)
    full, full_lse = oracle.paged_decode_attention(cfg.dtype, w.q, w.k_pool, w.v_pool, w.block_tables,
                                                   w.context_lens, w.scale, with_lse=True)
    bs = cfg.block_size
    for b in range(cfg.B):
        n = int(w.context_lens[b])
        parts, lses = [], []
        for start in range(0, n, P):
            m = min(P, n - start)
            sub_bt = w.block_tables[b:b + 1, start // bs:start // bs + (m + bs - 1) // bs].copy()
            o, l = oracle.paged_decode_attention(cfg.dtype, w.q[b:b + 1], w.k_pool, w.v_pool, sub_bt,
                                                 np.array([m], np.int32), w.scale, with_lse=True)
            parts.append(o[0])
            lses.append(l[0])
        lses = np.stack(lses)                    # [parts, H]
        L = np.logaddexp.reduce(lses, axis=0)    # [H]
        merged = np.einsum("ph,phd->hd", np.exp(lses - L[None]), np.stack(parts))
        assert np.max(np.abs(merged - full[b])) <= 1e-12
        assert np.max(np.abs(L - full_lse[b])) <= 1e-12


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_append_writes_exactly_the_target_rows(oracle_lib, dtype):
    rng = np.random.default_rng(9)
    lens = [15, 16, 1, 33]   # the new token goes to slots 15, 0 (fresh block), 1, 1
    B, H, D = 4, 3, 16
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, dtype, B, H, H, D, [n + 1 for n in lens])
    k_new = to_storage(rng.standard_normal((B, H, D)), dtype)
    v_new = to_storage(rng.standard_normal((B, H, D)), dtype)
    # expected pools: the old ones with only row `n` of each request replaced
    k_exp, v_exp = kp.copy(), vp.copy()
    for b, n in enumerate(lens):
        ids = bt[b, :-(-(n + 1) // 16)]
        for pool, new in ((k_exp, k_new), (v_exp, v_new)):
            seq = pool[ids].transpose(0, 2, 1, 3).reshape(len(ids) * 16, H, D).copy()
            seq[n] = new[b]
            pool[ids] = seq.reshape(len(ids), 16, H, D).transpose(0, 2, 1, 3)
    oracle.kv_append(dtype, k_new, v_new, kp, vp, bt, np.array(lens, dtype=np.int32), 16)
    assert np.array_equal(kp.view(np.uint8), k_exp.view(np.uint8))
    assert np.array_equal(vp.view(np.uint8), v_exp.view(np.uint8))


def test_append_then_attend_equals_sdpa_on_history_plus_new(oracle_lib):
    w = make_workload(get_config("c1"))                    # append config: positions = ctx - 1
    out, kp, vp = oracle.run_step(w)
    Ks, Vs = [], []
    for b in range(w.cfg.B):
        n = int(w.context_lens[b])
        nb = -(-n // 16)
        hist = int(w.positions[b])
        for pool, new, lst in ((w.k_pool, w.k_new, Ks), (w.v_pool, w.v_new, Vs)):
            seq = pool[w.block_tables[b, :nb]].transpose(0, 2, 1, 3).reshape(nb * 16, 2, 64)[:hist]
            lst.append(np.concatenate([seq, new[b][None]], axis=0))
    ref = sdpa_reference("f32", w.q, Ks, Vs, w.scale, 2, 2)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_rejects_out_of_range_tables(oracle_lib):
    rng = np.random.default_rng(10)
    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, "f32", 2, 2, 2, 8, [5, 20])
    bad = bt.copy()
    bad[1, 1] = kp.shape[0]
    with pytest.raises(oracle.OracleError):
        oracle.paged_decode_attention("f32", q, kp, vp, bad, ctx, np.float32(1.0))
    with pytest.raises(oracle.OracleError):
        oracle.paged_decode_attention("f32", q, kp, vp, bt, np.array([5, 33], np.int32), np.float32(1.0))
    with pytest.raises(oracle.OracleError):
        oracle.kv_append("f32", q[:, :, :8].copy(), q[:, :, :8].copy(), kp, vp, bt,
                         np.array([5, 32], np.int32), 16)


# ---------------------------------------------------------------------------
# planted mistakes: each mutated copy of oracle.c must fail at least one pin
# ---------------------------------------------------------------------------

MUTATIONS = {
    "slot_and_head_swapped": (r"\(\(\(int64_t\)table\[t / block_size\] \* H_kv \+ g\) \* block_size \+\s*t % block_size\)",
                              "(((int64_t)table[t / block_size] * block_size + t % block_size) * H_kv + g)"),
    "wrong_block_index": (r"table\[t / block_size\]", "table[(t / block_size) / 2]"),
    "query_head_not_grouped": (r"int32_t g = h / G;", "int32_t g = h % H_kv;"),
    "softmax_sign": (r"exp\(s\[t\] - m\)", "exp(m - s[t])"),
    "scale_dropped": (r"s\[t\] = \(double\)scale \* dot;", "s[t] = dot;"),
    "f16_bias_off_by_one": (r"ex - 25\)", "ex - 24)"),
    "last_token_dropped": (r"for \(int32_t t = 0; t < n; \+\+t\) \{ s\[t\] = exp",
                           "for (int32_t t = 0; t < n - 1; ++t) { s[t] = exp"),
}


def _pin_suite(lib_path):
    """A compact run of the pins above against a given build of oracle.c; True if all pass."""
    saved = oracle._lib, oracle._LIB_PATH
    try:
        oracle._lib = None
        oracle._LIB_PATH = lib_path
        try:
            for dtype in DTYPES:
                bits = np.arange(1 << 16, dtype=np.uint16)
                if dtype != "f32":
                    mine = oracle.decode(dtype, bits)
                    ref = f64_of(dtype, bits)
                    ok = np.isnan(ref)
                    if not np.array_equal(mine[~ok], ref[~ok]):
                        return False
                for shape in SHAPES:
                    B, H_q, H_kv, D, lens = shape
                    rng = np.random.default_rng(123)
                    q, kp, vp, bt, ctx, Ks, Vs = contiguous_case(rng, dtype, B, H_q, H_kv, D, lens)
                    scale = np.float32(1.0 / math.sqrt(D))
                    got = oracle.paged_decode_attention(dtype, q, kp, vp, bt, ctx, scale)
                    ref = sdpa_reference(dtype, q, Ks, Vs, scale, H_q, H_kv)
                    if not np.max(np.abs(got - ref)) <= 1e-12:
                        return False
        except oracle.OracleError:
            return False
        return True
    finally:
        oracle._lib, oracle._LIB_PATH = saved


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_mistakes_are_caught(oracle_lib):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        # the unmutated source passes the compact suite
        base = os.path.join(tmp, "base.so")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", base,
                        os.path.join(os.path.dirname(oracle.__file__), "oracle.c"), "-lm"], check=True)
        assert _pin_suite(base)
        for name, (pat, rep) in MUTATIONS.items():
            mutated, count = re.subn(pat, rep, src)
            assert count >= 1, f"mutation {name} did not apply"
            c = os.path.join(tmp, name + ".c")
            so = os.path.join(tmp, name + ".so")
            open(c, "w").write(mutated)
            subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"], check=True)
            assert not _pin_suite(so), f"planted mistake '{name}' was not caught"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


# ---------------------------------------------------------------------------
# Appends of one step write distinct slots ("从 PagedAttention 到 Prefill-Decode
# 分离的深度解析", section 2.2, step three: each new token is given its own slot)
# ---------------------------------------------------------------------------

def _two_appends(dtype, same_slot):
    """Two requests whose tables share physical block 3: positions 5 and 5 (the same
    slot) or 5 and 6 (neighbouring slots of the shared block)."""
    H_kv, D, nb = 2, 64, 6
    rng = np.random.default_rng(5)
    k_new = to_storage(rng.standard_normal((2, H_kv, D)), dtype)
    v_new = to_storage(rng.standard_normal((2, H_kv, D)), dtype)
    bt = np.array([[3, 1], [3, 0]], np.int32)
    pos = np.array([5, 5 if same_slot else 6], np.int32)
    return k_new, v_new, bt, pos, nb, H_kv, D


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_aliased_append_is_rejected_and_writes_nothing(oracle_lib, dtype):
    k_new, v_new, bt, pos, nb, H_kv, D = _two_appends(dtype, True)
    sdt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    kp = np.zeros((nb, H_kv, 16, D), sdt)
    vp = np.zeros((nb, H_kv, 16, D), sdt)
    with pytest.raises(oracle.OracleError):
        oracle.kv_append(dtype, k_new, v_new, kp, vp, bt, pos, 16)
    assert not kp.view(np.uint8).any() and not vp.view(np.uint8).any()
    # neighbouring slots of one shared block are two distinct targets
    k_new, v_new, bt, pos, nb, H_kv, D = _two_appends(dtype, False)
    oracle.kv_append(dtype, k_new, v_new, kp, vp, bt, pos, 16)
    assert np.array_equal(kp[3, :, 5].view(np.uint8), k_new[0].view(np.uint8))
    assert np.array_equal(kp[3, :, 6].view(np.uint8), k_new[1].view(np.uint8))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_aliased_quantizing_append_is_rejected(oracle_lib, fmt):
    k_new, v_new, bt, pos, nb, H_kv, D = _two_appends("bf16", True)
    if fmt == "fp8":
        kp = np.full((nb, H_kv, 16, D), 0x7F, np.uint8)
        ks = np.full((nb, H_kv, 16), np.nan, np.float32)
        fn = oracle.kv_append_fp8
    else:
        kp = np.full((nb, H_kv, 16, D // 2), 0x77, np.uint8)
        ks = np.full((nb, H_kv, 16, D // 32), 0xFF, np.uint8)
        fn = oracle.kv_append_mxfp4
    vp, vs = kp.copy(), ks.copy()
    before = [a.copy() for a in (kp, vp, ks, vs)]
    with pytest.raises(oracle.OracleError):
        fn("bf16", k_new, v_new, kp, vp, ks, vs, bt, pos, 16)
    for a, b in zip((kp, vp, ks, vs), before):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
