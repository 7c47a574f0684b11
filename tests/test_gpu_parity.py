"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

kv_append is compared bit for bit over the whole pools; attention outputs
(float32) must satisfy max|g - r| <= atol and max |g - r| / max(|r|, atol/rtol)
<= rtol with (atol, rtol) = (1e-5, 1e-5) for f32 inputs and (2e-3, 1e-2) for
f16/bf16 inputs.  Every input is seeded and synthetic; every slot that holds no
valid token is NaN, so a stray read shows up as a NaN output.
"""
import math

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from workloads import get_config, make_workload, to_storage
from workloads.device import to_numpy_bits, to_tensor, upload

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def errors(got, ref, dtype):
    atol, rtol = TOL[dtype]
    g = np.asarray(got, dtype=np.float64)
    err = np.abs(g - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    return float(np.nanmax(err)) if err.size else 0.0, float(np.nanmax(rel)) if rel.size else 0.0


def assert_close(got, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ea, er = errors(got, ref, dtype)
    assert ea <= atol and er <= rtol, f"{what}: max_abs={ea:.3e} (<= {atol}), max_rel={er:.3e} (<= {rtol})"


_cache = {}


def prepared(name, seed=None, **over):
    """(workload, pools after the oracle's append, oracle output) for a config, cached."""
    key = (name, seed, tuple(sorted(over.items())))
    if key not in _cache:
        cfg = get_config(name, **over)
        w = make_workload(cfg, seed)
        out, kp, vp = oracle.run_step(w)
        _cache.clear()        # keep at most one large workload alive
        _cache[key] = (w, kp, vp, out)
    return _cache[key]


def run_attention(torch, w, kp, vp, partition_size, ctx=None):
    d = w.cfg.dtype
    q = to_tensor(w.q, d, "cuda")
    k = to_tensor(kp, d, "cuda")
    v = to_tensor(vp, d, "cuda")
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens if ctx is None else ctx).cuda()
    maxc = int((w.context_lens if ctx is None else ctx).max())
    out = pkv.paged_decode_attention(q, k, v, bt, cl, float(w.scale), maxc, partition_size=partition_size)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---------------------------------------------------------------------------
# kv_append: bit-exact over the whole pools
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c3"])
def test_kv_append_bit_exact(torch_dev, name):
    torch = torch_dev
    w, kp_ref, vp_ref, _ = prepared(name)
    t = upload(w)
    pkv.kv_append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"], t["block_tables"], t["positions"])
    torch.cuda.synchronize()
    d = w.cfg.dtype
    assert np.array_equal(to_numpy_bits(t["k_pool"], d).view(np.uint8), kp_ref.view(np.uint8))
    assert np.array_equal(to_numpy_bits(t["v_pool"], d).view(np.uint8), vp_ref.view(np.uint8))


def test_kv_append_gqa_and_strided_rows(torch_dev):
    """Append from a packed qkv row buffer (row stride > H_kv*D), grouped heads, bf16."""
    torch = torch_dev
    cfg = get_config("c5", B=5, lengths=("fixed", (1, 16, 17, 300, 4096)), pool=("factor", 1.5), append=True)
    w = make_workload(cfg, seed=3)
    kp_ref, vp_ref = w.k_pool.copy(), w.v_pool.copy()
    oracle.kv_append("bf16", w.k_new, w.v_new, kp_ref, vp_ref, w.block_tables, w.positions, 16)
    t = upload(w)
    H_q, H_kv, D = cfg.H_q, cfg.H_kv, cfg.D
    qkv = torch.zeros((cfg.B, H_q + 2 * H_kv, D), dtype=torch.bfloat16, device="cuda")
    qkv[:, H_q:H_q + H_kv] = t["k_new"]
    qkv[:, H_q + H_kv:] = t["v_new"]
    pkv.kv_append(qkv[:, H_q:H_q + H_kv], qkv[:, H_q + H_kv:], t["k_pool"], t["v_pool"], t["block_tables"],
                  t["positions"])
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_bits(t["k_pool"], "bf16").view(np.uint8), kp_ref.view(np.uint8))
    assert np.array_equal(to_numpy_bits(t["v_pool"], "bf16").view(np.uint8), vp_ref.view(np.uint8))


# ---------------------------------------------------------------------------
# attention parity on the five workloads, at full size, over partition sizes
# ---------------------------------------------------------------------------

CASES = [
    ("c1", 0), ("c1", 16),
    ("c2", 0), ("c2", 256), ("c2", 512),
    ("c3", 0), ("c3", 512),
    ("c4", 512), ("c4", 0), ("c4", 1024),
    ("c5", 1024), ("c5", 0), ("c5", 512),
]


@pytest.mark.parametrize("name,P", CASES)
def test_attention_parity(torch_dev, name, P):
    w, kp, vp, ref = prepared(name)
    got = run_attention(torch_dev, w, kp, vp, P)
    assert_close(got, ref, w.cfg.dtype, f"{name} P={P} [{pkv.last_launch()}]")


@pytest.mark.parametrize("name,P", [("c1", 0), ("c3", 0), ("c3", 512), ("c5", 1024)])
def test_fused_step_parity(torch_dev, name, P):
    """append_decode_attention: one launch writes the new token and attends over it."""
    torch = torch_dev
    if name == "c5":
        w, kp_ref, vp_ref, ref = prepared("c5", B=6, lengths=("uniform", 4096, 16384), append=True)
    else:
        w, kp_ref, vp_ref, ref = prepared(name)
    t = upload(w)
    out = pkv.append_decode_attention(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"], t["block_tables"],
                                      t["positions"], float(w.scale), int(w.context_lens.max()), partition_size=P)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, w.cfg.dtype, f"fused {name} P={P} [{pkv.last_launch()}]")
    d = w.cfg.dtype
    assert np.array_equal(to_numpy_bits(t["k_pool"], d).view(np.uint8), kp_ref.view(np.uint8))
    assert np.array_equal(to_numpy_bits(t["v_pool"], d).view(np.uint8), vp_ref.view(np.uint8))


# ---------------------------------------------------------------------------
# shapes, dtypes and head groupings beyond the five workloads
# ---------------------------------------------------------------------------

EDGE_LENS = (0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 200, 511, 512, 513, 1000)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("P", [0, 32, 256])
def test_shapes_and_ragged_lengths(torch_dev, dtype, D, G, P):
    H_kv = 2
    cfg = get_config("c2", B=len(EDGE_LENS), H_q=H_kv * G, H_kv=H_kv, D=D, dtype=dtype,
                     lengths=("fixed", EDGE_LENS), pool=("factor", 1.3))
    w = make_workload(cfg, seed=G * 100 + D + P)
    ref = oracle.paged_decode_attention(dtype, w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    got = run_attention(torch_dev, w, w.k_pool, w.v_pool, P)
    assert np.array_equal(got[0], np.zeros_like(got[0]))          # empty context -> zero row
    assert_close(got, ref, dtype, f"{dtype} D={D} G={G} P={P} [{pkv.last_launch()}]")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 8])
def test_fused_step_small(torch_dev, dtype, G):
    torch = torch_dev
    lens = (1, 2, 16, 17, 33, 100, 257)
    cfg = get_config("c3", B=len(lens), H_q=4 * G, H_kv=4, dtype=dtype, lengths=("fixed", lens), append=True)
    w = make_workload(cfg, seed=7 + G)
    ref, kp_ref, vp_ref = oracle.run_step(w)
    for P in (0, 32):
        t = upload(w)
        out = pkv.append_decode_attention(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"],
                                          t["block_tables"], t["positions"], float(w.scale), max(lens),
                                          partition_size=P)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, dtype, f"fused {dtype} G={G} P={P} [{pkv.last_launch()}]")
        assert np.array_equal(to_numpy_bits(t["k_pool"], dtype).view(np.uint8), kp_ref.view(np.uint8))
        assert np.array_equal(to_numpy_bits(t["v_pool"], dtype).view(np.uint8), vp_ref.view(np.uint8))


def test_query_from_packed_qkv_rows(torch_dev):
    """q given as a strided view into a packed [B, H_q + 2 H_kv, D] buffer."""
    torch = torch_dev
    cfg = get_config("c5", B=4, lengths=("fixed", (5, 70, 600, 1200)), pool=("factor", 1.2))
    w = make_workload(cfg, seed=9)
    ref = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    t = upload(w)
    qkv = torch.zeros((cfg.B, cfg.H_q + 2 * cfg.H_kv, cfg.D), dtype=torch.bfloat16, device="cuda")
    qkv[:, :cfg.H_q] = t["q"]
    out = pkv.paged_decode_attention(qkv[:, :cfg.H_q], t["k_pool"], t["v_pool"], t["block_tables"],
                                     t["context_lens"], float(w.scale), 1200, partition_size=256)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", "packed q")


# ---------------------------------------------------------------------------
# closed forms and invariances (bit-level where the kernel guarantees it)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,G", [("f32", 1), ("f16", 1), ("bf16", 1), ("f16", 8), ("bf16", 8)])
@pytest.mark.parametrize("P", [0, 16])
def test_single_token_returns_v0_exactly(torch_dev, dtype, G, P):
    cfg = get_config("c2", B=3, H_q=2 * G, H_kv=2, dtype=dtype, lengths=("fixed", (1, 1, 1)), pool=("blocks", 9))
    w = make_workload(cfg, seed=2)
    got = run_attention(torch_dev, w, w.k_pool, w.v_pool, P)
    v0 = oracle.decode(dtype, w.v_pool[w.block_tables[:, 0]][:, :, 0, :])     # [B, H_kv, D]
    assert np.array_equal(got, np.repeat(v0, G, axis=1).astype(np.float32))


@pytest.mark.parametrize("dtype,G", [("f16", 1), ("bf16", 8)])
def test_identical_v_rows_return_that_row(torch_dev, dtype, G):
    cfg = get_config("c2", B=2, H_q=2 * G, H_kv=2, dtype=dtype, lengths=("fixed", (300, 1111)), pool=("factor", 1.0))
    w = make_workload(cfg, seed=4)
    vp = w.v_pool.copy()
    rows = to_storage(np.random.default_rng(1).standard_normal((2, 2, 128)), dtype)
    for b in range(2):
        nb = -(-int(w.context_lens[b]) // 16)
        n = int(w.context_lens[b])
        seq = vp[w.block_tables[b, :nb]].transpose(0, 2, 1, 3).reshape(nb * 16, 2, 128).copy()
        seq[:n] = rows[b][None]
        vp[w.block_tables[b, :nb]] = seq.reshape(nb, 16, 2, 128).transpose(0, 2, 1, 3)
    for P in (0, 256):
        got = run_attention(torch_dev, w, w.k_pool, vp, P)
        ref = np.repeat(oracle.decode(dtype, rows), G, axis=1)
        assert_close(got, ref, dtype, f"identical rows P={P}")


def _relocate(k, v, bt, seed):
    sigma = np.random.default_rng(seed).permutation(k.shape[0]).astype(np.int32)
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[sigma] = k
    v2[sigma] = v
    return k2, v2, np.where(bt >= 0, sigma[np.maximum(bt, 0)], -1).astype(np.int32)


@pytest.mark.parametrize("name,P,over", [("c2", 0, dict(B=4)), ("c4", 512, dict(B=6)), ("c5", 1024, dict(B=3))])
def test_block_relocation_is_bit_identical(torch_dev, name, P, over):
    torch = torch_dev
    w = make_workload(get_config(name, **over), seed=5)
    a = run_attention(torch, w, w.k_pool, w.v_pool, P)
    k2, v2, bt2 = _relocate(w.k_pool, w.v_pool, w.block_tables, 6)
    w.block_tables = bt2
    b = run_attention(torch, w, k2, v2, P)
    assert np.array_equal(a, b)
    c = run_attention(torch, w, k2, v2, P)          # and a repeated run
    assert np.array_equal(b, c)


def test_batch_permutation_and_shared_blocks(torch_dev):
    torch = torch_dev
    w = make_workload(get_config("c4", B=5), seed=8)
    base = run_attention(torch, w, w.k_pool, w.v_pool, 512)
    p = np.array([3, 0, 4, 1, 2])
    w2 = make_workload(get_config("c4", B=5), seed=8)
    w2.q, w2.block_tables, w2.context_lens = w.q[p].copy(), w.block_tables[p].copy(), w.context_lens[p].copy()
    perm = run_attention(torch, w2, w.k_pool, w.v_pool, 512)
    assert np.array_equal(perm, base[p])
    # two requests pointing at the same physical blocks with the same query see the same output
    w3 = make_workload(get_config("c4", B=5), seed=8)
    w3.block_tables = w.block_tables.copy()
    w3.block_tables[1] = w.block_tables[0]
    w3.context_lens = w.context_lens.copy()
    w3.context_lens[1] = w.context_lens[0]
    w3.q = w.q.copy()
    w3.q[1] = w.q[0]
    shared = run_attention(torch, w3, w.k_pool, w.v_pool, 512)
    assert np.array_equal(shared[1], shared[0])
    assert np.array_equal(shared[0], base[0])


def test_bad_device_metadata_gives_nan_rows(torch_dev):
    """Out-of-range block ids or lengths never fault: the kernels' own checks turn them into NaN rows."""
    torch = torch_dev
    cfg = get_config("c2", B=4, H_q=4, H_kv=4, lengths=("fixed", (40, 40, 40, 40)), pool=("factor", 2.0))
    w = make_workload(cfg, seed=10)
    ref = oracle.paged_decode_attention("f16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    bt = w.block_tables.copy()
    bt[1, 1] = w.n_blocks + 5            # past the pool
    bt[2, 0] = -7                        # negative
    ctx = w.context_lens.copy()
    ctx[3] = 41                          # longer than max_context_len = 40
    for P in (0, 16):
        q = to_tensor(w.q, "f16", "cuda")
        k = to_tensor(w.k_pool, "f16", "cuda")
        v = to_tensor(w.v_pool, "f16", "cuda")
        out = pkv.paged_decode_attention(q, k, v, torch.from_numpy(bt).cuda(), torch.from_numpy(ctx).cuda(),
                                         float(w.scale), 40, partition_size=P)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert_close(got[0], ref[0], "f16", f"good row P={P}")
        assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))


# every launch-shape variant the library instantiates, forced through the plan's overrides
# (kind, waves, blocks per chunk, chunks in flight or ring slots): every grouped variant the library instantiates
GQA_VARIANTS = [(0, 4, 1, 1), (0, 4, 1, 2), (0, 2, 1, 1), (0, 2, 1, 2), (0, 4, 2, 1), (1, 2, 1, 2), (1, 2, 1, 3),
                (1, 2, 1, 4), (1, 4, 1, 2), (1, 4, 1, 3), (1, 8, 1, 2), (2, 2, 1, 1), (2, 2, 1, 2), (2, 4, 1, 1),
                (2, 2, 2, 1), (2, 4, 1, 2), (2, 8, 1, 1)]
# (waves, blocks per chunk, chunks in flight): every per-head variant the library instantiates
MHA_VARIANTS = [(4, 2, 1), (4, 2, 2), (4, 2, 3), (4, 1, 2), (4, 1, 4), (8, 2, 1), (8, 2, 2)]


def _with_env(env, fn):
    import os
    saved = {k: os.environ.get(k) for k in env}
    try:
        os.environ.update({k: str(v) for k, v in env.items()})
        return fn()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("variant", GQA_VARIANTS)
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
def test_gqa_launch_variants(torch_dev, variant, dtype, D):
    kind, nw, ch, pf = variant
    lens = (0, 1, 15, 16, 17, 100, 513, 1024, 3000, 4500)   # 4500 unsplit: two windows of block ids
    w_attn = make_workload(get_config("c5", B=len(lens), H_q=16, H_kv=2, D=D, dtype=dtype, lengths=("fixed", lens),
                                      pool=("factor", 1.2)), seed=32)
    ref_attn = oracle.paged_decode_attention(dtype, w_attn.q, w_attn.k_pool, w_attn.v_pool, w_attn.block_tables,
                                             w_attn.context_lens, w_attn.scale)
    env = {"PKV_GQA_KIND": kind, "PKV_GQA_NW": nw, "PKV_GQA_CH": ch, "PKV_GQA_PF": pf, "PKV_GQA_EVEN": 0}
    for P in (0, 512):
        got = _with_env(env, lambda: run_attention(torch_dev, w_attn, w_attn.k_pool, w_attn.v_pool, P))
        launch = pkv.last_launch()
        assert f"nw={nw} ch={ch} pf={pf}" in launch, launch
        assert ("_lds" in launch) == (kind == 1) and ("_kdma" in launch) == (kind == 2), launch
        assert_close(got, ref_attn, dtype, f"attn {variant} P={P} [{launch}]")
    # fused step (lengths >= 1 only)
    wf = make_workload(get_config("c5", B=len(lens) - 1, H_q=16, H_kv=2, D=D, dtype=dtype,
                                  lengths=("fixed", lens[1:]), pool=("factor", 1.2), append=True), seed=33)
    ref, kp_ref, vp_ref = oracle.run_step(wf)
    for P in (0, 512):
        t = upload(wf)
        out = _with_env(env, lambda: pkv.append_decode_attention(
            t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"], t["block_tables"], t["positions"],
            float(wf.scale), max(lens), partition_size=P))
        torch_dev.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, dtype, f"fused {variant} P={P} [{pkv.last_launch()}]")
        assert np.array_equal(to_numpy_bits(t["k_pool"], dtype).view(np.uint8), kp_ref.view(np.uint8))
        assert np.array_equal(to_numpy_bits(t["v_pool"], dtype).view(np.uint8), vp_ref.view(np.uint8))


@pytest.mark.parametrize("variant", MHA_VARIANTS)
@pytest.mark.parametrize("dtype,D", [("f16", 128), ("bf16", 64), ("f32", 128)])
def test_mha_launch_variants(torch_dev, variant, dtype, D):
    nw, ch, pf = variant
    lens = (0, 1, 15, 16, 17, 100, 513, 1024, 3000, 4500)   # 4500 unsplit: two windows of block ids
    cfg = get_config("c2", B=len(lens), H_q=4, H_kv=4, D=D, dtype=dtype, lengths=("fixed", lens),
                     pool=("factor", 1.2))
    w = make_workload(cfg, seed=41)
    ref = oracle.paged_decode_attention(dtype, w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    env = {"PKV_MHA_NW": nw, "PKV_MHA_CH": ch, "PKV_MHA_PF": pf}
    if dtype == "f32" and D == 128:      # the plan caps f32 D128 at one 2-block chunk in flight
        ch, pf = 2, 1
    for P in (0, 512):
        got = _with_env(env, lambda: run_attention(torch_dev, w, w.k_pool, w.v_pool, P))
        launch = pkv.last_launch()
        assert f"nw={nw} ch={ch} pf={pf}" in launch, launch
        assert_close(got, ref, dtype, f"mha {variant} P={P} [{launch}]")


@pytest.mark.parametrize("name,P,env", [
    ("c4", 256, {}), ("c5", 1024, {"PKV_GQA_EVEN": 0}), ("c5f8", 1024, {}), ("c5f4", 1024, {}),
    ("c3f8", 512, {}), ("c3f4", 512, {}), ("c5", 512, {"PKV_GQA_EVEN": 0, "PKV_GQA_KIND": 1}),
    ("c5", 512, {"PKV_GQA_EVEN": 0, "PKV_GQA_KIND": 0})])
def test_partition_order_is_bit_identical(torch_dev, name, P, env):
    """Dealing partitions last-first (the default) or first-first changes only the dispatch
    order: every partition is the same work and the merge adds them in index order, so the
    outputs and pools agree bit for bit, and match the oracle."""
    import os
    torch = torch_dev
    over = dict(B=6, lengths=("fixed", (1, 700, 5000, 33, 4096, 2047)), append=True)
    w = make_workload(get_config(name, **over), seed=61)
    ref = oracle.run_step(w)[0]
    outs = []
    for rev in (1, 0):
        def step():
            d = upload(w)
            kw = dict(partition_size=P)
            if w.cfg.kv_dtype == "fp8":
                o = pkv.append_decode_attention_fp8(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                                    d["k_scale"], d["v_scale"], d["block_tables"], d["positions"],
                                                    float(w.scale), int(w.context_lens.max()), **kw)
            elif w.cfg.kv_dtype == "mxfp4":
                o = pkv.append_decode_attention_mxfp4(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                                      d["k_scale"], d["v_scale"], d["block_tables"], d["positions"],
                                                      float(w.scale), int(w.context_lens.max()), **kw)
            else:
                o = pkv.append_decode_attention(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                                d["block_tables"], d["positions"], float(w.scale),
                                                int(w.context_lens.max()), **kw)
            torch.cuda.synchronize()
            pools = ("k_pool", "v_pool") + (("k_scale", "v_scale") if w.cfg.kv_dtype else ())
            return o.cpu().numpy(), {k: d[k].cpu() for k in pools}, pkv.last_launch()
        outs.append(_with_env({**env, "PKV_PART_REV": rev}, step))
    (o1, p1, l1), (o0, p0, l0) = outs
    assert l1 == l0 and "n_parts=1 " not in l1, l1
    assert np.array_equal(o1.view(np.uint32), o0.view(np.uint32)), l1
    for k in p1:
        assert torch.equal(p1[k].view(torch.uint8), p0[k].view(torch.uint8)), k
    assert_close(o1, ref, w.cfg.dtype, f"{name} P={P} [{l1}]")
