"""GPU parity of the FP8 (OCP E4M3) K/V cache through the C ABI against the oracle.

The quantizing append is compared bit for bit (codes and scales, whole pools);
attention outputs must satisfy the same (atol, rtol) as the f16/bf16 path
((1e-5, 1e-5) for f32 q).  Unwritten slots hold the NaN code with a NaN scale,
so a stray read shows up as a NaN output."""
import math

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_decode_loop import bits_equal
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits, to_tensor, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def small_partitions(monkeypatch):
    """The grouped low-precision kernels split at no less than 2048 tokens by default; these
    tests exercise the caller's own small partitions (the floor has its own tests)."""
    monkeypatch.setenv("PKV_LP_MIN_PART", "0")

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
EDGE_LENS = (1, 2, 15, 16, 17, 31, 33, 64, 255, 257, 700)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def assert_close(got, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    assert err.max() <= atol and rel.max() <= rtol, f"{what}: max_abs={err.max():.3e} max_rel={rel.max():.3e}"


def cfg_for(dtype, D, H_q, H_kv, lens, P=0, append=True):
    return get_config("c3f8", dtype=dtype, D=D, H_q=H_q, H_kv=H_kv, B=len(lens), lengths=("fixed", tuple(lens)),
                      pool=("factor", 1.3), append=append, partition_size=P)


def run(torch, w, P, append):
    d = upload(w, "cuda")
    if append:
        out = pkv.append_decode_attention_fp8(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["k_scale"],
                                              d["v_scale"], d["block_tables"], d["positions"], float(w.scale),
                                              w.max_context_len, partition_size=P)
    else:
        out = pkv.paged_decode_attention_fp8(d["q"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                                             d["block_tables"], d["context_lens"], float(w.scale),
                                             w.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    return out.cpu().numpy(), d


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_kv_append_fp8_bit_exact(torch_dev, dtype, D):
    t = torch_dev
    cfg = cfg_for(dtype, D, 8, 4, [5, 16, 17, 40, 1, 33])
    w = make_workload(cfg, 21)
    ref_k, ref_v, ref_ks, ref_vs = w.k_pool.copy(), w.v_pool.copy(), w.k_scale.copy(), w.v_scale.copy()
    oracle.kv_append_fp8(dtype, w.k_new, w.v_new, ref_k, ref_v, ref_ks, ref_vs, w.block_tables, w.positions, 16)
    d = upload(w, "cuda")
    pkv.kv_append_fp8(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                      d["block_tables"], d["positions"])
    t.cuda.synchronize()
    assert bits_equal(d["k_pool"].cpu().numpy(), ref_k) and bits_equal(d["v_pool"].cpu().numpy(), ref_v)
    assert bits_equal(d["k_scale"].cpu().numpy(), ref_ks) and bits_equal(d["v_scale"].cpu().numpy(), ref_vs)


def test_kv_append_fp8_rounding_cases(torch_dev):
    """Rows built to hit ties, the clamp at 448, subnormal codes and an all-zero row, bit for bit."""
    t = torch_dev
    H_kv, D, nb = 4, 64, 8
    rows = np.zeros((4, H_kv, D), np.float32)
    rows[0, 0, :5] = [300, 1.0625, 1.1875, 17, 500]                 # ties to even, clamp
    rows[0, 1, :4] = [1.0, -0.5, 0.0, 3.0]
    rows[0, 2, :3] = [256.0, 2.0 ** -9 * 3, -2.0 ** -8 * 1.5]      # subnormal codes and a tie among them
    rows[1] = np.linspace(-7, 7, H_kv * D, dtype=np.float32).reshape(H_kv, D)
    rows[2, :, 0] = 1e-30                                            # maximum below the f32 normal range
    # rows[3] stays zero
    bt = np.arange(nb, dtype=np.int32).reshape(4, 2)
    pos = np.array([0, 3, 17, 9], np.int32)
    kp = np.full((nb, H_kv, 16, D), 0x7F, np.uint8)
    ks = np.full((nb, H_kv, 16), np.nan, np.float32)
    ref = [kp.copy(), kp.copy(), ks.copy(), ks.copy()]
    oracle.kv_append_fp8("f32", rows, -rows, *ref, bt, pos, 16)
    dev = [t.from_numpy(a.copy()).cuda() for a in (kp, kp, ks, ks)]
    pkv.kv_append_fp8(t.from_numpy(rows).cuda(), t.from_numpy(-rows).cuda(), *dev, t.from_numpy(bt).cuda(),
                      t.from_numpy(pos).cuda())
    t.cuda.synchronize()
    for g, r in zip(dev, ref):
        assert bits_equal(g.cpu().numpy(), r)


@pytest.mark.parametrize("dtype,D,H_q,H_kv", [("bf16", 128, 8, 8), ("f16", 128, 16, 2), ("bf16", 64, 8, 1),
                                              ("f32", 64, 4, 4), ("f16", 64, 4, 2), ("f32", 128, 2, 1)])
@pytest.mark.parametrize("P", [0, 32, 256])
@pytest.mark.parametrize("append", [False, True])
def test_fp8_attention_parity(torch_dev, dtype, D, H_q, H_kv, P, append):
    cfg = cfg_for(dtype, D, H_q, H_kv, EDGE_LENS, P=P, append=append)
    w = make_workload(cfg, 31)
    ref, (kp, ks), (vp, vs) = oracle.run_step(w)
    got, d = run(torch_dev, w, P, append)
    assert_close(got, ref, dtype, f"{dtype} D{D} G{H_q // H_kv} P{P} append={append}")
    if append:
        assert bits_equal(d["k_pool"].cpu().numpy(), kp) and bits_equal(d["v_pool"].cpu().numpy(), vp)
        assert bits_equal(d["k_scale"].cpu().numpy(), ks) and bits_equal(d["v_scale"].cpu().numpy(), vs)


@pytest.mark.parametrize("variant", ["4,2,1", "4,2,2", "8,2,2", "4,4,1"])
def test_fp8_every_launch_variant(torch_dev, monkeypatch, variant):
    nw, ch, pf = variant.split(",")
    monkeypatch.setenv("PKV_FP8_NW", nw)
    monkeypatch.setenv("PKV_FP8_CH", ch)
    monkeypatch.setenv("PKV_FP8_PF", pf)
    for dtype, D, P, G in (("bf16", 128, 0, 1), ("f16", 64, 64, 1), ("f32", 128, 0, 2)):
        cfg = cfg_for(dtype, D, 4, 4 // G, (1, 17, 200, 1000, 2049), P=P)
        w = make_workload(cfg, 41)
        ref, _, _ = oracle.run_step(w)
        got, _ = run(torch_dev, w, P, True)
        launch = pkv.last_launch()
        assert launch.startswith("fp8 ") and f"nw={nw} ch={ch} pf={pf}" in launch, launch
        assert_close(got, ref, dtype, f"variant {variant} {dtype} D{D} P{P}")


# (waves, blocks per chunk, chunks in flight, waves per SIMD, K staged through LDS): every
# variant the library instantiates for the grouped FP8 kernel
GQA8_VARIANTS = ["2,1,1,2,0", "2,1,2,2,0", "4,1,1,2,0", "2,2,1,2,0", "4,2,1,2,0", "2,1,1,3,0", "4,1,1,3,0",
                 "2,1,1,2,1", "2,1,2,2,1", "2,1,3,2,1", "4,1,1,2,1", "4,1,2,2,1", "2,2,1,2,1", "2,1,1,3,1",
                 "4,1,2,3,1"]


@pytest.mark.parametrize("variant", GQA8_VARIANTS)
def test_fp8_grouped_every_launch_variant(torch_dev, monkeypatch, variant):
    nw, ch, pf, wpe, kd = variant.split(",")
    monkeypatch.setenv("PKV_GQA8_NW", nw)
    monkeypatch.setenv("PKV_GQA8_CH", ch)
    monkeypatch.setenv("PKV_GQA8_PF", pf)
    monkeypatch.setenv("PKV_GQA8_WPE", wpe)
    monkeypatch.setenv("PKV_GQA8_KDMA", kd)
    tag = f"nw={nw} ch={ch} pf={pf} wpe={wpe}" + (" kdma" if kd == "1" else "")
    # 4500 tokens unsplit: more than one 256-block window of ids per workgroup
    for dtype, D, P, H_q, H_kv, append in (("bf16", 128, 0, 8, 1, True), ("f16", 64, 64, 16, 2, True),
                                           ("bf16", 128, 256, 12, 4, False)):
        cfg = cfg_for(dtype, D, H_q, H_kv, (1, 17, 200, 1000, 2049, 4500), P=P, append=append)
        w = make_workload(cfg, 43)
        ref, pk, pv = oracle.run_step(w)
        got, d = run(torch_dev, w, P, append)
        launch = pkv.last_launch()
        assert launch.startswith("gqa_mfma_fp8") and tag + " " in launch, launch
        assert_close(got, ref, dtype, f"grouped variant {variant} {dtype} D{D} P{P}")
        if append:
            assert bits_equal(d["k_pool"].cpu().numpy(), pk[0]) and bits_equal(d["k_scale"].cpu().numpy(), pk[1])
            assert bits_equal(d["v_pool"].cpu().numpy(), pv[0]) and bits_equal(d["v_scale"].cpu().numpy(), pv[1])


def test_fp8_single_token_is_exact(torch_dev):
    """A one-token context returns that token's dequantized V row bit for bit."""
    cfg = cfg_for("bf16", 128, 4, 2, (1, 1, 1))
    w = make_workload(cfg, 51)
    ref, _, (vp, vs) = oracle.run_step(w)
    got, _ = run(torch_dev, w, 0, True)
    G = 2
    for b in range(3):
        blk = w.block_tables[b, 0]
        for h in range(4):
            row = oracle.e4m3_decode(vp[blk, h // G, 0]) * float(vs[blk, h // G, 0])
            assert np.array_equal(got[b, h].astype(np.float64), row)


def test_fp8_bad_metadata_gives_nan_rows(torch_dev):
    t = torch_dev
    cfg = cfg_for("f16", 128, 4, 4, (40, 40, 40), append=False)
    w = make_workload(cfg, 61)
    w.block_tables[1, 1] = w.n_blocks + 5          # out of range: request 1 gets NaN rows
    ctx = w.context_lens.copy()
    ctx[2] = 10 ** 6                                # longer than max_context_len: NaN rows
    d = upload(w, "cuda")
    out = pkv.paged_decode_attention_fp8(d["q"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                                         d["block_tables"], t.from_numpy(ctx).cuda(), float(w.scale), 40)
    t.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
