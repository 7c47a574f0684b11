"""GPU parity of the MXFP4 (OCP E2M1 codes, E8M0 block scales) K/V cache through the C ABI.

The quantizing append is compared bit for bit (code and scale bytes, whole
pools); attention outputs must satisfy the same (atol, rtol) as the f16/bf16
path ((1e-5, 1e-5) for f32 q): the kernel decodes codes exactly, so only the
float32 accumulation order separates it from the oracle.  Unwritten slots hold
code 7 (6.0) under scale byte 255 (NaN in E8M0), so a stray read shows up as a
non-finite output."""
import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_decode_loop import bits_equal
from workloads import get_config, make_workload, to_storage
from workloads.device import to_tensor, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def small_partitions(monkeypatch):
    """The grouped low-precision kernels split at no less than 2048 tokens by default; these
    tests exercise the caller's own small partitions (the floor has its own tests)."""
    monkeypatch.setenv("PKV_LP_MIN_PART", "0")

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
EDGE_LENS = (1, 2, 15, 16, 17, 31, 33, 64, 255, 257, 700)
# (kernel kind, waves, blocks per chunk or in flight): kind 0 = per-head vector-unit kernel
# (blocks per chunk), kind 1 = grouped MFMA kernel over an LDS ring (f16/bf16 q, G <= 16;
# chunks in flight per wave)
# kind 0: (nw, ch); kind 1: (nw, pf[, KV heads per workgroup])
MX4_VARIANTS = ["0,4,2", "0,8,2", "1,4,1", "1,4,2", "1,4,3", "1,2,2", "1,2,4", "1,4,1,2", "1,4,2,2", "1,4,1,4",
                "1,4,2,4", "1,8,1,4", "1,8,2,4", "1,8,1,8", "1,8,2,8", "1,8,3,8"]


def mx4_variant_env(variant, H_kv):
    """(environment, launch-string tag) of a variant.  A kind-1 variant whose heads per workgroup
    do not divide H_kv runs with one head per workgroup, and if that shape is not built, as the
    default (4 waves, 1 chunk in flight)."""
    kind, nw, x, *hg = variant.split(",")
    if kind == "0":
        return {"PKV_MX4_KIND": kind, "PKV_MX4_NW": nw, "PKV_MX4_CH": x}, f"nw={nw} ch={x} "
    hg = int(hg[0]) if hg else 1
    env = {"PKV_MX4_KIND": kind, "PKV_MX4_NW": nw, "PKV_MX4_PF": x, "PKV_MX4_HG": str(hg)}
    if H_kv % hg:
        hg = 1
        if f"1,{nw},{x}" not in MX4_VARIANTS:
            nw, x = "4", "1"
    return env, f"nw={nw} ch=1 pf={x} hg={hg} "


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
    return get_config("c3f4", dtype=dtype, D=D, H_q=H_q, H_kv=H_kv, B=len(lens), lengths=("fixed", tuple(lens)),
                      pool=("factor", 1.3), append=append, partition_size=P)


def run(torch, w, P, append):
    d = upload(w, "cuda")
    if append:
        out = pkv.append_decode_attention_mxfp4(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                                d["k_scale"], d["v_scale"], d["block_tables"], d["positions"],
                                                float(w.scale), w.max_context_len, partition_size=P)
    else:
        out = pkv.paged_decode_attention_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                                               d["block_tables"], d["context_lens"], float(w.scale),
                                               w.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    return out.cpu().numpy(), d


def pools_equal(d, pk, pv):
    return (bits_equal(d["k_pool"].cpu().numpy(), pk[0]) and bits_equal(d["k_scale"].cpu().numpy(), pk[1])
            and bits_equal(d["v_pool"].cpu().numpy(), pv[0]) and bits_equal(d["v_scale"].cpu().numpy(), pv[1]))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_kv_append_mxfp4_bit_exact(torch_dev, dtype, D):
    t = torch_dev
    cfg = cfg_for(dtype, D, 8, 4, [5, 16, 17, 40, 1, 33])
    w = make_workload(cfg, 21)
    ref = [w.k_pool.copy(), w.v_pool.copy(), w.k_scale.copy(), w.v_scale.copy()]
    oracle.kv_append_mxfp4(dtype, w.k_new, w.v_new, *ref, w.block_tables, w.positions, 16)
    d = upload(w, "cuda")
    pkv.kv_append_mxfp4(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                        d["block_tables"], d["positions"])
    t.cuda.synchronize()
    for name, r in zip(("k_pool", "v_pool", "k_scale", "v_scale"), ref):
        assert bits_equal(d[name].cpu().numpy(), r), name


def test_kv_append_mxfp4_rounding_cases(torch_dev):
    """Rows built to land on every E2M1 midpoint (ties to the even code), on the
    saturation above 6, on an all-zero block, on subnormal and huge maxima and
    on negative zero, compared bit for bit (f32 source, so no rounding on load)."""
    t = torch_dev
    H_kv, D, nb = 4, 64, 8
    rows = np.zeros((4, H_kv, D), np.float32)
    # block with amax 4 (E = 0): every midpoint of the grid, both signs, and values that saturate
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows[0, 0, :7] = mids
    rows[0, 0, 7:14] = [-x for x in mids]
    rows[0, 0, 14:18] = [4.0, 0.2499, 0.7501, -0.0]
    rows[0, 0, 32:36] = [7.9, 6.5, 5.5, -7.0]                        # amax 7.9: E = 0, 6.5 and 7.9 saturate
    rows[0, 1, :32] = np.linspace(-3, 3, 32, dtype=np.float32)       # E = -1
    rows[0, 1, 32:] = 0.0                                            # all-zero block: scale byte 0
    rows[0, 2, :4] = [2.0 ** -140, -(2.0 ** -145), 2.0 ** -149, 0.0]  # subnormal maximum: E = -127
    rows[0, 2, 32:35] = [3.0e38, -1.0e38, 2.0e37]                    # E = 125
    rows[0, 3, :32] = 2.0 ** -126 * np.arange(1, 33, dtype=np.float32)  # smallest normal exponents: clamp at -127
    rows[1] = np.linspace(-7, 7, H_kv * D, dtype=np.float32).reshape(H_kv, D)
    rows[2] = (np.arange(H_kv * D, dtype=np.float32).reshape(H_kv, D) % 13 - 6) * 0.125
    # rows[3] stays zero
    bt = np.arange(nb, dtype=np.int32).reshape(4, 2)
    pos = np.array([0, 3, 17, 9], np.int32)
    kp = np.full((nb, H_kv, 16, D // 2), 0x77, np.uint8)
    ks = np.full((nb, H_kv, 16, D // 32), 0xFF, np.uint8)
    ref = [kp.copy(), kp.copy(), ks.copy(), ks.copy()]
    oracle.kv_append_mxfp4("f32", rows, -rows, *ref, bt, pos, 16)
    dev = [t.from_numpy(a.copy()).cuda() for a in (kp, kp, ks, ks)]
    pkv.kv_append_mxfp4(t.from_numpy(rows).cuda(), t.from_numpy(-rows).cuda(), *dev, t.from_numpy(bt).cuda(),
                        t.from_numpy(pos).cuda())
    t.cuda.synchronize()
    for g, r in zip(dev, ref):
        assert bits_equal(g.cpu().numpy(), r)


@pytest.mark.parametrize("qdt,D", [("f32", 64), ("bf16", 64), ("f16", 128)])
def test_mxfp4_decode_every_code_and_extreme_scales(torch_dev, monkeypatch, qdt, D):
    """A one-token context returns its dequantized V row bit for bit: rows
    covering all 16 codes under scale bytes 0 (2^-127), 1, 127, 200 and 252 (254
    for the vector-unit kernel, whose products overflow to inf as f32 does; the
    MFMA kernel's p = hi + lo form turns an infinite V element into NaN, and the
    quantizing append never writes a scale above 252).  f32 q takes the per-head
    kernel, f16/bf16 q the grouped MFMA kernel."""
    t = torch_dev
    monkeypatch.setenv("PKV_MX4_KIND", "0" if qdt == "f32" else "1")
    H_kv = 2
    nb = 5
    kp = np.full((nb, H_kv, 16, D // 2), 0x77, np.uint8)
    ks = np.full((nb, H_kv, 16, D // 32), 0xFF, np.uint8)
    vp, vs = kp.copy(), ks.copy()
    sc_bytes = [0, 1, 127, 200, 254 if qdt == "f32" else 252]
    for b in range(nb):
        for g in range(H_kv):
            kp[b, g, 0] = 0                                          # all-zero K: every score equal
            ks[b, g, 0] = 127
            codes = np.arange(D // 2, dtype=np.uint8)
            vp[b, g, 0] = ((codes % 16) | (((codes + 7 * g) % 16) << 4)).astype(np.uint8)
            vs[b, g, 0] = [sc_bytes[(b + k * (2 + g)) % len(sc_bytes)] for k in range(D // 32)]
    q = to_storage(np.ones((nb, H_kv, D), np.float32), qdt)
    bt = np.arange(nb, dtype=np.int32).reshape(nb, 1)
    ctx = np.ones(nb, np.int32)
    dev = {k: t.from_numpy(v).cuda() for k, v in (("kp", kp), ("vp", vp), ("ks", ks), ("vs", vs), ("bt", bt),
                                                    ("ctx", ctx))}
    dev["q"] = to_tensor(q, qdt, "cuda")
    out = pkv.paged_decode_attention_mxfp4(dev["q"], dev["kp"], dev["vp"], dev["ks"], dev["vs"], dev["bt"],
                                           dev["ctx"], 0.125, 16)
    t.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.mxfp4_dequantize(vp[:, :, 0], vs[:, :, 0])
    assert pkv.last_launch().startswith("mxfp4 " if qdt == "f32" else "mxfp4_mfma "), pkv.last_launch()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("qdt,D", [("f16", 128), ("bf16", 128), ("f16", 64), ("bf16", 64)])
def test_mxfp4_per_head_scores_over_k_scales(torch_dev, monkeypatch, qdt, D):
    """The per-head kernel's packed q . k (f16 codes at unit scale times the block
    scale; bf16 codes with the scale folded in) against the oracle, with K scale
    bytes drawn from 0 (2^-127), 1, 40, 90, 120, 127 and 132 instead of the
    workload's narrow range: every exponent from the subnormal end to 2^5."""
    monkeypatch.setenv("PKV_MX4_KIND", "0")
    cfg = cfg_for(qdt, D, 4, 4, (1, 17, 200, 700), append=False)
    w = make_workload(cfg, 71)
    rng = np.random.default_rng(72)
    written = w.k_scale != 0xFF
    w.k_scale[written] = rng.choice(np.array([0, 1, 40, 90, 120, 127, 132], np.uint8), size=int(written.sum()))
    ref, _, _ = oracle.run_step(w)
    got, _ = run(torch_dev, w, 0, False)
    assert pkv.last_launch().startswith("mxfp4 "), pkv.last_launch()
    assert_close(got, ref, qdt, f"{qdt} D{D}")


@pytest.mark.parametrize("dtype,D,H_q,H_kv", [("f16", 128, 8, 8), ("bf16", 128, 16, 2), ("bf16", 64, 8, 1),
                                              ("f32", 64, 4, 4), ("f16", 64, 4, 2), ("f32", 128, 2, 1),
                                              ("f16", 128, 16, 1), ("f16", 64, 12, 4)])
@pytest.mark.parametrize("P", [0, 32, 256])
@pytest.mark.parametrize("append", [False, True])
def test_mxfp4_attention_parity(torch_dev, dtype, D, H_q, H_kv, P, append):
    cfg = cfg_for(dtype, D, H_q, H_kv, EDGE_LENS, P=P, append=append)
    w = make_workload(cfg, 31)
    ref, pk, pv = oracle.run_step(w)
    got, d = run(torch_dev, w, P, append)
    assert_close(got, ref, dtype, f"{dtype} D{D} G{H_q // H_kv} P{P} append={append}")
    if append:
        assert pools_equal(d, pk, pv)
    # f16/bf16 q with grouped heads takes the MFMA kernel, f32 q and one head per KV head the per-head one
    mfma = dtype != "f32" and H_q // H_kv > 1
    assert pkv.last_launch().startswith("mxfp4_mfma " if mfma else "mxfp4 "), pkv.last_launch()


@pytest.mark.parametrize("variant", MX4_VARIANTS)
def test_mxfp4_every_launch_variant(torch_dev, monkeypatch, variant):
    kind = variant.split(",")[0]
    name = "mxfp4_mfma " if kind == "1" else "mxfp4 "
    # 4500 tokens unsplit: more than one 256-block window of ids per workgroup; 8 KV heads:
    # every heads-per-workgroup count divides them; G = 16 on 4 KV heads: head groups on the
    # one-block-per-product path
    cases = [("f16", 128, 0, 4, 4, True), ("bf16", 64, 64, 8, 2, True), ("bf16", 128, 256, 16, 1, False),
             ("f16", 64, 0, 6, 2, False), ("bf16", 128, 512, 32, 8, True), ("f16", 64, 0, 64, 8, False),
             ("bf16", 128, 256, 64, 4, True)]
    if kind == "0":
        cases.append(("f32", 128, 256, 4, 2, False))
    for dtype, D, P, H_q, H_kv, append in cases:
        env, tag = mx4_variant_env(variant, H_kv)
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        cfg = cfg_for(dtype, D, H_q, H_kv, (1, 17, 200, 1000, 2049, 4500), P=P, append=append)
        w = make_workload(cfg, 41)
        ref, pk, pv = oracle.run_step(w)
        got, d = run(torch_dev, w, P, append)
        launch = pkv.last_launch()
        assert launch.startswith(name) and tag in launch, launch
        assert_close(got, ref, dtype, f"variant {variant} {dtype} D{D} P{P}")
        if append:
            assert pools_equal(d, pk, pv)


def test_mxfp4_bad_metadata_gives_nan_rows(torch_dev):
    t = torch_dev
    cfg = cfg_for("f16", 128, 4, 4, (40, 40, 40), append=False)
    w = make_workload(cfg, 61)
    w.block_tables[1, 1] = w.n_blocks + 5          # out of range: request 1 gets NaN rows
    ctx = w.context_lens.copy()
    ctx[2] = 10 ** 6                                # longer than max_context_len: NaN rows
    d = upload(w, "cuda")
    out = pkv.paged_decode_attention_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                                           d["block_tables"], t.from_numpy(ctx).cuda(), float(w.scale), 40)
    t.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_grouped_partition_floor(torch_dev, monkeypatch, dtype):
    """Default plan: the grouped MXFP4 kernel splits at no less than 2048 tokens (a multiple of
    the caller's partition), unsplit when that covers every context; both it and the caller's
    own partitions (PKV_LP_MIN_PART=0) match the oracle, fused step pools bit-exact."""
    torch = torch_dev
    lens = (1, 17, 2047, 2048, 2049, 4500, 700)
    for P, want in ((32, 2048), (1024, 2048), (3008, 3008)):
        cfg = cfg_for(dtype, 128, 16, 2, lens, P=P, append=True)
        w = make_workload(cfg, seed=81 + P)
        ref, kp, vp = oracle.run_step(w)
        for floor in (None, "0"):
            if floor is None:
                monkeypatch.delenv("PKV_LP_MIN_PART", raising=False)
            else:
                monkeypatch.setenv("PKV_LP_MIN_PART", floor)
            got, d = run(torch, w, P, True)
            launch = pkv.last_launch()
            part = want if floor is None else P
            assert launch.startswith("mxfp4_mfma ") and f"part_tokens={part} " in launch, launch
            assert_close(got, ref, dtype, f"P={P} floor={floor} [{launch}]")
            assert pools_equal(d, kp, vp), launch
