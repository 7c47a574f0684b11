"""GPU parity of the grouped MXFP4 kernel's even split through the C ABI.

The batch's blocks, requests end to end, are cut into equal runs; a workgroup streams one
run for a group of nw KV heads, one head per wave, and writes each piece it meets (a whole
request as the output, any other for the merge kernel).  PKV_MX4_EVEN=2 takes the split
whenever it fits.  Outputs are checked against the fp64 oracle to the f16/bf16 bound
(2e-3, 1e-2); the fused step's pools (codes and scale bytes) bit for bit.
"""
import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_mxfp4 import assert_close, cfg_for, pools_equal, run, torch_dev  # noqa: F401 (fixture)
from workloads import make_workload
from workloads.device import upload

pytestmark = pytest.mark.gpu

LENS = (1, 17, 200, 1000, 2049, 4500, 16, 33)


@pytest.fixture(autouse=True)
def even_split(monkeypatch):
    monkeypatch.setenv("PKV_MX4_EVEN", "2")
    monkeypatch.setenv("PKV_MX4_KIND", "1")      # the grouped kernel also for one query head per KV head
    monkeypatch.setenv("PKV_LP_MIN_PART", "0")
    for k in ("PKV_MX4_EVEN_NW", "PKV_MX4_EVEN_PF"):
        monkeypatch.delenv(k, raising=False)


def expect_even(tag=""):
    launch = pkv.last_launch()
    assert launch.startswith("mxfp4_mfma_even ") and tag in launch, launch
    return launch


def attention(torch, w, P, bt=None, ctx=None, maxc=None, ws=None):
    """paged_decode_attention_mxfp4 over the workload's pools, with optional table / length overrides."""
    d = upload(w, "cuda")
    bt_t = d["block_tables"] if bt is None else torch.from_numpy(np.ascontiguousarray(bt)).cuda()
    ctx_t = d["context_lens"] if ctx is None else torch.from_numpy(np.ascontiguousarray(ctx)).cuda()
    out = pkv.paged_decode_attention_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"], bt_t, ctx_t,
                                           float(w.scale), w.max_context_len if maxc is None else maxc,
                                           partition_size=P, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("append", [True, False])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_even_split_matches_oracle(torch_dev, dtype, D, G, append):
    """Four KV heads (one 4-wave workgroup per run), two blocks per output product for
    G <= 8, one above; runs cut requests at both ends and hold several whole ones."""
    cfg = cfg_for(dtype, D, 4 * G, 4, LENS, P=256, append=append)
    w = make_workload(cfg, 900 + G)
    ref, pk, pv = oracle.run_step(w)
    got, d = run(torch_dev, w, 256, append)
    launch = expect_even("nw=4 ch=1 pf=1 hg=4 ")
    assert_close(got, ref, dtype, f"{dtype} D{D} G{G} [{launch}]")
    if append:
        assert pools_equal(d, pk, pv), launch


@pytest.mark.parametrize("nw,pf", [(8, 1), (4, 1), (4, 2), (2, 2)])
def test_even_split_every_variant(torch_dev, monkeypatch, nw, pf):
    """Every built (waves, chunks in flight) shape on eight KV heads, fused step."""
    monkeypatch.setenv("PKV_MX4_EVEN_NW", str(nw))
    monkeypatch.setenv("PKV_MX4_EVEN_PF", str(pf))
    for dtype, G in (("bf16", 8), ("f16", 3)):
        cfg = cfg_for(dtype, 128, 8 * G, 8, LENS, P=512, append=True)
        w = make_workload(cfg, 910 + nw * 10 + pf)
        ref, pk, pv = oracle.run_step(w)
        got, d = run(torch_dev, w, 512, True)
        launch = expect_even(f"nw={nw} ch=1 pf={pf} hg={nw} ")
        assert_close(got, ref, dtype, f"nw={nw} pf={pf} {dtype} G{G} [{launch}]")
        assert pools_equal(d, pk, pv), launch


def test_even_split_default_shape_follows_the_kv_heads(torch_dev):
    """Without an override the workgroup takes 4 KV heads when they divide H_kv, else 2 (with
    two chunks in flight); one KV head has no even split."""
    for H_kv, tag in ((8, "nw=4 ch=1 pf=1 "), (4, "nw=4 ch=1 pf=1 "), (6, "nw=2 ch=1 pf=2 "), (1, None)):
        cfg = cfg_for("bf16", 64, 2 * H_kv, H_kv, (300, 70, 1200), P=128, append=True)
        w = make_workload(cfg, 920 + H_kv)
        ref, pk, pv = oracle.run_step(w)
        got, d = run(torch_dev, w, 128, True)
        launch = pkv.last_launch()
        if tag is None:
            assert launch.startswith("mxfp4_mfma "), launch
        else:
            assert launch.startswith("mxfp4_mfma_even ") and tag in launch, launch
        assert_close(got, ref, "bf16", f"H_kv={H_kv} [{launch}]")
        assert pools_equal(d, pk, pv), launch


def test_even_split_single_long_request(torch_dev):
    """One request: every run lies inside it, so its rows merge from many pieces (more than
    the merge's one-wave-per-row limit of 16)."""
    cfg = cfg_for("bf16", 128, 16, 2, (30000,), P=64, append=True)
    w = make_workload(cfg, 930)
    ref, pk, pv = oracle.run_step(w)
    got, d = run(torch_dev, w, 64, True)
    launch = expect_even()
    assert_close(got, ref, "bf16", f"single request [{launch}]")
    assert pools_equal(d, pk, pv), launch


@pytest.mark.parametrize("B", [1024, 1025])
def test_even_split_batch_limit(torch_dev, B):
    """The prefix sum holds up to 1024 requests; one more takes the per-partition kernel."""
    rng = np.random.default_rng(B)
    lens = tuple(int(x) for x in rng.integers(0, 80, size=B))
    cfg = cfg_for("f16", 64, 8, 4, lens, P=32, append=False)
    w = make_workload(cfg, 940)
    ref, _, _ = oracle.run_step(w)
    got, _ = run(torch_dev, w, 32, False)
    launch = pkv.last_launch()
    assert launch.startswith("mxfp4_mfma_even " if B <= 1024 else "mxfp4_mfma "), launch
    zero = np.array(lens) == 0
    assert np.array_equal(got[zero], np.zeros_like(got[zero]))
    assert_close(got, ref, "f16", f"B={B} [{launch}]")


def test_even_split_bad_metadata_gives_nan_rows(torch_dev):
    """A block id past the pool or negative, or a length above max_context_len, makes that
    request's rows NaN; the other requests are exact."""
    lens = (300, 300, 300, 300, 17, 1000)
    cfg = cfg_for("bf16", 128, 16, 4, lens, P=64, append=False)
    w = make_workload(cfg, 950)
    ref, _, _ = oracle.run_step(w)
    bt = w.block_tables.copy()
    bt[1, 5] = w.n_blocks + 3
    bt[2, 18] = -1                        # the row's last block (tokens 288 .. 299)
    ctx = w.context_lens.copy()
    ctx[3] = 1001
    got = attention(torch_dev, w, 64, bt=bt, ctx=ctx, maxc=1000)
    launch = expect_even()
    for b in (1, 2, 3):
        assert np.all(np.isnan(got[b])), b
    good = [0, 4, 5]
    assert_close(got[good], ref[good], "bf16", f"good rows [{launch}]")


def test_even_split_repeatable_and_workspace_reuse(torch_dev):
    """Two calls sharing one workspace, the second with other lengths: both match the oracle,
    and a repeated call is bit-identical."""
    torch = torch_dev
    lens0 = (900, 33, 4000, 1, 2500)
    cfg = cfg_for("bf16", 128, 32, 8, lens0, P=256, append=False)
    w = make_workload(cfg, 960)
    ws = torch.empty(pkv.decode_workspace_bytes(5, 32, 128, w.max_context_len, 256), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for lens in (lens0, (850, 20, 4000, 0, 7)):   # within each request's blocks
        ctx = np.array(lens, dtype=np.int32)
        got = attention(torch, w, 256, ctx=ctx, ws=ws)
        expect_even()
        ref = oracle.paged_decode_attention_mxfp4("bf16", w.q, w.k_pool, w.v_pool, w.k_scale, w.v_scale,
                                                  w.block_tables, ctx, w.scale)
        assert_close(got, ref, "bf16", f"lens {lens}")
        outs.append(got)
    again = attention(torch, w, 256, ctx=np.array(lens0, dtype=np.int32), ws=ws)
    assert np.array_equal(again, outs[0])


def test_even_split_batch_with_no_blocks(torch_dev):
    """Every request empty, then every length past max_context_len: nothing is streamed and
    the merge writes zero rows, then NaN rows."""
    cfg = cfg_for("bf16", 64, 16, 4, (40, 40, 40, 40, 40), P=32, append=False)
    w = make_workload(cfg, 970)
    got = attention(torch_dev, w, 32, ctx=np.zeros(5, dtype=np.int32), maxc=40)
    expect_even()
    assert np.array_equal(got, np.zeros_like(got))
    got = attention(torch_dev, w, 32, ctx=np.full(5, 41, dtype=np.int32), maxc=40)
    expect_even()
    assert np.all(np.isnan(got))


def test_even_split_off_and_unsplit_steps_keep_the_partition_kernel(torch_dev, monkeypatch):
    """PKV_MX4_EVEN=0, or a step the caller does not split, runs the per-partition kernel."""
    cfg = cfg_for("bf16", 128, 16, 4, (700, 40), P=0, append=True)
    w = make_workload(cfg, 980)
    ref, pk, pv = oracle.run_step(w)
    got, d = run(torch_dev, w, 0, True)
    assert pkv.last_launch().startswith("mxfp4_mfma "), pkv.last_launch()
    assert_close(got, ref, "bf16", "unsplit")
    monkeypatch.setenv("PKV_MX4_EVEN", "0")
    got, d = run(torch_dev, w, 128, True)
    assert pkv.last_launch().startswith("mxfp4_mfma "), pkv.last_launch()
    assert_close(got, ref, "bf16", "even split off")
    assert pools_equal(d, pk, pv)


@pytest.mark.parametrize("B,lo,hi,even", [(32, 4096, 16384, True), (16, 4096, 16384, False),
                                           (32, 2048, 8192, False), (64, 128, 4096, False)])
def test_default_plan_takes_the_even_split_for_long_batches(torch_dev, monkeypatch, B, lo, hi, even):
    """Default plan (no override; 8 KV heads, 64 query heads, the bench's 1024-token partition):
    the even split when the batch's worst case -- B requests of the longest context -- holds at
    least 96 blocks per run and that context is at least 8192 tokens, the per-partition kernel
    at its 2048-token floor otherwise; both match the oracle, pools bit-exact."""
    for k in ("PKV_MX4_EVEN", "PKV_LP_MIN_PART"):
        monkeypatch.delenv(k, raising=False)
    lens = [int(x) for x in np.random.default_rng(B + hi).integers(lo, hi, size=B)]
    lens[0] = hi
    cfg = cfg_for("bf16", 128, 64, 8, tuple(lens), P=1024, append=True)
    w = make_workload(cfg, 990 + B)
    ref, pk, pv = oracle.run_step(w)
    got, d = run(torch_dev, w, 1024, True)
    launch = pkv.last_launch()
    assert launch.startswith("mxfp4_mfma_even " if even else "mxfp4_mfma "), launch
    assert_close(got, ref, "bf16", f"B={B} [{launch}]")
    assert pools_equal(d, pk, pv), launch
