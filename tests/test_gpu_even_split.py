"""GPU: the even split of a grouped 16-bit split step (the batch's blocks, requests end to
end, cut into equal runs with one wave per run and KV head; then a log-sum-exp merge of each
row's pieces) against the fp64 oracle.

Small batches give runs of about 16 blocks, so requests are cut into many pieces at varied
offsets, runs cross from one request into the next, and a request of one block is a whole
piece; lengths mix 0, ragged tails and block multiples; the fused step writes the new token
from the piece holding the row's last block (pools bit-exact).  Out-of-range lengths and
block ids give NaN rows for their request only.  Tolerances as elsewhere:
(atol, rtol) = (2e-3, 1e-2) for f16/bf16.
"""
import os

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits, to_tensor, upload

pytestmark = pytest.mark.gpu

TOL = {"f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
LENS = (0, 1, 15, 16, 17, 33, 100, 255, 256, 257, 700, 1000, 1500)
EVEN_VARIANTS = [(4, 1), (2, 1), (8, 1)]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


@pytest.fixture(autouse=True)
def force_even(monkeypatch):
    """These batches are small: the plan's default takes the even split only for batches of
    at least ~1/16 as many requests as runs; 2 takes it wherever it applies."""
    monkeypatch.setenv("PKV_GQA_EVEN", "2")


@pytest.fixture
def env(monkeypatch):
    def set_(d):
        for k, v in d.items():
            monkeypatch.setenv(k, str(v))
    return set_


def assert_close(got, ref, dtype, what):
    atol, rtol = TOL[dtype]
    g = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    assert err.max() <= atol and rel.max() <= rtol, f"{what}: max_abs={err.max():.3e} max_rel={rel.max():.3e}"


def attention(torch, w, P, bt=None, ctx=None, maxc=None):
    d = w.cfg.dtype
    q = to_tensor(w.q, d, "cuda")
    k = to_tensor(w.k_pool, d, "cuda")
    v = to_tensor(w.v_pool, d, "cuda")
    bt = torch.from_numpy(w.block_tables if bt is None else bt).cuda()
    ctx = w.context_lens if ctx is None else ctx
    maxc = int(w.context_lens.max()) if maxc is None else maxc
    out = pkv.paged_decode_attention(q, k, v, bt, torch.from_numpy(ctx).cuda(), float(w.scale), maxc,
                                     partition_size=P)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [2, 4, 8, 16])
def test_even_split_attention(torch_dev, dtype, D, G):
    cfg = get_config("c5", B=len(LENS), H_q=2 * G, H_kv=2, D=D, dtype=dtype, lengths=("fixed", LENS),
                     pool=("factor", 1.3))
    w = make_workload(cfg, seed=700 + G + D)
    ref = oracle.paged_decode_attention(dtype, w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    for P in (32, 256):
        got = attention(torch_dev, w, P)
        launch = pkv.last_launch()
        assert launch.startswith("gqa_mfma_even ") and "even_waves=" in launch, launch
        assert np.array_equal(got[0], np.zeros_like(got[0]))          # empty context -> zero rows
        assert_close(got, ref, dtype, f"{dtype} D={D} G={G} P={P} [{launch}]")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("G", [4, 8])
def test_even_split_fused_step(torch_dev, dtype, G):
    torch = torch_dev
    lens = LENS[1:]
    cfg = get_config("c5", B=len(lens), H_q=2 * G, H_kv=2, dtype=dtype, lengths=("fixed", lens),
                     pool=("factor", 1.3), append=True)
    w = make_workload(cfg, seed=710 + G)
    ref, kp_ref, vp_ref = oracle.run_step(w)
    for P in (32, 1024):
        t = upload(w)
        out = pkv.append_decode_attention(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"],
                                          t["block_tables"], t["positions"], float(w.scale), max(lens),
                                          partition_size=P)
        torch.cuda.synchronize()
        launch = pkv.last_launch()
        assert launch.startswith("gqa_mfma_even ") and launch.endswith("fused_append"), launch
        assert_close(out.cpu().numpy(), ref, dtype, f"fused {dtype} G={G} P={P} [{launch}]")
        assert np.array_equal(to_numpy_bits(t["k_pool"], dtype).view(np.uint8), kp_ref.view(np.uint8))
        assert np.array_equal(to_numpy_bits(t["v_pool"], dtype).view(np.uint8), vp_ref.view(np.uint8))


@pytest.mark.parametrize("variant", EVEN_VARIANTS)
def test_even_split_variants_and_against_the_other_split(torch_dev, env, variant):
    """Every instantiated (waves, blocks ahead) shape, and the per-partition split it replaces
    (PKV_GQA_EVEN=0), on one long-context batch: both match the oracle."""
    nw, pf = variant
    lens = (4096, 7000, 16384, 9, 12000, 5000)
    cfg = get_config("c5", B=len(lens), lengths=("fixed", lens), pool=("factor", 1.2))
    w = make_workload(cfg, seed=720 + nw)
    ref = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    env({"PKV_GQA_EVEN_NW": nw, "PKV_GQA_EVEN_PF": pf})
    got = attention(torch_dev, w, 1024)
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_even ") and f"nw={nw} ch=1 pf={pf}" in launch, launch
    assert_close(got, ref, "bf16", f"even {variant} [{launch}]")
    env({"PKV_GQA_EVEN": 0})
    got2 = attention(torch_dev, w, 1024)
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_kdma "), launch
    assert_close(got2, ref, "bf16", f"per-partition split [{launch}]")


def test_even_split_single_long_request(torch_dev):
    """One request: every run lies inside it, so each row is merged from many pieces."""
    cfg = get_config("c5", B=1, H_q=16, H_kv=2, lengths=("fixed", (60000,)), pool=("factor", 1.0))
    w = make_workload(cfg, seed=730)
    ref = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    got = attention(torch_dev, w, 512)
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_even "), launch
    assert_close(got, ref, "bf16", f"single request [{launch}]")


@pytest.mark.parametrize("B", [1024, 1025])
def test_even_split_batch_limit(torch_dev, B):
    """The prefix sum holds up to 1024 requests; one more takes the per-partition split."""
    rng = np.random.default_rng(B)
    lens = tuple(int(x) for x in rng.integers(0, 80, size=B))
    cfg = get_config("c5", B=B, H_q=8, H_kv=2, D=64, dtype="f16", lengths=("fixed", lens), pool=("factor", 1.1))
    w = make_workload(cfg, seed=740)
    ref = oracle.paged_decode_attention("f16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    got = attention(torch_dev, w, 32)
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_even " if B <= 1024 else "gqa_mfma_kdma "), launch
    zero = np.array(lens) == 0
    assert np.array_equal(got[zero], np.zeros_like(got[zero]))
    assert_close(got, ref, "f16", f"B={B} [{launch}]")


def test_even_split_bad_metadata_gives_nan_rows(torch_dev):
    """A block id past the pool or negative, or a length above max_context_len, makes that
    request's rows NaN (every KV head's wave meets the bad id); the other requests are exact."""
    lens = (300, 300, 300, 300, 17, 1000)
    cfg = get_config("c5", B=len(lens), H_q=8, H_kv=2, lengths=("fixed", lens), pool=("factor", 2.0))
    w = make_workload(cfg, seed=750)
    ref = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    bt = w.block_tables.copy()
    bt[1, 5] = w.n_blocks + 3
    bt[2, 18] = -1                        # the row's last block (tokens 288 .. 299)
    ctx = w.context_lens.copy()
    ctx[3] = 1001
    got = attention(torch_dev, w, 64, bt=bt, ctx=ctx, maxc=1000)
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_even "), launch
    for b in (1, 2, 3):
        assert np.all(np.isnan(got[b])), b
    good = [0, 4, 5]
    assert_close(got[good], ref[good], "bf16", f"good rows [{launch}]")


def test_even_split_repeatable_and_workspace_reuse(torch_dev):
    """Two calls sharing one workspace, the second with other lengths: both match the oracle,
    and a repeated call is bit-identical (pieces merged in index order)."""
    torch = torch_dev
    cfg = get_config("c5", B=5, H_q=16, H_kv=2, lengths=("fixed", (900, 33, 4000, 1, 2500)), pool=("factor", 1.3))
    w = make_workload(cfg, seed=760)
    ref = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    d = upload(w)
    ws = torch.empty(pkv.decode_workspace_bytes(5, 16, 128, 4000, 256), dtype=torch.uint8, device="cuda")
    outs = []
    for lens in ((900, 33, 4000, 1, 2500), (850, 20, 4000, 0, 7)):   # within each request's blocks
        ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
        o = pkv.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], ctx, float(w.scale),
                                       4000, partition_size=256, workspace=ws)
        torch.cuda.synchronize()
        assert pkv.last_launch().startswith("gqa_mfma_even ")
        r = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables,
                                          np.array(lens, dtype=np.int32), w.scale)
        assert_close(o.cpu().numpy(), r, "bf16", f"lens {lens}")
        outs.append(o.clone())
    ctx = torch.tensor((900, 33, 4000, 1, 2500), dtype=torch.int32, device="cuda")
    again = pkv.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], ctx, float(w.scale),
                                       4000, partition_size=256, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again, outs[0])
    assert_close(outs[0].cpu().numpy(), ref, "bf16", "first call")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
def test_even_split_merge_of_many_pieces_beside_short_rows(torch_dev, dtype, D):
    """Two query heads per request, so a merge workgroup's four rows span two requests: rows of
    a hundred pieces (shared by the four waves) next to an empty request, a one-piece request
    and a length past max_context_len (NaN)."""
    torch = torch_dev
    lens = (0, 40000, 17, 30000, 5, 40000)
    cfg = get_config("c5", B=len(lens), H_q=2, H_kv=1, D=D, dtype=dtype, lengths=("fixed", lens),
                     pool=("factor", 1.0))
    w = make_workload(cfg, seed=770 + D)
    ref = oracle.paged_decode_attention(dtype, w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    ctx = w.context_lens.copy()
    ctx[4] = 40001
    got = attention(torch, w, 256, ctx=ctx, maxc=40000)
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_even "), launch
    assert np.array_equal(got[0], np.zeros_like(got[0]))
    assert np.all(np.isnan(got[4]))
    good = [1, 2, 3, 5]
    assert_close(got[good], ref[good], dtype, f"{dtype} D={D} [{launch}]")


@pytest.mark.parametrize("B,lo,hi,even", [(32, 4096, 16384, True), (16, 4096, 16384, True), (8, 1024, 16384, False),
                                           (8, 4096, 32768, True), (4, 4096, 8192, False)])
def test_default_plan_takes_the_even_split_for_long_runs(torch_dev, monkeypatch, B, lo, hi, even):
    """Default plan (no override, 8 KV heads, 256 runs of one resident round): the even split
    when the batch's worst case -- B requests of the longest context -- holds at least 64
    blocks per run (here B * hi / 16 >= 16384, the longest request being hi tokens), nw-partition
    spans otherwise; both match the oracle."""
    monkeypatch.delenv("PKV_GQA_EVEN", raising=False)
    lens = [int(x) for x in np.random.default_rng(B + hi).integers(lo, hi, size=B)]
    lens[0] = hi
    cfg = get_config("c5", B=B, lengths=("fixed", tuple(lens)), pool=("factor", 1.1))
    w = make_workload(cfg, seed=780 + B)
    ref = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    got = attention(torch_dev, w, 1024)
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_even " if even else "gqa_mfma_kdma "), launch
    assert_close(got, ref, "bf16", f"B={B} [{launch}]")


def test_even_split_batch_with_no_blocks(torch_dev):
    """Every request empty, then every length past max_context_len: the split streams nothing
    (one run of nothing) and the merge writes zero rows, then NaN rows."""
    cfg = get_config("c5", B=5, H_q=16, H_kv=2, lengths=("fixed", (40, 40, 40, 40, 40)), pool=("factor", 1.5))
    w = make_workload(cfg, seed=790)
    zero = np.zeros(5, dtype=np.int32)
    got = attention(torch_dev, w, 32, ctx=zero, maxc=40)
    assert pkv.last_launch().startswith("gqa_mfma_even "), pkv.last_launch()
    assert np.array_equal(got, np.zeros_like(got))
    got = attention(torch_dev, w, 32, ctx=np.full(5, 41, dtype=np.int32), maxc=40)
    assert np.all(np.isnan(got))
