"""The fused step as persistent workgroups (pkv_append_decode_attention_persistent)
against the oracle: outputs to the f16/bf16 tolerance, pools bit-exact, for grids
from one workgroup (every unit on one CU) to more workgroups than units."""
import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits, upload

from tests.test_gpu_parity import assert_close, prepared

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def run(torch, w, n_wg, P, max_ctx):
    t = upload(w)
    out = pkv.append_decode_attention_persistent(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"],
                                                 t["block_tables"], t["positions"], float(w.scale), max_ctx, n_wg,
                                                 partition_size=P)
    torch.cuda.synchronize()
    return out.cpu().numpy(), t


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P", [0, 256])
def test_persistent_step_parity(torch_dev, dtype, D, P):
    lens = (1, 2, 16, 17, 33, 100, 257, 1000, 4500)   # 4500 unsplit: two windows of block ids
    cfg = get_config("c3", B=len(lens), H_q=4, H_kv=4, D=D, dtype=dtype, lengths=("fixed", lens), append=True)
    w = make_workload(cfg, seed=61 + D + P)
    ref, kp_ref, vp_ref = oracle.run_step(w)
    for n_wg in (1, 7, 256, 4096):
        got, t = run(torch_dev, w, n_wg, P, max(lens))
        launch = pkv.last_launch()
        fields = dict(f.split("=") for f in launch.split() if "=" in f)
        assert launch.startswith("mha_persistent") and int(fields["grid"]) == min(n_wg, int(fields["units"])), launch
        assert_close(got, ref, dtype, f"persistent {dtype} D{D} P{P} n_wg={n_wg} [{launch}]")
        assert np.array_equal(to_numpy_bits(t["k_pool"], dtype).view(np.uint8), kp_ref.view(np.uint8))
        assert np.array_equal(to_numpy_bits(t["v_pool"], dtype).view(np.uint8), vp_ref.view(np.uint8))


def test_persistent_full_c3_step(torch_dev):
    """The large-batch workload at full size on 64 workgroups."""
    w, kp_ref, vp_ref, ref = prepared("c3")
    got, t = run(torch_dev, w, 64, 0, int(w.context_lens.max()))
    assert_close(got, ref, w.cfg.dtype, f"persistent c3 [{pkv.last_launch()}]")
    d = w.cfg.dtype
    assert np.array_equal(to_numpy_bits(t["k_pool"], d).view(np.uint8), kp_ref.view(np.uint8))
    assert np.array_equal(to_numpy_bits(t["v_pool"], d).view(np.uint8), vp_ref.view(np.uint8))


def test_persistent_refuses_grouped_and_f32(torch_dev):
    for dtype, H_q, H_kv in (("f32", 4, 4), ("bf16", 8, 2)):
        cfg = get_config("c3", B=2, H_q=H_q, H_kv=H_kv, D=64, dtype=dtype, lengths=("fixed", (5, 40)), append=True)
        w = make_workload(cfg, seed=3)
        with pytest.raises(pkv.PkvError):
            run(torch_dev, w, 8, 0, 40)


def test_persistent_step_beside_mfma_neighbour(torch_dev):
    """The step on 8 CUs while the MFMA-bound probe holds the others: same results."""
    torch = torch_dev
    lib = pkv.load_library()
    lens = (1, 17, 100, 257, 1000, 2049)
    cfg = get_config("c3", B=len(lens), H_q=8, H_kv=8, dtype="bf16", lengths=("fixed", lens), append=True)
    w = make_workload(cfg, seed=71)
    ref, kp_ref, vp_ref = oracle.run_step(w)
    n_cus = lib.pkv_device_cu_count()
    assert n_cus > 8
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    sg, sa = torch.cuda.Stream(), torch.cuda.Stream()
    t = upload(w)
    torch.cuda.synchronize()
    import ctypes
    assert lib.pkv_probe_mfma_burn(n_cus - 8, 20000, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(sg.cuda_stream)) == 0
    with torch.cuda.stream(sa):
        out = pkv.append_decode_attention_persistent(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"],
                                                     t["block_tables"], t["positions"], float(w.scale), max(lens), 8,
                                                     stream=sa)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    assert_close(out.cpu().numpy(), ref, "bf16", f"persistent beside neighbour [{pkv.last_launch()}]")
    assert np.array_equal(to_numpy_bits(t["k_pool"], "bf16").view(np.uint8), kp_ref.view(np.uint8))
    assert np.array_equal(to_numpy_bits(t["v_pool"], "bf16").view(np.uint8), vp_ref.view(np.uint8))


def _gemm_bound(a, b_t):
    """|g - r| bound for a float32 accumulation of K bf16 products (exact in float32):
    K * 2^-24 * sum_k |a_ik b_jk| per element, plus the float32 rounding of r itself."""
    A, Bt = np.abs(a.astype(np.float64)), np.abs(b_t.astype(np.float64))
    return a.shape[1] * 2.0 ** -24 * (A @ Bt.T) + 1e-30


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (512, 768, 320), (768, 256, 1024)])
def test_gemm_neighbour_matches_torch(torch_dev, M, N, K):
    """The HBM-streaming GEMM neighbour against a plain PyTorch reference on the CPU, on 1, 3
    and more workgroups than tiles."""
    torch = torch_dev
    g = torch.Generator().manual_seed(M + N + K)
    a = (torch.rand((M, K), generator=g) * 2 - 1).to(torch.bfloat16)
    b_t = (torch.rand((N, K), generator=g) * 2 - 1).to(torch.bfloat16)
    ref = (a.double() @ b_t.double().T).numpy()                  # bf16 values are exact in float64
    bound = _gemm_bound(a.float().numpy(), b_t.float().numpy())
    da, db = a.cuda(), b_t.cuda()
    for n_wg in (1, 3, 64):
        c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        pkv.probe_gemm_bf16(da, db, c, n_wg)
        torch.cuda.synchronize()
        got = c.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), n_wg
        err = np.abs(got - ref)
        assert np.all(err <= bound), f"n_wg={n_wg}: max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}"


def test_gemm_neighbour_refuses_bad_shapes(torch_dev):
    torch = torch_dev
    a = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    lib = pkv.load_library()
    import ctypes
    V = ctypes.c_void_p
    for M, N, K in ((250, 256, 64), (256, 100, 64), (256, 256, 48), (256, 256, 0)):
        assert lib.pkv_probe_gemm_bf16(4, V(a.data_ptr()), V(a.data_ptr()), V(c.data_ptr()), M, N, K, None) == -2
    assert lib.pkv_probe_gemm_bf16(0, V(a.data_ptr()), V(a.data_ptr()), V(c.data_ptr()), 256, 256, 64, None) == -2


def test_persistent_step_beside_gemm_neighbour(torch_dev):
    """The step on 8 CUs while the GEMM neighbour streams its operands on all the others:
    both results hold (the step against the oracle, sampled GEMM rows against float64)."""
    torch = torch_dev
    lib = pkv.load_library()
    lens = (1, 17, 100, 257, 1000, 2049)
    cfg = get_config("c3", B=len(lens), H_q=8, H_kv=8, dtype="bf16", lengths=("fixed", lens), append=True)
    w = make_workload(cfg, seed=72)
    ref, kp_ref, vp_ref = oracle.run_step(w)
    n_cus = lib.pkv_device_cu_count()
    M = N = K = 2048
    g = torch.Generator().manual_seed(9)
    a = (torch.rand((M, K), generator=g) * 2 - 1).to(torch.bfloat16)
    b_t = (torch.rand((N, K), generator=g) * 2 - 1).to(torch.bfloat16)
    da, db = a.cuda(), b_t.cuda()
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    sg, sa = torch.cuda.Stream(), torch.cuda.Stream()
    t = upload(w)
    torch.cuda.synchronize()
    pkv.probe_gemm_bf16(da, db, c, n_cus - 8, stream=sg)
    with torch.cuda.stream(sa):
        out = pkv.append_decode_attention_persistent(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"],
                                                     t["block_tables"], t["positions"], float(w.scale), max(lens), 8,
                                                     stream=sa)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", f"persistent beside the GEMM [{pkv.last_launch()}]")
    assert np.array_equal(to_numpy_bits(t["k_pool"], "bf16").view(np.uint8), kp_ref.view(np.uint8))
    assert np.array_equal(to_numpy_bits(t["v_pool"], "bf16").view(np.uint8), vp_ref.view(np.uint8))
    rows = np.random.default_rng(1).choice(M, 6, replace=False)
    got = c.cpu().numpy()[rows].astype(np.float64)
    want = (a[rows].double() @ b_t.double().T).numpy()
    assert np.all(np.abs(got - want) <= _gemm_bound(a[rows].float().numpy(), b_t.float().numpy()))
