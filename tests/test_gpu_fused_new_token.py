"""GPU parity of the fused low-precision step at the new token's edge positions.

In the fused step the grouped FP8 and MXFP4 kernels quantize the new token
themselves (the workgroup whose partition ends at the new position) and write it
to the pools; the per-head kernels and the plain path are covered elsewhere.
These cases put the new position at slot 0 and slot 15 of a block, alone in its
partition and at a partition's end, with ragged and full last blocks, for
grouped heads on the two-block (G <= 8) and one-block (G = 16) paths: the
output must match the oracle and the pools the oracle's append bit for bit."""
import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from workloads import get_config, make_workload
from workloads.device import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def small_partitions(monkeypatch):
    """The grouped low-precision kernels split at no less than 2048 tokens by default; these
    tests exercise the caller's own small partitions (the floor has its own tests)."""
    monkeypatch.setenv("PKV_LP_MIN_PART", "0")

TOL = {"f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
# context lengths n: the new token sits at n - 1
LENS = (1, 2, 16, 17, 32, 33, 48, 49, 64, 65, 100)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and a.view(np.uint8).tobytes() == b.view(np.uint8).tobytes()


@pytest.mark.parametrize("kv", ["fp8", "mx4"])
@pytest.mark.parametrize("dtype,D,H_q,H_kv", [("bf16", 128, 16, 2), ("f16", 128, 16, 1), ("f16", 64, 8, 4)])
@pytest.mark.parametrize("P", [0, 32])
def test_fused_new_token_edges(torch_dev, kv, dtype, D, H_q, H_kv, P):
    torch = torch_dev
    base = "c3f8" if kv == "fp8" else "c3f4"
    cfg = get_config(base, dtype=dtype, D=D, H_q=H_q, H_kv=H_kv, B=len(LENS), lengths=("fixed", LENS),
                     pool=("factor", 1.3), append=True, partition_size=P)
    w = make_workload(cfg, 83)
    ref, pk, pv = oracle.run_step(w)
    d = upload(w, "cuda")
    call = pkv.append_decode_attention_fp8 if kv == "fp8" else pkv.append_decode_attention_mxfp4
    out = call(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
               d["block_tables"], d["positions"], float(w.scale), w.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    launch = pkv.last_launch()
    assert launch.startswith("gqa_mfma_fp8" if kv == "fp8" else "mxfp4_mfma "), launch
    got = out.cpu().numpy().astype(np.float64)
    atol, rtol = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{kv} {dtype} G{H_q // H_kv} P{P}: non-finite output"
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    assert err.max() <= atol and rel.max() <= rtol, \
        f"{kv} {dtype} G{H_q // H_kv} P{P}: max_abs={err.max():.3e} max_rel={rel.max():.3e} [{launch}]"
    assert bits_equal(d["k_pool"].cpu().numpy(), pk[0]) and bits_equal(d["v_pool"].cpu().numpy(), pv[0])
    assert bits_equal(d["k_scale"].cpu().numpy(), pk[1]) and bits_equal(d["v_scale"].cpu().numpy(), pv[1])
