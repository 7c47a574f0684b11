"""GPU parity of the exact step bench.py times, at full size, for every workload it can time.

The C-ABI call and its arguments come from bench.resident_steps (the same function the
timed region replays); the test runs that call once on the first input set and checks every
output row against the fp64 oracle, (2e-3, 1e-2) for f16/bf16 q and (1e-5, 1e-5) for f32 q,
and the whole K/V pools (FP8 and MXFP4: codes and scales) bit for bit against the oracle's
append.  The launch string of that call must also be the one the Python binding's own call
picks for the same arguments.
"""
import ctypes

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_decode_loop import bits_equal
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
# the kernel each workload's step must run (prefix of pkv.last_launch())
KERNEL = {"c1": "mha ", "c2": "mha ", "c3": "mha ", "c4": "mha ", "c5": "gqa_mfma_even ", "c3f8": "fp8 ",
          "c5f8": "gqa_mfma_fp8 ", "c3f4": "mxfp4 ", "c5f4": "mxfp4_mfma_even "}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c3f8", "c5f8", "c3f4", "c5f4"])
def test_bench_step_parity(torch_dev, name):
    import bench

    torch = torch_dev
    dev = torch.device("cuda:0")
    lib = pkv.load_library()
    cfg = get_config(name)
    P = cfg.partition_size
    w = make_workload(cfg, None, append=True)            # what bench.main draws by default
    calls, sets = bench.resident_steps(lib, torch, pkv, dev, w, True, P, 1)
    fn, args = calls[0]
    print(f"{name}: B={cfg.B} sum(n)={int(w.context_lens.sum())} P={P}", flush=True)
    rc = fn(*args, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, pkv.last_launch()
    launch = pkv.last_launch()
    torch.cuda.synchronize()
    got = sets[0]["out"].cpu().numpy()
    assert launch.startswith(KERNEL[name]) and "fused_append" in launch, launch
    if name == "c5f8":                      # the grouped FP8 kernel's 2048-token floor
        assert "part_tokens=2048 " in launch, launch

    ref, kp, vp = oracle.run_step(w)
    atol, rtol = TOL[cfg.dtype]
    g = got.astype(np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output [{launch}]"
    err = np.abs(g - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    assert err.max() <= atol and rel.max() <= rtol, \
        f"{name}: max_abs={err.max():.3e} max_rel={rel.max():.3e} [{launch}]"
    s = sets[0]
    if cfg.fp8 or cfg.mxfp4:
        assert bits_equal(s["k_pool"].cpu().numpy(), kp[0]) and bits_equal(s["k_scale"].cpu().numpy(), kp[1])
        assert bits_equal(s["v_pool"].cpu().numpy(), vp[0]) and bits_equal(s["v_scale"].cpu().numpy(), vp[1])
    else:
        assert bits_equal(to_numpy_bits(s["k_pool"], cfg.dtype), kp)
        assert bits_equal(to_numpy_bits(s["v_pool"], cfg.dtype), vp)
    print(f"{name}: max_abs={err.max():.2e} max_rel={rel.max():.2e} [{launch}]", flush=True)

    # the binding's own call over the same tensors plans the same launch
    del sets, calls
    from workloads.device import upload
    d = upload(w, dev)
    if cfg.fp8 or cfg.mxfp4:
        f = pkv.append_decode_attention_fp8 if cfg.fp8 else pkv.append_decode_attention_mxfp4
        f(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"], d["block_tables"],
          d["positions"], float(w.scale), w.max_context_len, partition_size=P)
    else:
        pkv.append_decode_attention(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["block_tables"],
                                    d["positions"], float(w.scale), w.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    assert pkv.last_launch() == launch, (pkv.last_launch(), launch)
