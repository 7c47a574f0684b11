"""The allocation-free fused step (pkv_append_decode_attention_noalloc) through the C ABI.

Its split partials live in the library's own device array instead of a caller's
workspace; everything else is pkv_append_decode_attention's.  Two calls in a row,
the second on a smaller batch (so the array still holds the first call's larger
partials), must each equal the workspace entry point's output bit for bit and the
fp64 oracle to (2e-3, 1e-2) (f16/bf16) or (1e-5, 1e-5) (f32), with the pools after the
step bit-exact.  A split whose partials exceed PKV_NOALLOC_SCRATCH_BYTES is refused
with PKV_ERR_WORKSPACE before anything is launched.
"""
import ctypes

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_decode_loop import bits_equal
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits, upload

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
DT = {"f32": 0, "f16": 1, "bf16": 2}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def _call(lib, fn, w, d, P, out, ws=None):
    cfg = w.cfg
    V = ctypes.c_void_p
    args = [DT[cfg.dtype], V(out.data_ptr()), V(d["q"].data_ptr()), cfg.H_q * cfg.D, V(d["k_new"].data_ptr()),
            V(d["v_new"].data_ptr()), cfg.H_kv * cfg.D, V(d["k_pool"].data_ptr()), V(d["v_pool"].data_ptr()),
            V(d["block_tables"].data_ptr()), w.block_tables.shape[1], V(d["positions"].data_ptr()), cfg.B, cfg.H_q,
            cfg.H_kv, cfg.D, cfg.block_size, w.n_blocks, w.max_context_len, ctypes.c_float(float(w.scale)), P]
    if ws is not None:
        args += [V(ws.data_ptr()), ws.numel()]
    import torch
    return fn(*args, V(torch.cuda.current_stream().cuda_stream))


# (workload, overrides, partition size): the first call of each pair is the larger one
PAIRS = [
    (("c5", dict(B=8, lengths=("uniform", 4096, 16384)), 1024), ("c5", dict(B=3, lengths=("fixed", (1, 700, 5000))), 512)),
    (("c4", dict(B=16), 512), ("c4", dict(B=2, lengths=("fixed", (513, 40))), 256)),
    (("c1", {}, 16), ("c1", dict(B=1, lengths=("fixed", (9,))), 16)),
    (("c3", dict(B=6), 0), ("c3", dict(B=2, lengths=("fixed", (1, 300))), 0)),
]


# the even split of the grouped kernel keeps its prefix and pieces in the array too
EVEN = [(("c5", dict(B=12, lengths=("uniform", 4096, 16384)), 1024), ("c5", dict(B=5, lengths=("fixed", (1, 17, 700, 3000, 5000))), 256))]


@pytest.mark.parametrize("pair,env", [(p, {}) for p in PAIRS] + [(p, {"PKV_GQA_EVEN": "2"}) for p in EVEN],
                         ids=[f"{a[0]}-{b[0]}" for a, b in PAIRS] + ["c5-c5-even"])
def test_noalloc_matches_workspace_entry_point(torch_dev, monkeypatch, pair, env):
    torch = torch_dev
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    lib = pkv.load_library()
    for name, over, P in pair:
        cfg = get_config(name, append=True, **over)
        w = make_workload(cfg, 7)
        ref, kp, vp = oracle.run_step(w)
        d1, d2 = upload(w, "cuda"), upload(w, "cuda")
        out1 = torch.full((cfg.B, cfg.H_q, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
        out2 = out1.clone()
        need = pkv.decode_workspace_bytes(cfg.B, cfg.H_q, cfg.D, w.max_context_len, P)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        print(f"{name} B={cfg.B} P={P} partials={need} B", flush=True)
        assert _call(lib, lib.pkv_append_decode_attention, w, d1, P, out1, ws) == 0
        launch = pkv.last_launch()
        assert ("gqa_mfma_even " in launch) == bool(env), launch
        rc = _call(lib, lib.pkv_append_decode_attention_noalloc, w, d2, P, out2)
        assert rc == 0, lib.pkv_last_error().decode()
        assert pkv.last_launch() == launch
        torch.cuda.synchronize()
        a, b = out1.cpu().numpy(), out2.cpu().numpy()
        assert bits_equal(a, b), f"{name} P={P}: differs from the workspace entry point [{launch}]"
        atol, rtol = TOL[cfg.dtype]
        err = np.abs(b.astype(np.float64) - ref)
        assert np.all(np.isfinite(b)) and err.max() <= atol
        assert (err / np.maximum(np.abs(ref), atol / rtol)).max() <= rtol
        for t in (d1, d2):
            assert bits_equal(to_numpy_bits(t["k_pool"], cfg.dtype), kp)
            assert bits_equal(to_numpy_bits(t["v_pool"], cfg.dtype), vp)


def test_noalloc_refuses_partials_beyond_its_array(torch_dev):
    torch = torch_dev
    lib = pkv.load_library()
    cfg = get_config("c5", B=4, append=True, lengths=("fixed", (16, 16, 16, 16)))
    w = make_workload(cfg, 8)
    d = upload(w, "cuda")
    out = torch.empty((cfg.B, cfg.H_q, cfg.D), dtype=torch.float32, device="cuda")
    # claim a context of 2^24 tokens split every 16 tokens: 4 x 64 x 2^20 partitions of 129 floats
    w2 = make_workload(cfg, 8)
    w2.block_tables = np.zeros((cfg.B, 1 << 20), dtype=np.int32)
    big = {"max_context_len": 1 << 24}
    need = pkv.decode_workspace_bytes(cfg.B, cfg.H_q, cfg.D, big["max_context_len"], 16)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    bt = torch.from_numpy(w2.block_tables).cuda()
    V = ctypes.c_void_p
    rc = lib.pkv_append_decode_attention_noalloc(
        2, V(out.data_ptr()), V(d["q"].data_ptr()), cfg.H_q * cfg.D, V(d["k_new"].data_ptr()),
        V(d["v_new"].data_ptr()), cfg.H_kv * cfg.D, V(d["k_pool"].data_ptr()), V(d["v_pool"].data_ptr()),
        V(bt.data_ptr()), 1 << 20, V(d["positions"].data_ptr()), cfg.B, cfg.H_q, cfg.H_kv, cfg.D, 16, w.n_blocks,
        big["max_context_len"], ctypes.c_float(0.1), 16, V(torch.cuda.current_stream().cuda_stream))
    assert rc == -4, rc                       # PKV_ERR_WORKSPACE, nothing launched
    assert b"at most" in lib.pkv_last_error()
