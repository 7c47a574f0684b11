"""GPU: a local and an offloaded attention batch per step, captured over a (local capacity,
offloaded capacity) grid as two parallel graph branches (and, for comparison, one after the
other).  Each branch has its own q, new rows, pools, tables, positions, output and workspace.
Every replay -- for batch pairs that pick different buckets, padding rows included, with the
program's own eager GPU work and synchronisations between replays -- is checked against the
oracle: each branch's first B rows to the dtype's tolerance, both pools bit for bit; padding
rows come out NaN and rows past the bucket are never written."""
import copy

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_decode_loop import bits_equal
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits, upload

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def _first(w, B):
    """The workload's first B requests (pools shared)."""
    s = copy.copy(w)
    s.q, s.block_tables, s.context_lens = w.q[:B], w.block_tables[:B], w.context_lens[:B]
    s.positions, s.k_new, s.v_new = w.positions[:B], w.k_new[:B], w.v_new[:B]
    return s


class Branch:
    """Fixed device buffers for one branch, sized for its largest capacity, plus pristine pools."""

    def __init__(self, torch, w, cap, P):
        self.w, self.cap, self.P, self.torch = w, cap, P, torch
        d = upload(w)
        self.pristine = {k: d[k].clone() for k in ("k_pool", "v_pool") + (("k_scale", "v_scale") if w.cfg.kv_dtype
                                                                          else ())}
        self.bufs = {"q": d["q"], "k_new": d["k_new"], "v_new": d["v_new"], "k_pool": d["k_pool"],
                     "v_pool": d["v_pool"], "block_tables": d["block_tables"].clone(),
                     "positions": d["positions"].clone(),
                     "out": torch.full((cap, w.cfg.H_q, w.cfg.D), 7.0, dtype=torch.float32, device="cuda")}
        if w.cfg.kv_dtype:
            self.bufs["k_scale"], self.bufs["v_scale"] = d["k_scale"], d["v_scale"]
        self.bufs["partition_size"] = P
        if P:
            need = pkv.decode_workspace_bytes(cap, w.cfg.H_q, w.cfg.D, 2048, P)
            self.bufs["workspace"] = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.full_tables, self.full_pos = d["block_tables"].clone(), d["positions"].clone()

    def prepare(self, B):
        """Restore the pools, keep rows [0, B) and pad [B, cap) with position -1."""
        for k, v in self.pristine.items():
            self.bufs[k].copy_(v)
        self.bufs["positions"].copy_(self.full_pos)
        self.bufs["positions"][B:] = -1
        self.bufs["out"].fill_(7.0)

    def check(self, B, bucket_cap, what):
        w = self.w
        got = self.bufs["out"].cpu().numpy()
        if B:
            sub = _first(w, B)
            ref, kp, vp = oracle.run_step(sub)
            atol, rtol = TOL[w.cfg.dtype]
            g = got[:B].astype(np.float64)
            err = np.abs(g - ref)
            assert np.all(np.isfinite(g)) and err.max() <= atol, f"{what}: max_abs {err.max():.3e}"
            assert (err / np.maximum(np.abs(ref), atol / rtol)).max() <= rtol, what
            if w.cfg.kv_dtype:
                for k, r in (("k_pool", kp[0]), ("k_scale", kp[1]), ("v_pool", vp[0]), ("v_scale", vp[1])):
                    assert bits_equal(self.bufs[k].cpu().numpy(), r), f"{what}: {k}"
            else:
                assert bits_equal(to_numpy_bits(self.bufs["k_pool"], w.cfg.dtype), kp), what
                assert bits_equal(to_numpy_bits(self.bufs["v_pool"], w.cfg.dtype), vp), what
        else:
            for k, v in self.pristine.items():   # bitwise: unwritten slots hold NaN poison
                assert self.torch.equal(self.bufs[k].view(self.torch.uint8), v.view(self.torch.uint8)), what
        assert np.all(np.isnan(got[B:bucket_cap])), f"{what}: padding rows"
        assert np.all(got[bucket_cap:] == 7.0), f"{what}: rows past the bucket"


@pytest.mark.parametrize("parallel", [True, False])
@pytest.mark.parametrize("off_kind", ["", "fp8"])
def test_dual_graph_replays_match_oracle(torch_dev, parallel, off_kind):
    torch = torch_dev
    print(f"dual graphs parallel={parallel} offloaded={off_kind or 'f16'}", flush=True)
    lcaps, ocaps = [0, 2, 4, 6], [0, 3, 5]
    wl = make_workload(get_config("c5", B=6, lengths=("fixed", (1, 17, 300, 1025, 1500, 2048)), append=True,
                                  pool=("factor", 1.3)), 301)
    base = "c3f8" if off_kind == "fp8" else "c3"
    wo = make_workload(get_config(base, B=5, lengths=("fixed", (40, 2048, 16, 700, 129)), append=True), 302)
    local = Branch(torch, wl, lcaps[-1], 256)
    off = Branch(torch, wo, ocaps[-1], 0)
    # the local branch is split every 256 tokens, the offloaded one runs unsplit
    g = pkv.DualStepGraphs(local.bufs, off.bufs, float(wl.scale), lcaps, ocaps, 2048, parallel=parallel)
    s = torch.cuda.Stream()
    for Bl, Bo in ((6, 5), (1, 0), (0, 2), (3, 3), (4, 5), (0, 0), (2, 1), (6, 5)):
        local.prepare(Bl)
        off.prepare(Bo)
        torch.cuda.synchronize()
        g.launch(Bl, Bo, stream=s)
        torch.cuda.synchronize()
        lc = next(c for c in lcaps if c >= Bl)
        oc = next(c for c in ocaps if c >= Bo)
        local.check(Bl, lc, f"local B={Bl}")
        off.check(Bo, oc, f"offloaded B={Bo}")
        # the program's own eager work between replays
        x = torch.randn((512, 512), device="cuda")
        (x @ x).sum().item()


def test_dual_graph_argument_checks(torch_dev):
    torch = torch_dev
    wl = make_workload(get_config("c5", B=2, lengths=("fixed", (17, 300)), append=True), 303)
    a = Branch(torch, wl, 2, 256)
    b = Branch(torch, wl, 2, 256)
    with pytest.raises(pkv.PkvError):            # one workspace for two concurrent branches
        b.bufs["workspace"] = a.bufs["workspace"]
        pkv.DualStepGraphs(a.bufs, b.bufs, float(wl.scale), [2], [2], 300, partition_size=256)
    b.bufs["workspace"] = torch.empty_like(a.bufs["workspace"])
    with pytest.raises(pkv.PkvError):            # capacities must increase
        pkv.DualStepGraphs(a.bufs, b.bufs, float(wl.scale), [2, 2], [2], 300, partition_size=256)
    g = pkv.DualStepGraphs(a.bufs, b.bufs, float(wl.scale), [0, 2], [1, 2], 300, partition_size=256)
    with pytest.raises(pkv.PkvError):            # more than the largest capacity
        g.launch(3, 1)
    g.launch(0, 0)                               # nothing to run
