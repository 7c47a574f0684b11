"""GPU: the step's device metadata against the kernels' contract (pkv_check_step_metadata),
and the append entry points' debug mode (PKV_DEBUG_CHECKS=1).

Each new token is given a slot of its own ("从 PagedAttention 到 Prefill-Decode 分离的深度
解析", section 2.2, step three): two appends of one step that name the same (block, slot)
are reported as PKV_ERR_ALIASED_APPEND, a length or block id outside the contract's range as
PKV_ERR_INVALID_ARG.  With the debug mode on, an aliased step is refused before anything is
launched (pools and output untouched), and a valid step gives the same bits as without it.
"""
import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_decode_loop import bits_equal
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def _aliased(w, b0, b1):
    """Make requests b0 and b1 append to the same (block, slot): b1's table row and position
    become b0's (b0's history is then b1's too, so each table stays valid)."""
    w.block_tables[b1] = w.block_tables[b0]
    w.positions[b1] = w.positions[b0]
    w.context_lens[b1] = w.context_lens[b0]


def test_valid_steps_pass(torch_dev):
    for name in ("c1", "c3", "c5"):
        w = make_workload(get_config(name, append=True), 3)
        d = upload(w)
        assert pkv.check_step_metadata(d["block_tables"], positions=d["positions"], n_blocks=w.n_blocks,
                                       max_context_len=w.max_context_len) == 0, pkv.last_error()
        assert pkv.check_step_metadata(d["block_tables"], context_lens=d["context_lens"], n_blocks=w.n_blocks,
                                       max_context_len=w.max_context_len) == 0, pkv.last_error()


@pytest.mark.parametrize("B,pair", [(2, (0, 1)), (80, (7, 70)), (700, (3, 650))])
def test_aliased_appends_are_reported(torch_dev, B, pair):
    torch = torch_dev
    lens = tuple(int(x) for x in np.random.default_rng(B).integers(1, 300, B))
    w = make_workload(get_config("c3", B=B, H_q=2, H_kv=2, lengths=("fixed", lens), append=True), 4)
    _aliased(w, *pair)
    d = upload(w)
    st = pkv.check_step_metadata(d["block_tables"], positions=d["positions"], n_blocks=w.n_blocks,
                                 max_context_len=w.max_context_len)
    assert st == pkv.PKV_ERR_ALIASED_APPEND, (st, pkv.last_error())
    # two tables sharing the block, appending to neighbouring slots of it: distinct targets
    w2 = make_workload(get_config("c3", B=B, H_q=2, H_kv=2, lengths=("fixed", lens), append=True), 4)
    b0, b1 = pair
    if w2.positions[b0] % 16 == 15:
        w2.positions[b0] -= 1
    w2.block_tables[b1] = w2.block_tables[b0]
    w2.positions[b1] = w2.positions[b0] + 1
    tb = torch.from_numpy(w2.block_tables).cuda()
    tp = torch.from_numpy(w2.positions).cuda()
    assert pkv.check_step_metadata(tb, positions=tp, n_blocks=w2.n_blocks) == 0, pkv.last_error()
    tp[b1] = int(w2.positions[b0])            # and the same slot again: aliased
    assert pkv.check_step_metadata(tb, positions=tp, n_blocks=w2.n_blocks) == pkv.PKV_ERR_ALIASED_APPEND


def test_out_of_range_metadata_is_reported(torch_dev):
    torch = torch_dev
    w = make_workload(get_config("c3", B=4, H_q=2, H_kv=2, lengths=("fixed", (40, 40, 40, 40)), append=True), 5)
    bt = w.block_tables.copy()
    bt[2, 1] = w.n_blocks                                # a block id past the pool, read by attention
    d = upload(w)
    tb = torch.from_numpy(bt).cuda()
    assert pkv.check_step_metadata(tb, positions=d["positions"], n_blocks=w.n_blocks, max_context_len=40) == \
        pkv.PKV_ERR_INVALID_ARG
    assert pkv.check_step_metadata(tb, context_lens=d["context_lens"], n_blocks=w.n_blocks, max_context_len=40) == \
        pkv.PKV_ERR_INVALID_ARG
    # a plain kv_append only writes the last block, which is in range
    assert pkv.check_step_metadata(tb, positions=d["positions"], n_blocks=w.n_blocks) == 0
    ctx = torch.from_numpy(np.array([40, 41, 40, 40], np.int32)).cuda()   # longer than max_context_len
    assert pkv.check_step_metadata(d["block_tables"], context_lens=ctx, n_blocks=w.n_blocks, max_context_len=40) == \
        pkv.PKV_ERR_INVALID_ARG


@pytest.mark.parametrize("kv", ["", "fp8", "mxfp4"])
def test_debug_mode_refuses_an_aliased_step(torch_dev, monkeypatch, kv):
    torch = torch_dev
    base = {"": "c5", "fp8": "c5f8", "mxfp4": "c5f4"}[kv]
    lens = (17, 300, 1025, 2000)
    w = make_workload(get_config(base, B=4, lengths=("fixed", lens), append=True, partition_size=512), 6)
    ref, kp, vp = oracle.run_step(w)
    monkeypatch.setenv("PKV_DEBUG_CHECKS", "1")
    # a valid step runs as without the checks: same bits as the oracle's pools, same tolerance
    d = upload(w)
    sc = (d["k_scale"], d["v_scale"]) if kv else ()
    fused = {"": pkv.append_decode_attention, "fp8": pkv.append_decode_attention_fp8,
             "mxfp4": pkv.append_decode_attention_mxfp4}[kv]
    out = fused(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], *sc, d["block_tables"], d["positions"],
                float(w.scale), w.max_context_len, partition_size=512)
    torch.cuda.synchronize()
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(np.isfinite(err)) and err.max() <= 2e-3
    if kv:
        assert bits_equal(d["k_pool"].cpu().numpy(), kp[0]) and bits_equal(d["v_scale"].cpu().numpy(), vp[1])
    else:
        assert bits_equal(to_numpy_bits(d["k_pool"], "bf16"), kp)
    # an aliased one is refused, by the fused step and by the plain append, before any launch
    _aliased(w, 1, 3)
    d = upload(w)
    sc = (d["k_scale"], d["v_scale"]) if kv else ()
    pools = [t.clone() for t in (d["k_pool"], d["v_pool"], *sc)]
    out = torch.full((4, w.cfg.H_q, w.cfg.D), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        fused(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], *sc, d["block_tables"], d["positions"],
              float(w.scale), w.max_context_len, partition_size=512, out=out)
    assert e.value.status == pkv.PKV_ERR_ALIASED_APPEND
    append = {"": pkv.kv_append, "fp8": pkv.kv_append_fp8, "mxfp4": pkv.kv_append_mxfp4}[kv]
    with pytest.raises(pkv.PkvError) as e:
        append(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], *sc, d["block_tables"], d["positions"])
    assert e.value.status == pkv.PKV_ERR_ALIASED_APPEND
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    for a, b in zip((d["k_pool"], d["v_pool"], *sc), pools):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
