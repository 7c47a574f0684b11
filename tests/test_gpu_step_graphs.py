"""GPU: the fused decode step captured as HIP graphs over (batch, context)
capacity buckets, replayed many times with fresh data and with the program's
own eager GPU work and synchronisations between replays.  Every replay is
checked against the same step run eagerly through the library (on a second
copy of the pools) and against the oracle: outputs to the dtype's tolerance,
pools bit for bit.  Padding rows up to the bucket's batch capacity come out
NaN; rows beyond it are never touched."""
import math

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from oracle.block_manager import copy_blocks as oracle_copy_blocks
from tests.test_gpu_decode_loop import BS, TOL, bits_equal, draw, poisoned_pool
from workloads.device import to_numpy_bits, to_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def close(got, ref, dtype):
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    return float(err.max()) <= atol and float(rel.max()) <= rtol, (float(err.max()), float(rel.max()))


@pytest.mark.parametrize("dtype,H_q,H_kv,D,P,cow,seed", [
    ("f16", 8, 2, 128, 32, True, 201),
    ("bf16", 4, 4, 128, 0, True, 202),
    ("f32", 2, 2, 64, 16, False, 203),
    ("bf16", 16, 2, 64, 0, False, 204),
])
def test_graph_replays_match_eager_and_oracle(torch_dev, dtype, H_q, H_kv, D, P, cow, seed):
    t = torch_dev
    print(f"step graphs {dtype} H_q={H_q} H_kv={H_kv} D={D} P={P} cow={cow} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    Bmax, bcaps, ccaps = 8, [2, 4, 8], [48, 96, 160]
    W, n_blocks = ccaps[-1] // BS, 120
    scale = 1.0 / math.sqrt(D)
    kp = poisoned_pool(dtype, n_blocks, H_kv, D)
    vp = kp.copy()
    kg, vg = to_tensor(kp, dtype, "cuda"), to_tensor(vp, dtype, "cuda")     # graph side
    ke, ve = to_tensor(kp, dtype, "cuda"), to_tensor(vp, dtype, "cuda")     # eager side
    tdt = kg.dtype
    q_buf = t.zeros((Bmax, H_q, D), dtype=tdt, device="cuda")
    kn_buf = t.zeros((Bmax, H_kv, D), dtype=tdt, device="cuda")
    vn_buf = t.zeros((Bmax, H_kv, D), dtype=tdt, device="cuda")
    bt_buf = t.full((Bmax, W), -1, dtype=t.int32, device="cuda")
    pos_buf = t.full((Bmax,), -1, dtype=t.int32, device="cuda")
    out_buf = t.full((Bmax, H_q, D), 7.0, dtype=t.float32, device="cuda")
    cs = t.full((Bmax,), -1, dtype=t.int32, device="cuda") if cow else None
    cd = t.full((Bmax,), -1, dtype=t.int32, device="cuda") if cow else None
    graphs = pkv.StepGraphs(q_buf, kn_buf, vn_buf, kg, vg, bt_buf, pos_buf, out_buf, scale, bcaps, ccaps,
                            partition_size=P, cow_src=cs, cow_dst=cd)

    bm = pkv.BlockManager(n_blocks, BS, shuffle_seed=seed)
    live, next_id = [], [0]

    def write_prompt(sid, n):
        if n == 0:
            return
        kn, vn = draw(rng, dtype, (n, H_kv, D)), draw(rng, dtype, (n, H_kv, D))
        table = bm.block_table(sid)
        bt = np.full((n, W), -1, dtype=np.int32)
        bt[:, :table.size] = table
        pos = np.arange(n, dtype=np.int32)
        oracle.kv_append(dtype, kn, vn, kp, vp, bt, pos, BS)
        for k, v in ((kg, vg), (ke, ve)):
            pkv.kv_append(to_tensor(kn, dtype, "cuda"), to_tensor(vn, dtype, "cuda"), k, v,
                          t.from_numpy(bt).cuda(), t.from_numpy(pos).cuda())

    replays, used = 0, set()
    for step in range(30):
        # requests arrive, fork (copy-on-write) and finish between steps
        while len(live) < 2 or (rng.random() < 0.3 and len(live) < Bmax):
            sid, next_id[0] = next_id[0], next_id[0] + 1
            n = int(rng.integers(1, 100))
            bm.add_sequence(sid, n)
            write_prompt(sid, n)
            live.append(sid)
        if cow and rng.random() < 0.5 and len(live) < Bmax:
            sid, next_id[0] = next_id[0], next_id[0] + 1
            bm.fork(live[int(rng.integers(len(live)))], sid)
            live.append(sid)
        for sid in list(live):
            if bm.sequence_length(sid) >= ccaps[-1] - 1 or (len(live) > 2 and rng.random() < 0.08):
                bm.free_sequence(sid)
                live.remove(sid)
        B = int(rng.integers(1, len(live) + 1))                 # a varying subset runs this step
        ids = [live[int(j)] for j in rng.permutation(len(live))[:B]]
        tables, positions, pairs = bm.append_batch(ids, W)
        max_ctx = int(positions.max()) + 1
        q = draw(rng, dtype, (B, H_q, D))
        kn, vn = draw(rng, dtype, (B, H_kv, D)), draw(rng, dtype, (B, H_kv, D))

        # graph side: write the rows, pad, replay
        q_buf[:B].copy_(to_tensor(q, dtype, "cuda"))
        kn_buf[:B].copy_(to_tensor(kn, dtype, "cuda"))
        vn_buf[:B].copy_(to_tensor(vn, dtype, "cuda"))
        bt_buf.fill_(-1)
        bt_buf[:B].copy_(t.from_numpy(tables).cuda())
        pos_buf.fill_(-1)
        pos_buf[:B].copy_(t.from_numpy(positions).cuda())
        if cow:
            cs.fill_(-1)
            cd.fill_(-1)
            if len(pairs):
                cs[:len(pairs)].copy_(t.from_numpy(np.ascontiguousarray(pairs[:, 0])).cuda())
                cd[:len(pairs)].copy_(t.from_numpy(np.ascontiguousarray(pairs[:, 1])).cuda())
        else:
            assert len(pairs) == 0
        out_buf.fill_(7.0)
        graphs.launch(B, max_ctx, len(pairs))
        Bc = next(c for c in bcaps if c >= B)
        used.add((Bc, next(c for c in ccaps if c >= max_ctx)))
        replays += 1

        # unrelated eager GPU work between replays
        x = t.randn((256, 256), device="cuda")
        _ = (x @ x).sum().item()

        # eager side
        if len(pairs):
            pkv.copy_blocks(ke, ve, t.from_numpy(np.ascontiguousarray(pairs[:, 0])).cuda(),
                            t.from_numpy(np.ascontiguousarray(pairs[:, 1])).cuda())
        eager = pkv.append_decode_attention(
            to_tensor(q, dtype, "cuda"), to_tensor(kn, dtype, "cuda"), to_tensor(vn, dtype, "cuda"), ke, ve,
            t.from_numpy(tables).cuda(), t.from_numpy(positions).cuda(), scale, max_ctx, partition_size=P)

        # oracle
        oracle_copy_blocks(kp, vp, [tuple(int(x) for x in p) for p in pairs])
        oracle.kv_append(dtype, kn, vn, kp, vp, np.ascontiguousarray(tables), positions, BS)
        ref = oracle.paged_decode_attention(dtype, q, kp, vp, tables, positions + 1, scale)
        t.cuda.synchronize()

        got = out_buf.cpu().numpy().astype(np.float64)
        assert np.all(np.isnan(got[B:Bc])), "padding rows must come out NaN"
        assert np.all(got[Bc:] == 7.0), "rows beyond the bucket's capacity must be untouched"
        ok, e = close(got[:B], ref, dtype)
        assert ok, (step, "graph vs oracle", e)
        ok, e = close(got[:B], eager.cpu().numpy().astype(np.float64), dtype)
        assert ok, (step, "graph vs eager", e)
    assert bits_equal(to_numpy_bits(kg, dtype), kp) and bits_equal(to_numpy_bits(vg, dtype), vp)
    assert bits_equal(to_numpy_bits(ke, dtype), kp) and bits_equal(to_numpy_bits(ve, dtype), vp)
    assert len(used) >= 3, used
    with pytest.raises(pkv.PkvError):
        graphs.launch(Bmax + 1, 10)
    with pytest.raises(pkv.PkvError):
        graphs.launch(1, ccaps[-1] + 1)
    with pytest.raises(pkv.PkvError):
        graphs.launch(2, 10, 3)                          # more copies than the bucket's batch capacity
    if not cow:
        with pytest.raises(pkv.PkvError):
            graphs.launch(1, 10, 1)                      # captured without copy buffers
    graphs.close()
    print(f"  {replays} replays over buckets {sorted(used)}", flush=True)
