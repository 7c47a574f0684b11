"""GPU: the decoder (pkv_decoder_*), one call per decode step, in graph and
eager modes.  Requests arrive, fork and finish through the decoder's own block
manager, mirrored on the oracle's manager; every step's output rows are checked
against the oracle's attention over the oracle's pools, the copy count against
the oracle's copy pairs, and both pools bit for bit at the end."""
import math

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from oracle.block_manager import BlockManager as OracleBM
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


@pytest.mark.parametrize("dtype,H_q,H_kv,D,P,graphs,seed,kv", [
    ("f16", 8, 2, 128, 32, True, 301, "16"),
    ("bf16", 8, 8, 128, 0, True, 302, "16"),
    ("f32", 4, 4, 64, 0, False, 303, "16"),
    ("bf16", 16, 2, 128, 64, False, 304, "16"),
    ("bf16", 8, 2, 128, 32, False, 305, "fp8"),
    ("f16", 4, 4, 64, 0, True, 306, "fp8"),
    ("bf16", 8, 2, 128, 32, True, 307, "mx4"),     # grouped MFMA kernel, split, graphs
    ("f16", 4, 4, 128, 0, False, 308, "mx4"),      # per-head kernel, eager
    ("f32", 4, 2, 64, 64, True, 309, "mx4"),       # per-head kernel (f32 q), split, graphs
    ("bf16", 8, 2, 128, 32, True, 310, "mx4_even"),   # grouped MXFP4 even split (forced), graphs
    ("bf16", 16, 2, 128, 32, True, 311, "16_even"),   # grouped 16-bit even split (forced), graphs
])
def test_decoder_matches_oracle(torch_dev, monkeypatch, dtype, H_q, H_kv, D, P, graphs, seed, kv):
    t = torch_dev
    even = kv.endswith("_even")
    if even:   # the plans' even splits, wherever they fit (graph captures included)
        kv = kv[:-len("_even")]
        monkeypatch.setenv("PKV_MX4_EVEN" if kv == "mx4" else "PKV_GQA_EVEN", "2")
    launches = set()
    fp8, mx4 = kv == "fp8", kv == "mx4"
    print(f"decoder {dtype} H_q={H_q} H_kv={H_kv} D={D} P={P} graphs={graphs} seed={seed} kv={kv}", flush=True)
    rng = np.random.default_rng(seed)
    Bmax, W, n_blocks = 8, 12, 120
    scale = 1.0 / math.sqrt(D)
    tdt = {"f32": t.float32, "f16": t.float16, "bf16": t.bfloat16}[dtype]
    if fp8:
        kp = np.full((n_blocks, H_kv, BS, D), 0x7F, np.uint8)
        ksc = np.full((n_blocks, H_kv, BS), np.nan, np.float32)
        vsc = ksc.copy()
        k, v = t.from_numpy(kp.copy()).cuda(), t.from_numpy(kp.copy()).cuda()
        ks_d, vs_d = t.from_numpy(ksc.copy()).cuda(), t.from_numpy(vsc.copy()).cuda()
    elif mx4:   # unwritten slots: code 7 (6.0) under scale byte 255 (NaN)
        kp = np.full((n_blocks, H_kv, BS, D // 2), 0x77, np.uint8)
        ksc = np.full((n_blocks, H_kv, BS, D // 32), 0xFF, np.uint8)
        vsc = ksc.copy()
        k, v = t.from_numpy(kp.copy()).cuda(), t.from_numpy(kp.copy()).cuda()
        ks_d, vs_d = t.from_numpy(ksc.copy()).cuda(), t.from_numpy(vsc.copy()).cuda()
    else:
        kp = poisoned_pool(dtype, n_blocks, H_kv, D)
        k, v = to_tensor(kp, dtype, "cuda"), to_tensor(kp, dtype, "cuda")
    vp = kp.copy()
    q_buf = t.zeros((Bmax, H_q, D), dtype=tdt, device="cuda")
    kn_buf = t.zeros((Bmax, H_kv, D), dtype=tdt, device="cuda")
    vn_buf = t.zeros((Bmax, H_kv, D), dtype=tdt, device="cuda")
    out_buf = t.zeros((Bmax, H_q, D), dtype=t.float32, device="cuda")
    caps = dict(batch_caps=[2, 4, 8], ctx_caps=[64, 128, W * BS]) if graphs else {}
    if fp8 or mx4:
        caps.update(k_scale=ks_d, v_scale=vs_d)
    dec = pkv.Decoder(q_buf, kn_buf, vn_buf, k, v, out_buf, scale, W, partition_size=P, shuffle_seed=seed, **caps)
    bm, ora = dec.block_manager, OracleBM(n_blocks, BS, seed)
    live, next_id = [], [0]

    def write_prompt(sid, n):
        table = np.asarray(bm.block_table(sid), dtype=np.int32)
        assert list(table) == ora.block_table(sid)
        if n == 0:
            return
        kn, vn = draw(rng, dtype, (n, H_kv, D)), draw(rng, dtype, (n, H_kv, D))
        bt = np.full((n, W), -1, dtype=np.int32)
        bt[:, :table.size] = table
        pos = np.arange(n, dtype=np.int32)
        if fp8:
            oracle.kv_append_fp8(dtype, kn, vn, kp, vp, ksc, vsc, bt, pos, BS)
            pkv.kv_append_fp8(to_tensor(kn, dtype, "cuda"), to_tensor(vn, dtype, "cuda"), k, v, ks_d, vs_d,
                              t.from_numpy(bt).cuda(), t.from_numpy(pos).cuda())
        elif mx4:
            oracle.kv_append_mxfp4(dtype, kn, vn, kp, vp, ksc, vsc, bt, pos, BS)
            pkv.kv_append_mxfp4(to_tensor(kn, dtype, "cuda"), to_tensor(vn, dtype, "cuda"), k, v, ks_d, vs_d,
                                t.from_numpy(bt).cuda(), t.from_numpy(pos).cuda())
        else:
            oracle.kv_append(dtype, kn, vn, kp, vp, bt, pos, BS)
            pkv.kv_append(to_tensor(kn, dtype, "cuda"), to_tensor(vn, dtype, "cuda"), k, v,
                          t.from_numpy(bt).cuda(), t.from_numpy(pos).cuda())

    atol, rtol = TOL[dtype]
    total_copies = 0
    for step in range(40):
        while len(live) < 2 or (rng.random() < 0.3 and len(live) < Bmax):
            sid, next_id[0] = next_id[0], next_id[0] + 1
            n = int(rng.integers(0, 90))
            bm.add_sequence(sid, n)
            ora.add_sequence(sid, n)
            write_prompt(sid, n)
            live.append(sid)
        if rng.random() < 0.4 and len(live) < Bmax:
            sid, next_id[0] = next_id[0], next_id[0] + 1
            parent = live[int(rng.integers(len(live)))]
            bm.fork(parent, sid)
            ora.fork(parent, sid)
            live.append(sid)
        for sid in list(live):
            if bm.sequence_length(sid) >= W * BS - 1 or (len(live) > 2 and rng.random() < 0.07):
                bm.free_sequence(sid)
                ora.free_sequence(sid)
                live.remove(sid)
        B = int(rng.integers(1, len(live) + 1))
        ids = [live[int(j)] for j in rng.permutation(len(live))[:B]]
        q = draw(rng, dtype, (B, H_q, D))
        kn, vn = draw(rng, dtype, (B, H_kv, D)), draw(rng, dtype, (B, H_kv, D))
        q_buf[:B].copy_(to_tensor(q, dtype, "cuda"))
        kn_buf[:B].copy_(to_tensor(kn, dtype, "cuda"))
        vn_buf[:B].copy_(to_tensor(vn, dtype, "cuda"))
        n_copies = dec.step(ids)
        launches.add(pkv.last_launch().split(" ")[0])

        tables, positions, copies = ora.append_batch(ids, W)
        assert n_copies == len(copies)
        total_copies += n_copies
        oracle_copy_blocks(kp, vp, copies)
        tables = np.asarray(tables, dtype=np.int32)
        positions = np.asarray(positions, dtype=np.int32)
        if fp8:
            oracle_copy_blocks(ksc, vsc, copies)
            oracle.kv_append_fp8(dtype, kn, vn, kp, vp, ksc, vsc, tables, positions, BS)
            ref = oracle.paged_decode_attention_fp8(dtype, q, kp, vp, ksc, vsc, tables, positions + 1, scale)
        elif mx4:
            oracle_copy_blocks(ksc, vsc, copies)
            oracle.kv_append_mxfp4(dtype, kn, vn, kp, vp, ksc, vsc, tables, positions, BS)
            ref = oracle.paged_decode_attention_mxfp4(dtype, q, kp, vp, ksc, vsc, tables, positions + 1, scale)
        else:
            oracle.kv_append(dtype, kn, vn, kp, vp, tables, positions, BS)
            ref = oracle.paged_decode_attention(dtype, q, kp, vp, tables, positions + 1, scale)
        t.cuda.synchronize()
        got = out_buf[:B].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), step
        err = np.abs(got - ref)
        rel = err / np.maximum(np.abs(ref), atol / rtol)
        assert err.max() <= atol and rel.max() <= rtol, (step, float(err.max()), float(rel.max()))
        for sid in ids:
            assert list(bm.block_table(sid)) == ora.block_table(sid)
    assert total_copies > 0, "the stream never exercised copy-on-write"
    if even:
        assert {"mxfp4_mfma_even", "gqa_mfma_even"} & launches, launches
    if fp8 or mx4:
        assert bits_equal(k.cpu().numpy(), kp) and bits_equal(v.cpu().numpy(), vp)
        assert bits_equal(ks_d.cpu().numpy(), ksc) and bits_equal(vs_d.cpu().numpy(), vsc)
    else:
        assert bits_equal(to_numpy_bits(k, dtype), kp) and bits_equal(to_numpy_bits(v, dtype), vp)

    # errors leave the manager as it was and launch nothing
    before = [(s, bm.sequence_length(s)) for s in live]
    with pytest.raises(pkv.PkvError) as e:
        dec.step([live[0], 10 ** 9])
    assert e.value.status == pkv.PKV_ERR_SEQUENCE
    with pytest.raises(pkv.PkvError) as e:
        dec.step(list(range(Bmax + 1)))
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    assert [(s, bm.sequence_length(s)) for s in live] == before
    dec.close()
    print(f"  {total_copies} copy-on-write copies", flush=True)
