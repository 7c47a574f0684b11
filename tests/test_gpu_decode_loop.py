"""GPU: the paging lifecycle end to end.  The library's host block manager
drives many decode steps -- requests arrive (some sharing a prompt prefix),
fork, grow, and finish -- and each step runs copy_blocks (copy-on-write) and
the fused append + attention on the GPU.  The oracle runs the same stream with
its own block manager, its own pools and its own attention: block tables,
positions and copy pairs must match exactly, attention outputs to the f16/bf16
(or f32) tolerance, and both pools bit for bit at the end.

Also copy_blocks alone against a numpy copy, bit for bit."""
import math

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from oracle.block_manager import BlockManager as OracleBM
from oracle.block_manager import BlockManagerError
from oracle.block_manager import copy_blocks as oracle_copy_blocks
from workloads import to_storage
from workloads.device import to_numpy_bits, to_tensor

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
BS = 16


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and a.view(np.uint8).tobytes() == b.view(np.uint8).tobytes()


def poisoned_pool(dtype, n_blocks, H_kv, D):
    return to_storage(np.full((n_blocks, H_kv, BS, D), np.nan, dtype=np.float32), dtype)


def draw(rng, dtype, shape, std=1.0):
    return to_storage(rng.standard_normal(shape).astype(np.float32) * std, dtype)


class Loop:
    """The library's side (device pools + pkv.BlockManager) and the oracle's side
    (host pools + oracle BlockManager), fed the same requests."""

    def __init__(self, torch, dtype, n_blocks, H_q, H_kv, D, W, seed):
        self.t, self.dtype, self.H_q, self.H_kv, self.D, self.W = torch, dtype, H_q, H_kv, D, W
        self.rng = np.random.default_rng(seed)
        self.lib = pkv.BlockManager(n_blocks, BS, shuffle_seed=seed)
        self.ora = OracleBM(n_blocks, BS, seed)
        self.kp = poisoned_pool(dtype, n_blocks, H_kv, D)
        self.vp = self.kp.copy()
        self.k = to_tensor(self.kp, dtype, "cuda")
        self.v = to_tensor(self.vp, dtype, "cuda")
        self.live = []
        self.next_id = 0
        self.copies = 0
        self.shared_tokens = 0

    def both(self, name, *args):
        """Call a block-manager method on both sides; they must agree on success and on the error kind."""
        kinds = {pkv.PKV_ERR_OUT_OF_BLOCKS: "out_of_blocks", pkv.PKV_ERR_SEQUENCE: "sequence",
                 pkv.PKV_ERR_INVALID_ARG: "invalid"}
        res = []
        for side in (self.lib, self.ora):
            try:
                res.append(("ok", getattr(side, name)(*args)))
            except BlockManagerError as e:
                res.append(("err", e.kind))
            except pkv.PkvError as e:
                res.append(("err", kinds.get(e.status, e.status)))
        assert res[0][0] == res[1][0], (name, args, res)
        if res[0][0] == "err":
            assert res[0][1] == res[1][1], (name, args, res)
            return None
        return res

    def write_prompt(self, sid, start, n):
        """Write tokens start..n-1 of a new sequence (prefill is not part of this
        library: the test writes them with kv_append, one row per token)."""
        if n <= start:
            return
        m = n - start
        kn = draw(self.rng, self.dtype, (m, self.H_kv, self.D))
        vn = draw(self.rng, self.dtype, (m, self.H_kv, self.D))
        table = np.asarray(self.lib.block_table(sid), dtype=np.int32)
        assert list(table) == self.ora.block_table(sid)
        bt = np.full((m, self.W), -1, dtype=np.int32)
        bt[:, :table.size] = table
        pos = np.arange(start, n, dtype=np.int32)
        oracle.kv_append(self.dtype, kn, vn, self.kp, self.vp, bt, pos, BS)
        t = self.t
        pkv.kv_append(to_tensor(kn, self.dtype, "cuda"), to_tensor(vn, self.dtype, "cuda"), self.k, self.v,
                      t.from_numpy(bt).cuda(), t.from_numpy(pos).cuda())

    def add(self, n):
        sid = self.next_id
        self.next_id += 1
        if self.both("add_sequence", sid, n) is not None:
            self.live.append(sid)
            self.write_prompt(sid, 0, n)

    def add_shared(self, prefix, pt, n):
        sid = self.next_id
        self.next_id += 1
        r = self.both("add_sequence_shared", sid, n, prefix, pt)
        if r is not None:
            assert r[0][1] == r[1][1]
            shared = r[0][1]
            self.shared_tokens += shared
            self.live.append(sid)
            # tokens pt..n-1 are new; shared..pt-1 repeat the prefix's tokens: copy their bits
            if pt > shared:
                ptable = self.ora.block_table(prefix)
                rows = [(ptable[p // BS], p % BS) for p in range(shared, pt)]
                kn = np.stack([self.kp[b, :, s, :] for b, s in rows])
                vn = np.stack([self.vp[b, :, s, :] for b, s in rows])
                table = np.asarray(self.lib.block_table(sid), dtype=np.int32)
                bt = np.full((len(rows), self.W), -1, dtype=np.int32)
                bt[:, :table.size] = table
                pos = np.arange(shared, pt, dtype=np.int32)
                oracle.kv_append(self.dtype, kn, vn, self.kp, self.vp, bt, pos, BS)
                t = self.t
                pkv.kv_append(to_tensor(kn, self.dtype, "cuda"), to_tensor(vn, self.dtype, "cuda"), self.k,
                              self.v, t.from_numpy(bt).cuda(), t.from_numpy(pos).cuda())
            self.write_prompt(sid, max(pt, shared), n)

    def fork(self, parent):
        sid = self.next_id
        self.next_id += 1
        if self.both("fork", parent, sid) is not None:
            self.live.append(sid)

    def free(self, sid):
        assert self.both("free_sequence", sid) is not None
        self.live.remove(sid)

    def step(self, partition_size):
        """One decode step for every live sequence; returns the worst errors."""
        t, d = self.t, self.dtype
        ids = list(self.live)
        r = self.both("append_batch", ids, self.W)
        if r is None:
            return None
        (tables, positions, cow), (o_tables, o_positions, o_cow) = r[0][1], r[1][1]
        assert tables.tolist() == o_tables and positions.tolist() == o_positions
        assert [tuple(x) for x in cow.tolist()] == o_cow
        B = len(ids)
        q = draw(self.rng, d, (B, self.H_q, self.D))
        kn = draw(self.rng, d, (B, self.H_kv, self.D))
        vn = draw(self.rng, d, (B, self.H_kv, self.D))
        # oracle
        oracle_copy_blocks(self.kp, self.vp, o_cow)
        bt_o = np.ascontiguousarray(np.asarray(o_tables, dtype=np.int32))
        pos_o = np.asarray(o_positions, dtype=np.int32)
        oracle.kv_append(d, kn, vn, self.kp, self.vp, bt_o, pos_o, BS)
        scale = 1.0 / math.sqrt(self.D)
        ref = oracle.paged_decode_attention(d, q, self.kp, self.vp, bt_o, pos_o + 1, scale)
        # library
        if len(cow):
            pkv.copy_blocks(self.k, self.v, t.from_numpy(np.ascontiguousarray(cow[:, 0])).cuda(),
                            t.from_numpy(np.ascontiguousarray(cow[:, 1])).cuda())
            self.copies += len(cow)
        out = pkv.append_decode_attention(
            to_tensor(q, d, "cuda"), to_tensor(kn, d, "cuda"), to_tensor(vn, d, "cuda"), self.k, self.v,
            t.from_numpy(tables).cuda(), t.from_numpy(positions).cuda(), scale, int(positions.max()) + 1,
            partition_size=partition_size)
        t.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        atol, rtol = TOL[d]
        assert np.all(np.isfinite(got))
        err = np.abs(got - ref)
        rel = err / np.maximum(np.abs(ref), atol / rtol)
        return float(err.max()), float(rel.max())


@pytest.mark.parametrize("dtype,H_q,H_kv,D,P,seed", [
    ("f16", 8, 2, 128, 0, 101),
    ("bf16", 16, 2, 128, 32, 102),
    ("f32", 4, 4, 64, 0, 103),
    ("f16", 4, 4, 64, 48, 104),
])
def test_decode_loop_matches_oracle(torch_dev, dtype, H_q, H_kv, D, P, seed):
    print(f"decode loop {dtype} H_q={H_q} H_kv={H_kv} D={D} P={P} seed={seed}", flush=True)
    W, n_blocks, steps = 12, 72, 48
    loop = Loop(torch_dev, dtype, n_blocks, H_q, H_kv, D, W, seed)
    rng = np.random.default_rng(seed + 1)
    atol, rtol = TOL[dtype]
    worst = (0.0, 0.0)
    for s in range(steps):
        # requests come and go between steps (the continuous-batching pattern)
        if len(loop.live) < 3 or (rng.random() < 0.3 and len(loop.live) < 8):
            loop.add(int(rng.integers(0, 70)))
        if loop.live and rng.random() < 0.25 and len(loop.live) < 8:
            prefix = loop.live[int(rng.integers(len(loop.live)))]
            plen = loop.lib.sequence_length(prefix)
            pt = int(rng.integers(0, plen + 1))
            loop.add_shared(prefix, pt, min(pt + int(rng.integers(0, 20)), W * BS - 2))
        if loop.live and rng.random() < 0.3 and len(loop.live) < 8:
            loop.fork(loop.live[int(rng.integers(len(loop.live)))])
        for sid in list(loop.live):                     # finished, or about to outgrow the table
            if loop.lib.sequence_length(sid) >= W * BS - 1 or rng.random() < 0.06:
                loop.free(sid)
        if not loop.live:
            continue
        r = loop.step(P)
        while r is None:                                # pool exhausted on both sides: finish the longest
            longest = max(loop.live, key=loop.lib.sequence_length)
            loop.free(longest)
            if not loop.live:
                break
            r = loop.step(P)
        if r is not None:
            assert r[0] <= atol and r[1] <= rtol, (s, r)
            worst = (max(worst[0], r[0]), max(worst[1], r[1]))
    assert loop.copies > 0, "the stream never exercised copy-on-write"
    assert bits_equal(to_numpy_bits(loop.k, dtype), loop.kp)
    assert bits_equal(to_numpy_bits(loop.v, dtype), loop.vp)
    print(f"  worst abs {worst[0]:.2e} rel {worst[1]:.2e}, {loop.copies} block copies, "
          f"{loop.shared_tokens} shared prompt tokens", flush=True)


@pytest.mark.parametrize("dtype,H_kv,D", [("bf16", 8, 128), ("f16", 2, 64), ("f32", 4, 128), ("f32", 1, 64)])
def test_copy_blocks_bit_exact(torch_dev, dtype, H_kv, D):
    t = torch_dev
    rng = np.random.default_rng(7)
    n_blocks = 40
    kp = draw(rng, dtype, (n_blocks, H_kv, BS, D))
    vp = draw(rng, dtype, (n_blocks, H_kv, BS, D))
    perm = rng.permutation(n_blocks)
    src, dst = perm[:12].astype(np.int32), perm[12:24].astype(np.int32)
    src[3], dst[5] = -1, n_blocks          # out-of-range pairs are skipped
    k, v = to_tensor(kp, dtype, "cuda"), to_tensor(vp, dtype, "cuda")
    pkv.copy_blocks(k, v, t.from_numpy(src).cuda(), t.from_numpy(dst).cuda())
    pkv.copy_blocks(k, v, t.zeros(0, dtype=t.int32, device="cuda"), t.zeros(0, dtype=t.int32, device="cuda"))
    t.cuda.synchronize()
    pairs = [(int(a), int(b)) for a, b in zip(src, dst) if 0 <= a < n_blocks and 0 <= b < n_blocks]
    oracle_copy_blocks(kp, vp, pairs)
    assert bits_equal(to_numpy_bits(k, dtype), kp)
    assert bits_equal(to_numpy_bits(v, dtype), vp)


@pytest.mark.parametrize("H_kv,D", [(8, 128), (2, 64), (1, 64)])
def test_copy_blocks_mxfp4_bit_exact(torch_dev, H_kv, D):
    """Code and scale bytes of whole blocks move unchanged; the neighbours of every
    destination block (the scale tiles are only 32 or 64 bytes per head) stay as they were."""
    t = torch_dev
    rng = np.random.default_rng(11)
    n_blocks = 30
    kp = rng.integers(0, 256, (n_blocks, H_kv, BS, D // 2), dtype=np.uint8)
    vp = rng.integers(0, 256, (n_blocks, H_kv, BS, D // 2), dtype=np.uint8)
    ks = rng.integers(0, 256, (n_blocks, H_kv, BS, D // 32), dtype=np.uint8)
    vs = rng.integers(0, 256, (n_blocks, H_kv, BS, D // 32), dtype=np.uint8)
    perm = rng.permutation(n_blocks)
    src, dst = perm[:9].astype(np.int32), perm[9:18].astype(np.int32)
    src[2] = -1
    dst[6] = n_blocks                       # out of range: skipped
    dev = [t.from_numpy(a.copy()).cuda() for a in (kp, vp, ks, vs)]
    pkv.copy_blocks_mxfp4(*dev, t.from_numpy(src).cuda(), t.from_numpy(dst).cuda())
    t.cuda.synchronize()
    pairs = [(int(a), int(b)) for a, b in zip(src, dst) if 0 <= a < n_blocks and 0 <= b < n_blocks]
    oracle_copy_blocks(kp, vp, pairs)
    oracle_copy_blocks(ks, vs, pairs)
    for d, r in zip(dev, (kp, vp, ks, vs)):
        assert bits_equal(d.cpu().numpy(), r)


@pytest.mark.parametrize("H_kv,D", [(8, 128), (2, 64)])
def test_copy_blocks_fp8_bit_exact(torch_dev, H_kv, D):
    t = torch_dev
    rng = np.random.default_rng(9)
    n_blocks = 30
    kp = rng.integers(0, 256, (n_blocks, H_kv, BS, D), dtype=np.uint8)
    vp = rng.integers(0, 256, (n_blocks, H_kv, BS, D), dtype=np.uint8)
    ks = rng.standard_normal((n_blocks, H_kv, BS)).astype(np.float32)
    vs = rng.standard_normal((n_blocks, H_kv, BS)).astype(np.float32)
    perm = rng.permutation(n_blocks)
    src, dst = perm[:9].astype(np.int32), perm[9:18].astype(np.int32)
    src[2] = -1
    dev = [t.from_numpy(a.copy()).cuda() for a in (kp, vp, ks, vs)]
    pkv.copy_blocks_fp8(*dev, t.from_numpy(src).cuda(), t.from_numpy(dst).cuda())
    t.cuda.synchronize()
    pairs = [(int(a), int(b)) for a, b in zip(src, dst) if a >= 0]
    oracle_copy_blocks(kp, vp, pairs)
    oracle_copy_blocks(ks, vs, pairs)
    for d, r in zip(dev, (kp, vp, ks, vs)):
        assert bits_equal(d.cpu().numpy(), r)
