"""GPU parity with K/V pools larger than 4 GiB.

Every kernel forms a block's address as block id x block bytes in 64-bit
arithmetic; these cases place every block a request uses above byte offset
2^32 of its pool, so an offset truncated to 32 bits would read the poisoned
blocks below it and show up as a non-finite or wrong output.  A small
seeded workload is drawn and checked against the oracle as usual; on the GPU
its pools are copied into the top of pools of more than 4 GiB whose lower
blocks hold poison (NaN elements, E4M3 NaN codes with NaN scales, or E8M0 NaN
scale bytes), and its block table is shifted by the same number of blocks
(the result does not depend on where a block lies: "从 PagedAttention 到
Prefill-Decode 分离的深度解析", section 2.2).  The fused step (append + attention),
attention alone over the appended pools, and copy_blocks are checked; the
appended pools must match the oracle's bit for bit and the poison must be
untouched."""
import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from workloads import get_config, make_workload
from workloads.device import to_numpy_bits, to_tensor

pytestmark = pytest.mark.gpu

TOL = {"f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
LENS = (17, 700, 2100)
TWO32 = 1 << 32

# (kv format, q dtype, H_q, H_kv, partition size, expected launch prefix)
CASES = [
    ("16", "f16", 8, 8, 0, "mha "),
    ("16", "bf16", 64, 8, 1024, "gqa_mfma"),
    ("fp8", "f16", 8, 8, 0, "fp8 "),
    ("fp8", "bf16", 64, 8, 1024, "gqa_mfma_fp8"),
    ("mx4", "f16", 8, 8, 0, "mxfp4 "),
    ("mx4", "bf16", 64, 8, 1024, "mxfp4_mfma "),
    ("mx4_even", "bf16", 64, 8, 1024, "mxfp4_mfma_even "),   # the grouped MXFP4 kernel's even split, forced
]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def assert_close(got, ref, dtype, what):
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    assert err.max() <= atol and rel.max() <= rtol, f"{what}: max_abs={err.max():.3e} max_rel={rel.max():.3e}"


def bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and a.view(np.uint8).tobytes() == b.view(np.uint8).tobytes()


def int_view(torch, t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def big_pool(torch, small, off, extra, poison):
    """Device pool of off + len(small) + extra blocks: poison everywhere, then `small` at [off, off + n)."""
    n = small.shape[0]
    t = torch.empty((off + n + extra,) + tuple(small.shape[1:]), dtype=small.dtype, device="cuda")
    int_view(torch, t).fill_(poison)
    t[off:off + n].copy_(small.to("cuda"))
    return t


def poison_intact(torch, t, lo, hi, poison):
    return bool((int_view(torch, t[lo:hi]) == poison).all().item())


@pytest.mark.parametrize("kv,dtype,H_q,H_kv,P,prefix", CASES)
def test_pool_above_4gib(torch_dev, monkeypatch, kv, dtype, H_q, H_kv, P, prefix):
    torch = torch_dev
    D = 128
    if kv == "mx4_even":
        monkeypatch.setenv("PKV_MX4_EVEN", "2")
        kv = "mx4"
    base = {"16": "c3", "fp8": "c3f8", "mx4": "c3f4"}[kv]
    cfg = get_config(base, dtype=dtype, D=D, H_q=H_q, H_kv=H_kv, B=len(LENS), lengths=("fixed", LENS),
                     pool=("factor", 1.3), append=True, partition_size=P)
    w = make_workload(cfg, 53)
    ref, pk, pv = oracle.run_step(w)
    n = w.n_blocks

    if kv == "16":
        k_small, v_small = to_tensor(w.k_pool, dtype, "cpu"), to_tensor(w.v_pool, dtype, "cpu")
        nan = {"f16": 0x7E00, "bf16": 0x7FC0}[dtype]
        poisons = [nan, nan]
        smalls = [k_small, v_small]
        refs = [pk, pv]
    else:
        code_nan = 0x7F if kv == "fp8" else 0x77
        scale_nan = 0x7FC00000 if kv == "fp8" else 0xFF
        smalls = [torch.from_numpy(np.ascontiguousarray(a)) for a in (w.k_pool, w.v_pool, w.k_scale, w.v_scale)]
        poisons = [code_nan, code_nan, scale_nan, scale_nan]
        refs = [pk[0], pv[0], pk[1], pv[1]]
    blk_bytes = smalls[0][0].numel() * smalls[0].element_size()
    off = -(-(TWO32 + (1 << 20)) // blk_bytes)      # first used block starts past byte 2^32 (+1 MiB)
    assert off * blk_bytes > TWO32
    extra = 2                                       # room for copy_blocks targets past the workload's blocks
    big = [big_pool(torch, s, off, extra, p) for s, p in zip(smalls, poisons)]
    bt = np.where(w.block_tables >= 0, w.block_tables + off, -1).astype(np.int32)
    q = to_tensor(w.q, dtype, "cuda")
    k_new, v_new = to_tensor(w.k_new, dtype, "cuda"), to_tensor(w.v_new, dtype, "cuda")
    btd = torch.from_numpy(bt).cuda()
    pos = torch.from_numpy(w.positions).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    maxc = w.max_context_len
    scale = float(w.scale)

    if kv == "16":
        step = lambda: pkv.append_decode_attention(q, k_new, v_new, big[0], big[1], btd, pos, scale, maxc,
                                                   partition_size=P)
        attend = lambda: pkv.paged_decode_attention(q, big[0], big[1], btd, ctx, scale, maxc, partition_size=P)
    elif kv == "fp8":
        step = lambda: pkv.append_decode_attention_fp8(q, k_new, v_new, *big, btd, pos, scale, maxc,
                                                       partition_size=P)
        attend = lambda: pkv.paged_decode_attention_fp8(q, *big, btd, ctx, scale, maxc, partition_size=P)
    else:
        step = lambda: pkv.append_decode_attention_mxfp4(q, k_new, v_new, *big, btd, pos, scale, maxc,
                                                         partition_size=P)
        attend = lambda: pkv.paged_decode_attention_mxfp4(q, *big, btd, ctx, scale, maxc, partition_size=P)

    what = f"{kv} {dtype} G{H_q // H_kv} P{P} blocks from {off} ({off * blk_bytes / 2**30:.2f} GiB)"
    out = step()
    torch.cuda.synchronize()
    assert pkv.last_launch().startswith(prefix), pkv.last_launch()
    assert_close(out.cpu().numpy(), ref, dtype, what + " fused step")
    for t, r, p in zip(big, refs, poisons):
        got = t[off:off + n].cpu()
        got = to_numpy_bits(got, dtype) if kv == "16" else got.numpy()
        assert bits_equal(got, r), what + ": appended pool differs from the oracle's"
        assert poison_intact(torch, t, 0, off, p) and poison_intact(torch, t, off + n, off + n + extra, p), \
            what + ": a block outside the request's blocks was written"

    out2 = attend()
    torch.cuda.synchronize()
    assert_close(out2.cpu().numpy(), ref, dtype, what + " attention after the append")

    # copy two used blocks to the spare blocks at the very top of the pools
    src = torch.tensor([int(bt[1, 0]), int(bt[2, 3])], dtype=torch.int32, device="cuda")
    dst = torch.tensor([off + n, off + n + 1], dtype=torch.int32, device="cuda")
    if kv == "16":
        pkv.copy_blocks(big[0], big[1], src, dst)
    elif kv == "fp8":
        pkv.copy_blocks_fp8(*big, src, dst)
    else:
        pkv.copy_blocks_mxfp4(*big, src, dst)
    torch.cuda.synchronize()
    for t in big:
        assert torch.equal(t[off + n:off + n + 2].view(torch.uint8), t[src.long()].view(torch.uint8)), \
            what + ": copy_blocks"
    del big
    torch.cuda.empty_cache()
