"""CPU: the even split's work assignment, modelled step by step as the grouped kernel and
its merge perform it, on random batches (no GPU).

The batch's blocks, requests end to end, are cut into `runs` equal runs of tw blocks;
workgroup (S, g) streams super-run S (runs S nw .. S nw + nw - 1) for KV head g, a wave
per run; a wave writes a piece that is a whole request as the output and keeps its run's
cut first and last pieces, which the workgroup merges in token order into one piece per
(super-run, request) -- the output when they cover the request -- with id (S + b) H_kv + g.
The merge kernel takes super-runs r0 .. r1 of a request's blocks.  Checked: every
(request, KV head, block) is streamed exactly once; a kept last piece ends its run; each
request gets either one output or its super-runs' pieces, exactly the ids the merge
kernel reads; piece rows and the prefix fit the workspace that pkv_decode_workspace_bytes
sizes for the caller's partition.  The plan's sizing (runs, the workspace cap) is the
library's, restated.

The grouped MXFP4 kernel's even split is modelled the same way (plan_mx4, model_mx4): one run per
workgroup, streamed for nw KV heads at once (a wave per head), its pieces written straight to the
workspace with the run as the merge kernel's super-run.
"""
import random

import pytest

import paged_kv_decode_blocks_amd as pkv

MAX_BATCH, MAX_RUN, MIN_RUN = 1024, 256, 16


def plan(B, H_q, H_kv, D, max_ctx, P, resident_waves, nw):
    """Runs and grid of the even split for a call, or None when the plan cannot take it
    (the host's sizing; the performance gate is not modelled: the tests force the split)."""
    padded = -(-max_ctx // 16) * 16
    n_parts = -(-max_ctx // P) if 0 < P < padded else 1
    if n_parts <= 1 or B > MAX_BATCH:
        return None
    worst = B * -(-max_ctx // 16)                                # blocks per KV head
    cap = ((B * H_q * n_parts - B - 3) // H_q - B) * nw        # runs whose pieces fit
    need = -(-worst // MAX_RUN)
    resident = resident_waves // H_kv
    runs = min(max(resident, need), cap)
    if not (resident > 0 and runs >= need and runs >= 1):
        return None
    return {"even_waves": runs * H_kv, "grid": -(-runs // nw) * H_kv}


def model(B, H_q, H_kv, D, max_ctx, P, lens, fused, nw, resident_waves):
    pl = plan(B, H_q, H_kv, D, max_ctx, P, resident_waves, nw)
    if pl is None:
        return None
    G = H_q // H_kv
    ws_floats = pkv.decode_workspace_bytes(B, H_q, D, max_ctx, P) // 4
    nb = [0 if ((n < 1 or n > max_ctx) if fused else (n < 0 or n > max_ctx)) else -(-n // 16) for n in lens]
    pre = [0]
    for x in nb:
        pre.append(pre[-1] + x)
    total = pre[B]
    runs = max(1, min(pl["even_waves"] // H_kv, -(-total // MIN_RUN)))
    tw = max(1, -(-total // runs))
    assert tw <= MAX_RUN
    streamed, written, n_pieces = set(), {}, 0
    for wg in range(pl["grid"]):
        S, g = divmod(wg, H_kv)
        kept = []
        for w in range(nw):
            run = S * nw + w
            x0 = run0 = run * tw
            x1 = min(run0 + tw, total)
            if run >= runs or x0 >= x1:
                continue
            b = max(i for i in range(B) if pre[i] <= x0)          # the kernel's binary search
            while x0 < x1:
                seg0, nbb = pre[b], pre[b + 1] - pre[b]
                pend = min(x1, seg0 + nbb)
                blk0, np_ = x0 - seg0, pend - x0
                assert 1 <= np_ <= MAX_RUN
                for k in range(blk0, blk0 + np_):
                    assert (b, g, k) not in streamed
                    streamed.add((b, g, k))
                if blk0 == 0 and np_ == nbb:
                    written.setdefault((b, g), []).append(None)
                else:
                    slot = 0 if x0 == run0 else 1
                    assert slot == 0 or pend == x1                # a kept last piece ends the run
                    kept.append((w, slot, b, blk0 == 0, blk0 + np_ == nbb))
                x0 = pend
                if x0 < x1:
                    b += 1
                    while pre[b + 1] == pre[b]:
                        b += 1
        assert len({(w, k) for w, k, *_ in kept}) == len(kept)      # one piece per slot
        groups = []
        for w, k, b, starts, ends in sorted(kept):
            if groups and groups[-1][0] == b:
                groups[-1][2] = ends
            else:
                groups.append([b, starts, ends])
        for b, starts, ends in groups:
            if starts and ends:
                written.setdefault((b, g), []).append(None)
            else:
                pid = (S + b) * H_kv + g
                # piece rows after the prefix (B + 3 ints) in the lse area, G rows each in the o area
                assert (pid + 1) * G * D <= ws_floats
                assert B + 3 + (pid + 1) * G <= ws_floats
                written.setdefault((b, g), []).append((S, pid))
                n_pieces += 1
    ts = nw * tw                                                     # the merge kernel's view
    for b in range(B):
        if nb[b] == 0:
            continue
        r0, r1 = pre[b] // ts, (pre[b] + nb[b] - 1) // ts
        for g in range(H_kv):
            assert all((b, g, k) in streamed for k in range(nb[b]))
            got = written[(b, g)]
            if r0 == r1:
                assert got == [None], (b, g, got)
            else:
                assert sorted(got) == [(r, (r + b) * H_kv + g) for r in range(r0, r1 + 1)], (b, g, got)
    assert len(streamed) == total * H_kv
    return runs, tw, n_pieces


def test_c5_shaped_batch():
    rng = random.Random(5)
    lens = [rng.randint(4096, 16384) for _ in range(32)]
    runs, tw, n_pieces = model(32, 64, 8, 128, 16384, 1024, lens, True, 4, 2048)
    assert runs == 256 and n_pieces < 3 * 256               # ~3 pieces per (request, KV head)


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = random.Random(seed)
    done = 0
    for _ in range(60):
        H_kv = rng.choice([1, 2, 4, 8])
        G = rng.choice([2, 4, 8, 16])
        B = rng.choice([1, 2, 3, 7, 32, 100, rng.randint(1, 1100)])
        max_ctx = rng.choice([1, 16, 17, 100, 512, 2048, 5000])
        P = rng.choice([16, 32, 256, 1024])
        fused = rng.random() < 0.5
        lens = []
        for _ in range(B):
            r = rng.random()
            lens.append(0 if r < 0.05 else max_ctx + 1 if r < 0.08 else -3 if r < 0.1 else rng.randint(1, max_ctx))
        res = model(B, G * H_kv, H_kv, rng.choice([64, 128]), max_ctx, P, lens, fused,
                    rng.choice([2, 4, 8]), rng.choice([2048, 64, 8]))
        done += res is not None
    assert done >= 15


# The grouped MXFP4 kernel's even split: one run per workgroup, streamed for nw KV heads at
# once (a wave per head), so a run's pieces go straight to the workspace (no in-workgroup
# merge) and the merge kernel's super-run is the run itself.

def plan_mx4(B, H_q, H_kv, max_ctx, P, resident_wgs, nw):
    """Runs and grid of the MXFP4 even split, or None when the plan cannot take it (the
    host's sizing; the performance gate is not modelled)."""
    padded = -(-max_ctx // 16) * 16
    n_parts = -(-max_ctx // P) if 0 < P < padded else 1
    if n_parts <= 1 or B < 1 or B > MAX_BATCH or H_kv % nw:
        return None
    worst = B * -(-max_ctx // 16)
    cap = (B * H_q * n_parts - B - 3) // H_q - B
    need = -(-worst // MAX_RUN)
    resident = resident_wgs // (H_kv // nw)
    runs = min(max(resident, need), cap)
    if not (resident > 0 and runs >= need and runs >= 1):
        return None
    return {"even_waves": runs * H_kv, "grid": runs * (H_kv // nw)}


def model_mx4(B, H_q, H_kv, D, max_ctx, P, lens, fused, nw, resident_wgs):
    pl = plan_mx4(B, H_q, H_kv, max_ctx, P, resident_wgs, nw)
    if pl is None:
        return None
    G = H_q // H_kv
    ws_floats = pkv.decode_workspace_bytes(B, H_q, D, max_ctx, P) // 4
    nb = [0 if ((n < 1 or n > max_ctx) if fused else (n < 0 or n > max_ctx)) else -(-n // 16) for n in lens]
    pre = [0]
    for x in nb:
        pre.append(pre[-1] + x)
    total = pre[B]
    runs = max(1, min(pl["even_waves"] // H_kv, -(-total // MIN_RUN)))
    tw = max(1, -(-total // runs))
    assert tw <= MAX_RUN
    streamed, written = set(), {}
    for wg in range(pl["grid"]):
        S, hgi = divmod(wg, H_kv // nw)
        x0 = S * tw
        x1 = min(x0 + tw, total)
        if S >= runs or x0 >= x1:
            continue
        b = max(i for i in range(B) if pre[i] <= x0)
        while x0 < x1:
            seg0, nbb = pre[b], pre[b + 1] - pre[b]
            pend = min(x1, seg0 + nbb)
            blk0, np_ = x0 - seg0, pend - x0
            assert 1 <= np_ <= MAX_RUN                     # the piece's ids fit the window
            for g in range(hgi * nw, hgi * nw + nw):
                for k in range(blk0, blk0 + np_):
                    assert (b, g, k) not in streamed
                    streamed.add((b, g, k))
                if blk0 == 0 and np_ == nbb:
                    written.setdefault((b, g), []).append(None)
                else:
                    pid = (S + b) * H_kv + g
                    assert (pid + 1) * G * D <= ws_floats
                    assert B + 3 + (pid + 1) * G <= ws_floats
                    written.setdefault((b, g), []).append((S, pid))
            x0 = pend
            if x0 < x1:
                b += 1
                while pre[b + 1] == pre[b]:
                    b += 1
    for b in range(B):                                     # the merge kernel's view: super-run = run
        if nb[b] == 0:
            continue
        r0, r1 = pre[b] // tw, (pre[b] + nb[b] - 1) // tw
        for g in range(H_kv):
            got = written[(b, g)]
            if r0 == r1:
                assert got == [None], (b, g, got)
            else:
                assert sorted(got) == [(r, (r + b) * H_kv + g) for r in range(r0, r1 + 1)], (b, g, got)
    assert len(streamed) == total * H_kv
    return runs, tw


def test_mx4_c5_shaped_batch():
    rng = random.Random(7)
    lens = [rng.randint(4096, 16384) for _ in range(32)]
    runs, tw = model_mx4(32, 64, 8, 128, 16384, 1024, lens, True, 8, 256)
    assert runs == 256 and tw == -(-sum(-(-n // 16) for n in lens) // 256)


@pytest.mark.parametrize("seed", range(6))
def test_mx4_random_batches(seed):
    rng = random.Random(100 + seed)
    done = 0
    for _ in range(60):
        nw = rng.choice([2, 4, 8])
        H_kv = nw * rng.choice([1, 2, 3])
        G = rng.choice([1, 2, 4, 8, 16])
        B = rng.choice([1, 2, 3, 7, 32, 100, rng.randint(1, 1100)])
        max_ctx = rng.choice([1, 16, 17, 100, 512, 2048, 5000])
        P = rng.choice([16, 32, 256, 1024])
        fused = rng.random() < 0.5
        lens = []
        for _ in range(B):
            r = rng.random()
            lens.append(0 if r < 0.05 else max_ctx + 1 if r < 0.08 else -3 if r < 0.1 else rng.randint(1, max_ctx))
        res = model_mx4(B, G * H_kv, H_kv, rng.choice([64, 128]), max_ctx, P, lens, fused, nw,
                        rng.choice([512, 256, 64, 3]))
        done += res is not None
    assert done >= 15
