"""GPU parity on inputs that drive the online softmax's rescaling, for every kernel family.

Everywhere else the inputs give scores about N(0, 1), so after a pass's first
chunk the running maximum of a head's scores hardly ever grows by much.  The
grouped kernels (16-bit, FP8, MXFP4) and the per-head MXFP4 kernel move their
reference maximum lazily: only when some head's chunk maximum exceeds it by
more than 8 binary orders, and then they scale the weights and sums already
accumulated down by 2^(m_old - m_new).  That branch runs with live accumulators
only on inputs like these:

* climbing scores (``workloads.make_peaked_workload``): for half of the query
  heads a sawtooth that rises 64 binary orders (48 for f32 q, whose tolerance
  leaves less room for float32 rounding of larger scores) over every 512 tokens;
  each case checks from its own inputs that a wave's lazily moved maximum jumps
  by more than 8 orders at least twice inside every 512-token partition of the
  longest request, for the chunk and wave counts the grouped kernels use;
* a token that dominates by about 2^96: first in its context (the first chunk
  sets the maximum, nothing later moves it) or last (with the fused append, the
  appended token: the last chunk outweighs the whole history);
* huge logits: q ~ N(0, 30^2) with scale 1, scores in the hundreds, whose
  softmax is the row of the largest score; outputs are checked against the
  oracle and, where the two largest scores are far apart, against that V row.

Outputs must satisfy max|g - r| <= atol and max |g - r| / max(|r|, atol/rtol) <= rtol
against the fp64 oracle, (1e-5, 1e-5) for f32 q and (2e-3, 1e-2) otherwise; after
a fused step the pools (codes and scales) must equal the oracle's bit for bit.
"""
import copy
import math
from dataclasses import replace

import numpy as np
import pytest

import oracle
import paged_kv_decode_blocks_amd as pkv
from tests.test_gpu_decode_loop import bits_equal
from tests.test_gpu_fp8 import GQA8_VARIANTS
from tests.test_gpu_mxfp4 import MX4_VARIANTS, mx4_variant_env
from tests.test_gpu_parity import GQA_VARIANTS, MHA_VARIANTS
from workloads import get_config, make_peaked_workload, make_workload
from workloads.device import to_numpy_bits, upload

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
LOG2E = 1.4426950408889634
LENS = (1, 40, 700, 1500, 2600)        # request 2: dominant first token; 3: dominant last; 4: pure climb
H_KV = 2

# (id, K/V storage, q dtype, G, environment, launch-string prefix)
FAMILIES = [
    ("mha_f32", "", "f32", 1, {}, "mha "),
    ("mha_f16", "", "f16", 1, {}, "mha "),
    ("mha_bf16", "", "bf16", 1, {}, "mha "),
    ("mha_f32_grouped", "", "f32", 8, {}, "mha "),
    ("gqa_regs_bf16", "", "bf16", 8, {"PKV_GQA_KIND": "0"}, "gqa_mfma "),
    ("gqa_lds_f16", "", "f16", 8, {"PKV_GQA_KIND": "1", "PKV_GQA_PF": "2"}, "gqa_mfma_lds "),
    ("gqa_kdma_bf16", "", "bf16", 8, {"PKV_GQA_EVEN": "0"}, "gqa_mfma_kdma "),
    ("gqa_kdma_f16", "", "f16", 8, {"PKV_GQA_EVEN": "0"}, "gqa_mfma_kdma "),
    ("gqa_even_bf16", "", "bf16", 8, {"PKV_GQA_EVEN": "2"}, "gqa_mfma_even "),
    ("gqa_even_f16", "", "f16", 8, {"PKV_GQA_EVEN": "2"}, "gqa_mfma_even "),
    ("fp8_f16", "fp8", "f16", 1, {}, "fp8 "),
    ("fp8_f32_grouped", "fp8", "f32", 2, {}, "fp8 "),
    ("fp8_grouped_bf16", "fp8", "bf16", 8, {"PKV_LP_MIN_PART": "0"}, "gqa_mfma_fp8 "),
    ("fp8_grouped_regk_f16", "fp8", "f16", 8, {"PKV_GQA8_KDMA": "0"}, "gqa_mfma_fp8 "),
    ("mxfp4_head_bf16", "mxfp4", "bf16", 1, {}, "mxfp4 "),
    ("mxfp4_head_f32", "mxfp4", "f32", 2, {}, "mxfp4 "),
    ("mxfp4_mfma_bf16", "mxfp4", "bf16", 8, {"PKV_LP_MIN_PART": "0"}, "mxfp4_mfma "),
    ("mxfp4_mfma_f16", "mxfp4", "f16", 8, {"PKV_LP_MIN_PART": "0"}, "mxfp4_mfma "),
    ("mxfp4_mfma_floor_bf16", "mxfp4", "bf16", 8, {}, "mxfp4_mfma "),
    ("mxfp4_even_bf16", "mxfp4", "bf16", 8, {"PKV_MX4_EVEN": "2"}, "mxfp4_mfma_even "),
    ("mxfp4_even_f16", "mxfp4", "f16", 8, {"PKV_MX4_EVEN": "2"}, "mxfp4_mfma_even "),
]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    pkv.load_library()
    return torch


def assert_close(got, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), atol / rtol)
    assert err.max() <= atol and rel.max() <= rtol, f"{what}: max_abs={err.max():.3e} max_rel={rel.max():.3e}"


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def quantized(w, kv):
    """The workload with its history rows quantized into FP8 or MXFP4 pools by the oracle's own
    quantizing append, one call over every written (block, slot): what a cache filled token by
    token holds.  Unwritten slots keep the poison of their format."""
    cfg = replace(w.cfg, kv_dtype=kv)
    bs, H_kv, D = cfg.block_size, cfg.H_kv, cfg.D
    blk, slot = [], []
    for b in range(w.context_lens.size):
        x = np.arange(int(w.history_lens[b]))
        blk.append(w.block_tables[b, x // bs])
        slot.append(x % bs)
    blk = np.concatenate(blk).astype(np.int32)
    slot = np.concatenate(slot).astype(np.int32)
    rows_k = np.ascontiguousarray(w.k_pool[blk, :, slot, :])
    rows_v = np.ascontiguousarray(w.v_pool[blk, :, slot, :])
    if kv == "fp8":
        kc = np.full((w.n_blocks, H_kv, bs, D), 0x7F, np.uint8)
        ks = np.full((w.n_blocks, H_kv, bs), np.nan, np.float32)
        append = oracle.kv_append_fp8
    else:
        kc = np.full((w.n_blocks, H_kv, bs, D // 2), 0x77, np.uint8)
        ks = np.full((w.n_blocks, H_kv, bs, D // 32), 0xFF, np.uint8)
        append = oracle.kv_append_mxfp4
    vc, vs = kc.copy(), ks.copy()
    append(cfg.dtype, rows_k, rows_v, kc, vc, ks, vs, np.ascontiguousarray(blk[:, None]), slot, bs)
    w2 = copy.copy(w)
    w2.cfg = cfg
    w2.k_pool, w2.v_pool, w2.k_scale, w2.v_scale = kc, vc, ks, vs
    return w2


_cache = {}


def climbing(kv, dtype, G, append, lens=LENS):
    """(workload, oracle output, pools after the oracle's step) for climbing scores, cached."""
    key = ("climb", kv, dtype, G, append, lens)
    if key not in _cache:
        cfg = get_config("c2", B=len(lens), H_q=H_KV * G, H_kv=H_KV, D=128, dtype=dtype,
                         lengths=("fixed", lens), pool=("factor", 1.3), append=append)
        w = make_peaked_workload(cfg, 11 + G, rise_log2=48.0 if dtype == "f32" else 64.0,
                                 dominant_first=(2,), dominant_last=(3,))
        if kv:
            w = quantized(w, kv)
        ref, kp, vp = oracle.run_step(w)
        if len(_cache) > 8:
            _cache.clear()
        _cache[key] = (w, ref, kp, vp)
    return _cache[key]


def dequantized(w, kp, vp):
    """float64 K and V pools [n_blocks, H_kv, bs, D] as the oracle reads them."""
    kv = w.cfg.kv_dtype
    if kv == "fp8":
        return (oracle.e4m3_dequantize(*kp).astype(np.float64), oracle.e4m3_dequantize(*vp).astype(np.float64))
    if kv == "mxfp4":
        return (oracle.mxfp4_dequantize(*kp).astype(np.float64), oracle.mxfp4_dequantize(*vp).astype(np.float64))
    return oracle.decode(w.cfg.dtype, kp), oracle.decode(w.cfg.dtype, vp)


def scores(w, kf, b, h):
    """fp64 scores of query head h of request b over its context, in natural units."""
    n = int(w.context_lens[b])
    t = np.arange(n)
    K = kf[w.block_tables[b, t // 16], h // w.cfg.G, t % 16]
    q = oracle.decode(w.cfg.dtype, w.q[b, h])
    return float(w.scale) * (K @ q)


def lazy_jumps(s_log2, part_tokens, chunk_blocks, waves):
    """For each partition of ``s_log2`` (a head's scores in binary orders), the fewest times
    over ``waves`` waves (chunks of ``chunk_blocks`` 16-token blocks dealt round-robin) that a
    wave's reference maximum, moved only when a chunk's maximum exceeds it by more than 8,
    moves after the wave's first chunk.  Returns [(partition length, jumps)]."""
    res = []
    for p0 in range(0, s_log2.size, part_tokens):
        seg = s_log2[p0:p0 + part_tokens]
        nb = -(-seg.size // 16)
        bm = [seg[16 * i:16 * i + 16].max() for i in range(nb)]
        ch = [max(bm[c * chunk_blocks:(c + 1) * chunk_blocks]) for c in range(-(-nb // chunk_blocks))]
        counts = []
        for wv in range(waves):
            seq = ch[wv::waves]
            if not seq:
                continue
            m, c = seq[0], 0
            for x in seq[1:]:
                if x > m + 8.0:
                    c, m = c + 1, x
            counts.append(c)
        res.append((seg.size, min(counts)))
    return res


def assert_climbs(w, kp, P):
    """From the inputs: inside every 512-token partition of the pure-climb request, each
    climbing head's lazily moved maximum jumps at least twice, for the chunk/wave shapes of
    the grouped kernels (1 block x 4 or 2 waves, 2 blocks x 4 waves)."""
    kf = dequantized(w, kp, kp)[0]
    part = 512 if P == 0 else P
    b = 4
    for h in range(0, w.cfg.H_q, 2):                    # even heads of each group climb
        s = scores(w, kf, b, h) * LOG2E
        for chunk, waves in ((1, 4), (1, 2), (2, 4)):
            for length, jumps in lazy_jumps(s, part, chunk, waves):
                if length >= 512:
                    assert jumps >= 2, f"head {h}: {jumps} lazy jumps in a {length}-token partition " \
                                       f"({chunk} block chunks, {waves} waves)"


# ---------------------------------------------------------------------------
# running the step
# ---------------------------------------------------------------------------

def run(torch, w, P, append):
    d = upload(w, "cuda")
    kv = w.cfg.kv_dtype
    if kv:
        sc = (d["k_scale"], d["v_scale"])
        fa = pkv.append_decode_attention_fp8 if kv == "fp8" else pkv.append_decode_attention_mxfp4
        fd = pkv.paged_decode_attention_fp8 if kv == "fp8" else pkv.paged_decode_attention_mxfp4
    else:
        sc = ()
        fa, fd = pkv.append_decode_attention, pkv.paged_decode_attention
    if append:
        out = fa(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], *sc, d["block_tables"], d["positions"],
                 float(w.scale), w.max_context_len, partition_size=P)
    else:
        out = fd(d["q"], d["k_pool"], d["v_pool"], *sc, d["block_tables"], d["context_lens"], float(w.scale),
                 w.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    return out.cpu().numpy(), d


def assert_pools(w, d, kp, vp):
    if w.cfg.kv_dtype:
        assert bits_equal(d["k_pool"].cpu().numpy(), kp[0]) and bits_equal(d["k_scale"].cpu().numpy(), kp[1])
        assert bits_equal(d["v_pool"].cpu().numpy(), vp[0]) and bits_equal(d["v_scale"].cpu().numpy(), vp[1])
    else:
        assert bits_equal(to_numpy_bits(d["k_pool"], w.cfg.dtype), kp)
        assert bits_equal(to_numpy_bits(d["v_pool"], w.cfg.dtype), vp)


def expect(prefix, P):
    """The launch-string prefix a family shows at partition size P (the even splits are
    split-step plans: unsplit, the same family runs the per-partition grouped kernel)."""
    if P == 0:
        return {"gqa_mfma_even ": "gqa_mfma_kdma ", "mxfp4_mfma_even ": "mxfp4_mfma "}.get(prefix, prefix)
    return prefix


def _setenv(monkeypatch, env):
    for k, v in env.items():
        monkeypatch.setenv(k, v)


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("family", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("P", [0, 32, 512])
@pytest.mark.parametrize("append", [False, True])
def test_climbing_scores(torch_dev, monkeypatch, family, P, append):
    _, kv, dtype, G, env, prefix = family
    _setenv(monkeypatch, env)
    w, ref, kp, vp = climbing(kv, dtype, G, append)
    if P != 32:
        assert_climbs(w, kp, P)
    got, d = run(torch_dev, w, P, append)
    launch = pkv.last_launch()
    assert launch.startswith(expect(prefix, P)), launch
    assert_close(got, ref, dtype, f"{family[0]} P={P} append={append} [{launch}]")
    if append:
        assert_pools(w, d, kp, vp)


@pytest.mark.parametrize("family", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_dominant_tokens_give_their_rows(torch_dev, monkeypatch, family):
    """The climbing heads of request 2 (token 0 dominant) and 3 (the appended token dominant)
    return that token's V row: every other weight is below 2^-90 of it."""
    _, kv, dtype, G, env, prefix = family
    _setenv(monkeypatch, env)
    w, ref, kp, vp = climbing(kv, dtype, G, True)
    kf, vf = dequantized(w, kp, vp)
    for P in (0, 512):
        got, _ = run(torch_dev, w, P, True)
        for b, tok in ((2, 0), (3, int(w.context_lens[3]) - 1)):
            blk, slot = w.block_tables[b, tok // 16], tok % 16
            for h in range(0, w.cfg.H_q, 2):
                s = scores(w, kf, b, h)
                top = np.argsort(s)[-2:]
                assert top[1] == tok and (s[top[1]] - s[top[0]]) * LOG2E > 60, (b, h)
                row = vf[blk, h // G, slot]
                atol = TOL[dtype][0]
                assert np.abs(got[b, h] - row).max() <= atol, f"{family[0]} P={P} b={b} h={h}"


@pytest.mark.parametrize("family", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("P", [0, 512])
@pytest.mark.parametrize("append", [False, True])
def test_huge_logits_give_the_argmax_row(torch_dev, monkeypatch, family, P, append):
    _, kv, dtype, G, env, prefix = family
    _setenv(monkeypatch, env)
    base = "c3f8" if kv == "fp8" else "c3f4" if kv == "mxfp4" else "c2"
    cfg = get_config(base, B=4, H_q=H_KV * G, H_kv=H_KV, D=128, dtype=dtype, lengths=("fixed", (1, 40, 700, 2600)),
                     pool=("factor", 1.3), append=append, q_std=30.0, partition_size=P)
    w = make_workload(cfg, 21 + G)
    w.scale = np.float32(1.0)
    ref, kp, vp = oracle.run_step(w)
    got, d = run(torch_dev, w, P, append)
    launch = pkv.last_launch()
    assert launch.startswith(expect(prefix, P)), launch
    kf, vf = dequantized(w, kp, vp)
    if dtype == "f32":
        # f32 q: scores of ~10^3 carry float32 rounding of ~10^-4 (a correctly rounded float32
        # computation misses the oracle by up to 5e-5 here), which only a near tie of the two
        # largest scores passes on to the output.  Rows whose two largest scores are 10 or more
        # apart (runner-up weight <= e^-10) keep (1e-5, 1e-5); near-tied rows get the 16-bit bound.
        near = 0
        for b in range(cfg.B):
            for h in range(cfg.H_q):
                s = np.sort(scores(w, kf, b, h))
                tied = s.size > 1 and s[-1] - s[-2] < 10.0
                near += tied
                assert_close(got[b, h], ref[b, h], "f16" if tied else "f32",
                             f"{family[0]} huge logits b={b} h={h} P={P} append={append} [{launch}]")
        assert near <= cfg.B * cfg.H_q // 4, near
    else:
        assert_close(got, ref, dtype, f"{family[0]} huge logits P={P} append={append} [{launch}]")
    if append:
        assert_pools(w, d, kp, vp)
    n_checked = 0
    for b in range(cfg.B):
        n = int(w.context_lens[b])
        for h in range(cfg.H_q):
            s = scores(w, kf, b, h)
            assert np.max(np.abs(s)) > 100.0 or n < 40
            order = np.argsort(s)
            if n > 1 and s[order[-1]] - s[order[-2]] < 40.0:
                continue                       # runner-up within e^-40: not a one-row softmax
            t = int(order[-1])
            row = vf[w.block_tables[b, t // 16], h // G, t % 16]
            assert np.abs(got[b, h] - row).max() <= TOL[dtype][0], (b, h)
            n_checked += 1
    assert n_checked >= cfg.H_q * cfg.B // 2


VARIANT_CASES = ([("gqa", v) for v in GQA_VARIANTS] + [("even", v) for v in ("4,1", "2,1", "8,1")]
                 + [("mha", v) for v in MHA_VARIANTS]
                 + [("fp8g", v) for v in GQA8_VARIANTS] + [("mx4", v) for v in MX4_VARIANTS]
                 + [("fp8", v) for v in ("4,2,1", "4,2,2", "8,2,2", "4,4,1")])


def _variant_env(kind, v):
    if kind == "gqa":
        k, nw, ch, pf = v
        return {"PKV_GQA_KIND": str(k), "PKV_GQA_NW": str(nw), "PKV_GQA_CH": str(ch), "PKV_GQA_PF": str(pf),
                "PKV_GQA_EVEN": "0"}, f"nw={nw} ch={ch} pf={pf}"
    if kind == "even":
        nw, pf = v.split(",")
        return {"PKV_GQA_EVEN": "2", "PKV_GQA_EVEN_NW": nw, "PKV_GQA_EVEN_PF": pf}, f"nw={nw} ch=1 pf={pf}"
    if kind == "mha":
        nw, ch, pf = v
        return {"PKV_MHA_NW": str(nw), "PKV_MHA_CH": str(ch), "PKV_MHA_PF": str(pf)}, f"nw={nw} ch={ch} pf={pf}"
    if kind == "fp8g":
        nw, ch, pf, wpe, kd = v.split(",")
        return ({"PKV_GQA8_NW": nw, "PKV_GQA8_CH": ch, "PKV_GQA8_PF": pf, "PKV_GQA8_WPE": wpe, "PKV_GQA8_KDMA": kd,
                 "PKV_LP_MIN_PART": "0"},
                f"nw={nw} ch={ch} pf={pf} wpe={wpe}" + (" kdma" if kd == "1" else "") + " ")
    if kind == "fp8":
        nw, ch, pf = v.split(",")
        return {"PKV_FP8_NW": nw, "PKV_FP8_CH": ch, "PKV_FP8_PF": pf}, f"nw={nw} ch={ch} pf={pf}"
    env, tag = mx4_variant_env(v, H_KV)
    return {**env, "PKV_LP_MIN_PART": "0"}, tag


@pytest.mark.parametrize("kind,variant", VARIANT_CASES, ids=[f"{k}-{v}" for k, v in VARIANT_CASES])
def test_climbing_scores_every_launch_variant(torch_dev, monkeypatch, kind, variant):
    env, tag = _variant_env(kind, variant)
    _setenv(monkeypatch, env)
    kv = {"fp8g": "fp8", "fp8": "fp8", "mx4": "mxfp4"}.get(kind, "")
    G = 1 if kind in ("mha", "fp8") or (kind == "mx4" and variant.startswith("0")) else 8
    for dtype in ("bf16", "f16"):
        w, ref, kp, vp = climbing(kv, dtype, G, True)
        for P in ((32, 512) if kind == "even" else (0, 512)):   # the even split is a split-step plan
            got, d = run(torch_dev, w, P, True)
            launch = pkv.last_launch()
            assert tag in launch and (kind != "even" or launch.startswith("gqa_mfma_even ")), launch
            assert_close(got, ref, dtype, f"{kind} {variant} {dtype} P={P} [{launch}]")
            assert_pools(w, d, kp, vp)
