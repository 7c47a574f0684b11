"""Pins of the oracle's FP8 (OCP E4M3) K/V functions against things fixed
outside it: the OCP specification's E4M3 values, torch's float8_e4m3fn
decoding and round-to-nearest-even encoding, hand-worked rows, the grid's
error bound, torch SDPA in float64 on the dequantized values, and planted
mistakes that these pins must catch."""
import json
import math
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from workloads import to_storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3_values.json")
ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def torch_encode(v32):
    """float32 -> E4M3 code by torch (round to nearest even; magnitudes above 448 clamped first)."""
    t = torch.from_numpy(np.clip(np.asarray(v32, dtype=np.float32), -448, 448))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_specification_table(oracle_lib):
    for item in json.load(open(GOLDEN))["values"]:
        got = oracle.e4m3_decode(np.array([int(item["code"], 16)], np.uint8))[0]
        if item["value"] == "nan":
            assert math.isnan(got)
        else:
            assert got == item["value"] and math.copysign(1, got) == math.copysign(1, item["value"])


def test_decode_all_codes_matches_torch(oracle_lib):
    mine, ref = oracle.e4m3_decode(ALL), torch_decode(ALL)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], ref[~nan])
    pos = mine[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # the 127 non-negative finite codes increase
    assert np.array_equal(mine[0x80:0xFF], -pos)           # sign-magnitude


def test_quantize_hand_worked_rows(oracle_lib):
    codes, s = oracle.e4m3_quantize_row("f32", np.array([1.0, -0.5, 0.0, 3.0], np.float32))
    # amax 3: floor(log2 3) = 1, scale 2^(1-8); 1/s = 128 = 2^7 -> 0x70; -64 -> 0xE8; 384 = 1.5*2^8 -> 0x7C
    assert s == np.float32(2.0 ** -7) and list(codes) == [0x70, 0xE8, 0x00, 0x7C]
    codes, s = oracle.e4m3_quantize_row("f32", np.array([300, 1.0625, 1.1875, 17, 500], np.float32))
    # amax 500 -> scale 1; 300 nearer 288 (0x79) than 320; ties 1.0625 -> 1.0, 1.1875 -> 1.25, 17 -> 16;
    # 500 saturates to 448
    assert s == np.float32(1.0) and list(codes) == [0x79, 0x38, 0x3A, 0x58, 0x7E]
    codes, s = oracle.e4m3_quantize_row("f32", np.zeros(8, np.float32))
    assert s == np.float32(1.0) and not codes.any()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_quantize_matches_torch_rounding_and_bounds(oracle_lib, dtype):
    rng = np.random.default_rng(5)
    for trial in range(200):
        D = int(rng.choice([8, 64, 128]))
        mag = 10.0 ** rng.uniform(-6, 4)
        x32 = (rng.standard_normal(D) * mag).astype(np.float32)
        if trial % 7 == 0:
            x32[rng.integers(D)] = 0.0
        row = to_storage(x32, dtype)
        codes, s = oracle.e4m3_quantize_row(dtype, row)
        x = oracle.decode(dtype, row)
        amax = np.abs(x).max()
        e = math.floor(math.log2(amax))
        assert s == np.float32(2.0 ** max(e - 8, -126))            # power of two from the row maximum
        assert 256 <= amax / s < 512
        v = (x / float(s)).astype(np.float32)                      # exact: division by a power of two
        assert np.array_equal(codes, torch_encode(v))
        deq = oracle.e4m3_decode(codes) * float(s)
        err = np.abs(deq - x)
        normal = np.abs(v) >= 2.0 ** -6
        # half a unit in the last place: 2^-4 relative on the normal range, 2^-10 * scale below it,
        # plus the clamp above 448
        bound = np.where(normal, np.abs(x) * 2.0 ** -4, float(s) * 2.0 ** -10) + np.maximum(
            np.abs(x) - 448 * float(s), 0)
        assert np.all(err <= bound * (1 + 1e-12))


def test_append_fp8_writes_codes_and_scales(oracle_lib):
    rng = np.random.default_rng(6)
    B, H_kv, D, bs, nb = 3, 2, 64, 16, 9
    k_new = to_storage(rng.standard_normal((B, H_kv, D)).astype(np.float32), "bf16")
    v_new = to_storage(rng.standard_normal((B, H_kv, D)).astype(np.float32) * 3, "bf16")
    kp = np.full((nb, H_kv, bs, D), 0x7F, np.uint8)
    vp = kp.copy()
    ks = np.full((nb, H_kv, bs), np.nan, np.float32)
    vs = ks.copy()
    bt = np.array([[4, 0], [7, 2], [1, 8]], np.int32)
    pos = np.array([3, 16, 31], np.int32)
    oracle.kv_append_fp8("bf16", k_new, v_new, kp, vp, ks, vs, bt, pos, bs)
    written = set()
    for b in range(B):
        blk, slot = bt[b, pos[b] // bs], pos[b] % bs
        for g in range(H_kv):
            for new, pool, sc in ((k_new, kp, ks), (v_new, vp, vs)):
                c, s = oracle.e4m3_quantize_row("bf16", new[b, g])
                assert np.array_equal(pool[blk, g, slot], c) and sc[blk, g, slot] == s
            written.add((blk, slot))
    untouched = np.ones((nb, bs), bool)
    for blk, slot in written:
        untouched[blk, slot] = False
    assert np.all(kp.transpose(0, 2, 1, 3)[untouched] == 0x7F) and np.all(np.isnan(ks.transpose(0, 2, 1)[untouched]))


def random_codes(rng, shape):
    """Finite E4M3 codes with exponents concentrated like a quantized Gaussian row."""
    ex = np.clip(np.rint(rng.normal(12.5, 1.6, shape)), 0, 15).astype(np.uint8)
    man = rng.integers(0, 8, shape).astype(np.uint8)
    man = np.where((ex == 15) & (man == 7), 6, man).astype(np.uint8)
    sign = rng.integers(0, 2, shape).astype(np.uint8)
    return (sign << 7) | (ex << 3) | man


@pytest.mark.parametrize("q_dtype,H_q,H_kv,D", [("bf16", 4, 2, 64), ("f16", 2, 2, 128), ("f32", 8, 1, 64)])
def test_fp8_attention_matches_sdpa(oracle_lib, q_dtype, H_q, H_kv, D):
    """Contiguous case (block b of request r is block r*W + b) against torch SDPA in float64."""
    rng = np.random.default_rng(7)
    bs, lens = 16, [1, 17, 40]
    B, W = len(lens), 3
    nb = B * W
    kp, vp = random_codes(rng, (nb, H_kv, bs, D)), random_codes(rng, (nb, H_kv, bs, D))
    ks = (2.0 ** rng.integers(-12, -6, (nb, H_kv, bs))).astype(np.float32)
    vs = (2.0 ** rng.integers(-12, -6, (nb, H_kv, bs))).astype(np.float32)
    q = to_storage(rng.standard_normal((B, H_q, D)).astype(np.float32), q_dtype)
    bt = np.arange(nb, dtype=np.int32).reshape(B, W)
    ctx = np.array(lens, np.int32)
    scale = np.float32(1 / math.sqrt(D))
    got = oracle.paged_decode_attention_fp8(q_dtype, q, kp, vp, ks, vs, bt, ctx, scale)
    K = oracle.e4m3_decode(kp) * ks[..., None].astype(np.float64)
    V = oracle.e4m3_decode(vp) * vs[..., None].astype(np.float64)
    qd = oracle.decode(q_dtype, q)
    G = H_q // H_kv
    for b, n in enumerate(lens):
        Kb = torch.from_numpy(K[b * W:(b + 1) * W].transpose(1, 0, 2, 3).reshape(H_kv, W * bs, D)[:, :n])
        Vb = torch.from_numpy(V[b * W:(b + 1) * W].transpose(1, 0, 2, 3).reshape(H_kv, W * bs, D)[:, :n])
        Kb, Vb = Kb.repeat_interleave(G, 0), Vb.repeat_interleave(G, 0)
        qb = torch.from_numpy(qd[b]).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(qb, Kb, Vb, scale=float(scale)).squeeze(1).numpy()
        assert np.max(np.abs(got[b] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


# -- planted mistakes in the FP8 part of oracle.c --------------------------------

MUTATIONS = {
    "ties_away_from_zero": (r"\(err == best_err && \(c & 1\) == 0 && \(best & 1\) == 1\)", "(err == best_err)"),
    "scale_exponent_off_by_one": (r"E = e2 - 1 - 8;", "E = e2 - 8;"),
    "top_code_left_out": (r"for \(int c = 1; c <= 0x7E; \+\+c\)", "for (int c = 1; c < 0x7E; ++c)"),
    "bias_off_by_one": (r"ldexp\(1\.0 \+ man / 8\.0, ex - 7\)", "ldexp(1.0 + man / 8.0, ex - 8)"),
    "subnormal_scale": (r"ldexp\(\(double\)man, -9\)", "ldexp((double)man, -10)"),
    "sign_dropped": (r"codes\[d\] = \(uint8_t\)\(signbit\(v\) \? \(mag \| 0x80\) : mag\);", "codes[d] = mag;"),
}


def _fp8_pin_suite(lib_path):
    saved = oracle._lib, oracle._LIB_PATH
    try:
        oracle._lib = None
        oracle._LIB_PATH = lib_path
        try:
            test_decode_matches_specification_table(None)
            test_decode_all_codes_matches_torch(None)
            test_quantize_hand_worked_rows(None)
            test_quantize_matches_torch_rounding_and_bounds(None, "bf16")
        except (AssertionError, oracle.OracleError):
            return False
        return True
    finally:
        oracle._lib, oracle._LIB_PATH = saved


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_fp8_mistakes_are_caught(oracle_lib):
    path = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    src = open(path).read()
    tmp = tempfile.mkdtemp(prefix="oracle_fp8_mut_")
    try:
        base = os.path.join(tmp, "base.so")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", base, path, "-lm"], check=True)
        assert _fp8_pin_suite(base)
        for name, (pat, rep) in MUTATIONS.items():
            mutated, count = re.subn(pat, rep, src)
            assert count >= 1, f"mutation {name} did not apply"
            c, so = os.path.join(tmp, name + ".c"), os.path.join(tmp, name + ".so")
            open(c, "w").write(mutated)
            subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"], check=True)
            assert not _fp8_pin_suite(so), f"planted mistake '{name}' was not caught"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
