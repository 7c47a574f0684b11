"""Pins of the oracle's MXFP4 K/V functions against things fixed outside it:
the OCP MX specification's E2M1 and E8M0 values, hand-worked blocks, an
independent brute-force search of the E2M1 grid in Python, the grid's error
bound, torch SDPA in float64 on the dequantized values, and planted mistakes
that these pins must catch."""
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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e2m1_values.json")
GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def pack(codes4):
    """4-bit codes -> bytes, element 2k in the low nibble of byte k."""
    c = np.asarray(codes4, dtype=np.uint8)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.size * 2, np.uint8)
    out[0::2], out[1::2] = p & 15, p >> 4
    return out


def dequant_row(codes, scales):
    return oracle.mxfp4_dequantize(codes[None], scales[None])[0].astype(np.float64)


def test_e2m1_decode_matches_specification_table(oracle_lib):
    spec = json.load(open(GOLDEN))["e2m1"]
    got = oracle.e2m1_decode(pack([int(it["code"], 16) for it in spec]))
    for it, v in zip(spec, got):
        assert v == it["value"] and math.copysign(1, v) == math.copysign(1, it["value"])


def test_e8m0_scales_match_specification(oracle_lib):
    ones = pack([2] * 32)                                  # code 2 = 1.0
    for bits, expect in ((0x00, 2.0 ** -127), (0x7F, 1.0), (0x80, 2.0), (0xFE, 2.0 ** 127), (0x64, 2.0 ** -27)):
        assert np.all(dequant_row(ones, np.array([bits], np.uint8)) == expect)
    assert np.all(np.isnan(dequant_row(ones, np.array([0xFF], np.uint8))))


def test_quantize_hand_worked_blocks(oracle_lib):
    # amax 7.9: floor(log2 7.9) = 2, E = 0 (byte 127); 1.25 and -0.75 are ties -> even codes 1.0 and -1.0;
    # 0.2 < 0.25 -> 0; 7.9 saturates to 6
    x = np.zeros(32, np.float32)
    x[:6] = [6, 3, 1.25, -0.75, 0.2, 7.9]
    codes, s = oracle.mxfp4_quantize_row("f32", x)
    assert list(s) == [127]
    assert list(unpack(codes)[:6]) == [0x7, 0x5, 0x2, 0xA, 0x0, 0x7] and not unpack(codes)[6:].any()
    # amax 0.3: floor(log2 0.3) = -2, E = -4 (byte 123): 0.3*16 = 4.8 -> 4; 0.1*16 = 1.6 -> 1.5;
    # -0.05*16 = -0.8 -> -1.0; 0.15*16 = 2.4 -> 2
    x = np.zeros(32, np.float32)
    x[:4] = [0.3, 0.1, -0.05, 0.15]
    codes, s = oracle.mxfp4_quantize_row("f32", x)
    assert list(s) == [123] and list(unpack(codes)[:4]) == [0x6, 0x3, 0xA, 0x4]
    assert list(dequant_row(codes, s)[:4]) == [0.25, 0.09375, -0.0625, 0.125]
    # every tie of the grid at E = 0 (4.0 pins the exponent): ties go to the even code
    x = np.zeros(32, np.float32)
    x[:10] = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.26, 2.51]
    codes, s = oracle.mxfp4_quantize_row("f32", x)
    assert list(s) == [127]
    assert list(dequant_row(codes, s)[:10]) == [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 0.5, 3.0]
    # all zero -> E = -127 (byte 0), codes 0; tiny block -> E clamped at -127, codes round to 0
    codes, s = oracle.mxfp4_quantize_row("f32", np.zeros(32, np.float32))
    assert list(s) == [0] and not codes.any()
    codes, s = oracle.mxfp4_quantize_row("f32", np.full(32, 2.0 ** -140, np.float32))
    assert list(s) == [0] and not codes.any()
    # near the top of float32: amax 1.5 * 2^127 -> E = 125 (byte 252), value 6
    codes, s = oracle.mxfp4_quantize_row("f32", np.full(32, 1.5 * 2.0 ** 127, np.float32))
    assert list(s) == [252] and np.all(unpack(codes) == 0x7)
    # two blocks of one row take their own scales: 3 = 6 * 2^-1 (byte 126, code 6.0),
    # -0.375 = -6 * 2^-4 (byte 123, code -6.0)
    x = np.concatenate([np.full(32, 3.0, np.float32), np.full(32, -0.375, np.float32)])
    codes, s = oracle.mxfp4_quantize_row("f32", x)
    assert list(s) == [126, 123] and np.all(unpack(codes)[:32] == 0x7) and np.all(unpack(codes)[32:] == 0xF)


def brute_force_code(v):
    """Nearest E2M1 magnitude to |v| with ties to the even code, by direct search (independent of oracle.c)."""
    a = min(abs(v), 6.0)
    best = min(range(8), key=lambda c: (abs(a - GRID[c]), c & 1))
    return best | (8 if math.copysign(1, v) < 0 else 0)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_quantize_matches_brute_force_and_bounds(oracle_lib, dtype):
    rng = np.random.default_rng(11)
    for trial in range(150):
        D = int(rng.choice([32, 64, 128]))
        mag = 10.0 ** rng.uniform(-5, 3)
        x32 = (rng.standard_normal(D) * mag).astype(np.float32)
        if trial % 5 == 0:
            x32[rng.integers(D)] = 0.0
        row = to_storage(x32, dtype)
        codes, s = oracle.mxfp4_quantize_row(dtype, row)
        x = oracle.decode(dtype, row)
        deq = dequant_row(codes, s)
        for blk in range(D // 32):
            xb = x[blk * 32:(blk + 1) * 32]
            amax = np.abs(xb).max()
            E = max(min(math.frexp(amax)[1] - 1 - 2, 127), -127) if amax > 0 else -127
            assert s[blk] == E + 127
            got = unpack(codes)[blk * 32:(blk + 1) * 32]
            want = [brute_force_code(math.ldexp(float(v), -E)) for v in xb]
            assert list(got) == want
            # half the grid spacing where it is not clamped (0.25 below 2, 0.5 below 4, 1 up to 6), times 2^E
            u = np.abs(xb) / 2.0 ** E
            half = np.where(u < 2, 0.25, np.where(u < 4, 0.5, 1.0)) * 2.0 ** E
            err = np.abs(deq[blk * 32:(blk + 1) * 32] - xb)
            assert np.all(err <= half + np.maximum(np.abs(xb) - 6 * 2.0 ** E, 0) + 1e-300)


def test_append_mxfp4_writes_codes_and_scales(oracle_lib):
    rng = np.random.default_rng(12)
    B, H_kv, D, bs, nb = 3, 2, 64, 16, 9
    k_new = to_storage(rng.standard_normal((B, H_kv, D)).astype(np.float32), "bf16")
    v_new = to_storage(rng.standard_normal((B, H_kv, D)).astype(np.float32) * 3, "bf16")
    kp = np.full((nb, H_kv, bs, D // 2), 0x77, np.uint8)
    vp = kp.copy()
    ks = np.full((nb, H_kv, bs, D // 32), 0xFF, np.uint8)
    vs = ks.copy()
    bt = np.array([[4, 0], [7, 2], [1, 8]], np.int32)
    pos = np.array([3, 16, 31], np.int32)
    oracle.kv_append_mxfp4("bf16", k_new, v_new, kp, vp, ks, vs, bt, pos, bs)
    untouched = np.ones((nb, bs), bool)
    for b in range(B):
        blk, slot = bt[b, pos[b] // bs], pos[b] % bs
        for g in range(H_kv):
            for new, pool, sc in ((k_new, kp, ks), (v_new, vp, vs)):
                c, s = oracle.mxfp4_quantize_row("bf16", new[b, g])
                assert np.array_equal(pool[blk, g, slot], c) and np.array_equal(sc[blk, g, slot], s)
        untouched[blk, slot] = False
    assert np.all(kp.transpose(0, 2, 1, 3)[untouched] == 0x77)
    assert np.all(ks.transpose(0, 2, 1, 3)[untouched] == 0xFF)


@pytest.mark.parametrize("q_dtype,H_q,H_kv,D", [("bf16", 4, 2, 64), ("f16", 2, 2, 128), ("f32", 8, 1, 64)])
def test_mxfp4_attention_matches_sdpa(oracle_lib, q_dtype, H_q, H_kv, D):
    """Contiguous case (block b of request r is block r*W + b) against torch SDPA in float64 on
    values dequantized here from the specification's definitions."""
    rng = np.random.default_rng(13)
    bs, lens = 16, [1, 17, 40]
    B, W = len(lens), 3
    nb = B * W
    kp = rng.integers(0, 256, (nb, H_kv, bs, D // 2), dtype=np.uint8)
    vp = rng.integers(0, 256, (nb, H_kv, bs, D // 2), dtype=np.uint8)
    ks = rng.integers(122, 128, (nb, H_kv, bs, D // 32), dtype=np.uint8)
    vs = rng.integers(122, 128, (nb, H_kv, bs, D // 32), dtype=np.uint8)
    q = to_storage(rng.standard_normal((B, H_q, D)).astype(np.float32), q_dtype)
    bt = np.arange(nb, dtype=np.int32).reshape(B, W)
    ctx = np.array(lens, np.int32)
    scale = np.float32(1 / math.sqrt(D))
    got = oracle.paged_decode_attention_mxfp4(q_dtype, q, kp, vp, ks, vs, bt, ctx, scale)
    grid = np.array([math.copysign(GRID[c & 7], -1.0 if c & 8 else 1.0) for c in range(16)])

    def deq(codes, scales):
        vals = grid[np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[:-1] + (D,))]
        return vals * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=-1)

    K, V = deq(kp, ks), deq(vp, vs)
    qd = oracle.decode(q_dtype, q)
    G = H_q // H_kv
    for b, n in enumerate(lens):
        Kb = torch.from_numpy(K[b * W:(b + 1) * W].transpose(1, 0, 2, 3).reshape(H_kv, W * bs, D)[:, :n])
        Vb = torch.from_numpy(V[b * W:(b + 1) * W].transpose(1, 0, 2, 3).reshape(H_kv, W * bs, D)[:, :n])
        Kb, Vb = Kb.repeat_interleave(G, 0), Vb.repeat_interleave(G, 0)
        qb = torch.from_numpy(qd[b]).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(qb, Kb, Vb, scale=float(scale)).squeeze(1).numpy()
        assert np.max(np.abs(got[b] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


# -- planted mistakes in the MXFP4 part of oracle.c -------------------------------

MUTATIONS = {
    "ties_away_from_zero": (r"if \(err < best_err \|\| \(err == best_err && \(c & 1\) == 0 && \(best & 1\) == 1\)\) \{\n            best = c;\n            best_err = err;\n        \}\n    \}\n    return \(uint8_t\)best;\n\}\n\n/\* Quantize one row of D source elements \(D a multiple of 32\)",
                            "if (err <= best_err) {\n            best = c;\n            best_err = err;\n        }\n    }\n    return (uint8_t)best;\n}\n\n/* Quantize one row of D source elements (D a multiple of 32)"),
    "scale_exponent_off_by_one": (r"E = e2 - 1 - 2;", "E = e2 - 2;"),
    "top_code_left_out": (r"for \(int c = 1; c <= 7; \+\+c\)", "for (int c = 1; c < 7; ++c)"),
    "exponent_bias_off": (r"ldexp\(1\.0 \+ 0\.5 \* man, ex - 1\)", "ldexp(1.0 + 0.5 * man, ex - 2)"),
    "nibble_order_swapped": (r"dst\[i\] = e2m1_value\(\(uint8_t\)\(\(packed\[i >> 1\] >> \(4 \* \(i & 1\)\)\) & 15\)\);",
                             "dst[i] = e2m1_value((uint8_t)((packed[i >> 1] >> (4 * (1 - (i & 1)))) & 15));"),
    "sign_dropped": (r"if \(signbit\(v\)\) c \|= 8;", ""),
    "scale_bias_off": (r"scales\[blk\] = \(uint8_t\)\(E \+ 127\);", "scales[blk] = (uint8_t)(E + 128);"),
}


def _mxfp4_pin_suite(lib_path):
    saved = oracle._lib, oracle._LIB_PATH
    try:
        oracle._lib = None
        oracle._LIB_PATH = lib_path
        try:
            test_e2m1_decode_matches_specification_table(None)
            test_e8m0_scales_match_specification(None)
            test_quantize_hand_worked_blocks(None)
            test_quantize_matches_brute_force_and_bounds(None, "bf16")
        except (AssertionError, oracle.OracleError):
            return False
        return True
    finally:
        oracle._lib, oracle._LIB_PATH = saved


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_mxfp4_mistakes_are_caught(oracle_lib):
    path = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    src = open(path).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mxfp4_mut_")
    try:
        base = os.path.join(tmp, "base.so")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", base, path, "-lm"], check=True)
        assert _mxfp4_pin_suite(base)
        for name, (pat, rep) in MUTATIONS.items():
            mutated, count = re.subn(pat, rep, src)
            assert count == 1, f"mutation {name} applied {count} times"
            c, so = os.path.join(tmp, name + ".c"), os.path.join(tmp, name + ".so")
            open(c, "w").write(mutated)
            subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"], check=True)
            assert not _mxfp4_pin_suite(so), f"planted mistake '{name}' was not caught"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
