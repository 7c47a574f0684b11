"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side validation rejects bad arguments with the documented status codes
before anything is launched (no GPU needed for any of these calls)."""
import ctypes
import os
import re

import pytest

import paged_kv_decode_blocks_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

OK, E_NULL, E_ARG, E_UNSUP, E_WS = 0, -1, -2, -3, -4
# Aligned but bogus device address.  Every call below either fails validation or
# has B == 0, so nothing is ever launched with it; a call that passed validation
# with this pointer would launch a kernel on a bogus address, so none may.
FAKE = 0x10000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_decode_blocks_amd.build import build
        build()
    return pkv.load_library()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    decl = declared_symbols()
    assert set(decl) == set(pkv.EXPORTED_SYMBOLS)
    for name in decl:
        assert hasattr(lib, name), name
    # and from the dynamic symbol table itself
    nm = os.popen(f"nm -D --defined-only {pkv.LIB_PATH}").read()
    for name in decl:
        assert re.search(rf"\bT {name}\b", nm), name


def test_status_strings(lib):
    assert lib.pkv_status_string(0) == b"PKV_OK"
    assert lib.pkv_status_string(-4) == b"PKV_ERR_WORKSPACE"
    assert pkv.version() >= 100


def attn(lib, dtype=1, out=FAKE, q=FAKE, qrs=32 * 128, kp=FAKE, vp=FAKE, bt=FAKE, bts=64, ctx=FAKE, B=8, H_q=32,
         H_kv=32, D=128, bs=16, nb=1024, maxc=1024, scale=0.088, P=0, ws=None, wsb=0):
    return lib.pkv_paged_decode_attention(dtype, out, q, qrs, kp, vp, bt, bts, ctx, B, H_q, H_kv, D, bs, nb, maxc,
                                          scale, P, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), E_UNSUP),
    (dict(D=96, qrs=32 * 96), E_UNSUP),
    (dict(bs=32), E_UNSUP),
    (dict(H_q=30), E_ARG),
    (dict(H_kv=0), E_ARG),
    (dict(B=-1), E_ARG),
    (dict(nb=0), E_ARG),
    (dict(bts=0), E_ARG),
    (dict(maxc=1025), E_ARG),                       # > bt_stride * block_size
    (dict(maxc=-1), E_ARG),
    (dict(P=100), E_ARG),                           # not a multiple of the block size
    (dict(P=-16), E_ARG),
    (dict(q=None), E_NULL),
    (dict(ctx=None), E_NULL),
    (dict(out=FAKE + 4), E_ARG),                    # misaligned
    (dict(qrs=32 * 128 - 8), E_ARG),                # row stride too small
    (dict(qrs=32 * 128 + 4), E_ARG),                # row stride not a multiple of 16 bytes
    (dict(scale=float("inf")), E_ARG),
    (dict(H_q=64, H_kv=2, dtype=2, qrs=64 * 128), E_UNSUP),   # G = 32 on the grouped path
    (dict(P=256), E_WS),                            # split without workspace
    (dict(P=256, ws=FAKE, wsb=100), E_WS),          # too small
    (dict(P=256, ws=FAKE + 16, wsb=1 << 30), E_WS), # misaligned workspace
    (dict(B=0), OK),                                # nothing to do, nothing launched
    (dict(B=0, q=None, out=None), OK),
])
def test_attention_validation(lib, kw, status):
    assert attn(lib, **kw) == status
    if status != OK:
        assert lib.pkv_last_error() != b""


def test_workspace_bytes(lib):
    # 8 requests x 32 heads x 4 partitions x (128 + 1) floats, each part 256-aligned
    assert lib.pkv_decode_workspace_bytes(8, 32, 128, 1024, 256) == 8 * 32 * 4 * 128 * 4 + 8 * 32 * 4 * 4
    assert lib.pkv_decode_workspace_bytes(8, 32, 128, 1024, 0) == 0
    assert lib.pkv_decode_workspace_bytes(8, 32, 128, 1024, 1024) == 0       # one partition: no split
    assert lib.pkv_decode_workspace_bytes(3, 5, 64, 17, 16) == ((3 * 5 * 2 * 64 * 4 + 255) // 256 * 256
                                                                 + (3 * 5 * 2 * 4 + 255) // 256 * 256)


def test_append_validation(lib):
    f = lib.pkv_kv_append
    assert f(9, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, 64, FAKE, 8, 32, 128, 16, 1024, None) == E_UNSUP
    assert f(1, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, 64, None, 8, 32, 128, 16, 1024, None) == E_NULL
    assert f(1, FAKE, FAKE, 31 * 128, FAKE, FAKE, FAKE, 64, FAKE, 8, 32, 128, 16, 1024, None) == E_ARG
    assert f(1, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, 64, FAKE, 8, 32, 128, 8, 1024, None) == E_UNSUP
    assert f(1, FAKE, FAKE, 32 * 128, FAKE + 2, FAKE, FAKE, 64, FAKE, 8, 32, 128, 16, 1024, None) == E_ARG
    assert f(1, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, 64, FAKE, 0, 32, 128, 16, 1024, None) == OK


def test_fused_validation(lib):
    f = lib.pkv_append_decode_attention
    args = [1, FAKE, FAKE, 32 * 128, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, 64, FAKE, 8, 32, 32, 128, 16, 1024,
            1024, 0.088, 0, None, 0, None]
    bad = list(args)
    bad[11] = None                      # positions
    assert f(*bad) == E_NULL
    bad = list(args)
    bad[4] = None                       # k_new
    assert f(*bad) == E_NULL
    bad = list(args)
    bad[6] = 31 * 128                   # new_row_stride
    assert f(*bad) == E_ARG
    bad = list(args)
    bad[12] = 0                         # B = 0
    assert f(*bad) == OK


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(pkv.PkvError):
        pkv.load_library(str(tmp_path / "nope.so"))


def copy_blocks(lib, dtype=1, kp=FAKE, vp=FAKE, src=FAKE, dst=FAKE, n=4, H_kv=8, D=128, bs=16, nb=64):
    return lib.pkv_copy_blocks(dtype, kp, vp, src, dst, n, H_kv, D, bs, nb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=9), E_UNSUP),
    (dict(n=-1), E_ARG),
    (dict(H_kv=0), E_ARG),
    (dict(D=96), E_UNSUP),
    (dict(bs=8), E_UNSUP),
    (dict(nb=0), E_ARG),
    (dict(src=None), E_NULL),
    (dict(dst=None), E_NULL),
    (dict(kp=None), E_NULL),
    (dict(vp=FAKE + 4), E_ARG),
    (dict(n=0, kp=None, vp=None, src=None, dst=None), OK),   # nothing to copy: nothing launched
])
def test_copy_blocks_validation(lib, kw, status):
    assert copy_blocks(lib, **kw) == status
    if status:
        assert lib.pkv_last_error()
