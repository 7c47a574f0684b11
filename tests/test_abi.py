"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side validation rejects bad arguments with the documented status codes
before anything is launched (no GPU needed for any of these calls)."""
import ctypes
import os
import re

import numpy as np
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
    # a context of 4096 tokens split every 256 spans two 8-wave workgroups: partials needed
    (dict(P=256, maxc=4096, bts=256), E_WS),                            # split without workspace
    (dict(P=256, maxc=4096, bts=256, ws=FAKE, wsb=100), E_WS),          # too small
    (dict(P=256, maxc=4096, bts=256, ws=FAKE + 16, wsb=1 << 30), E_WS), # misaligned workspace
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


def test_persistent_validation(lib):
    f = lib.pkv_append_decode_attention_persistent
    args = [1, FAKE, FAKE, 32 * 128, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, 64, FAKE, 8, 32, 32, 128, 16, 1024,
            1024, 0.088, 0, None, 0, 64, None]
    for n_wg in (0, -3, 65537):
        bad = list(args)
        bad[23] = n_wg
        assert f(*bad) == E_ARG
    bad = list(args)
    bad[0] = 0                          # f32: not taken by the persistent step
    assert f(*bad) == E_UNSUP
    bad = list(args)
    bad[14] = 8                         # H_kv = 8 < H_q: grouped, not taken
    assert f(*bad) == E_UNSUP
    bad = list(args)
    bad[11] = None                      # positions
    assert f(*bad) == E_NULL
    bad = list(args)
    bad[12] = 0                         # B = 0
    assert f(*bad) == OK


def test_mfma_burn_validation(lib):
    f = lib.pkv_probe_mfma_burn
    assert f(8, 100, None, None) == E_NULL
    assert f(8, 100, FAKE + 2, None) == E_ARG
    for n_wg, iters in ((0, 100), (65537, 100), (8, 0), (8, (1 << 30) + 1)):
        assert f(n_wg, iters, FAKE, None) == E_ARG


def test_tile_read_probe_validation(lib):
    f = lib.pkv_probe_tile_read
    # k_pool, v_pool, k_scale, v_scale, n_blocks, heads, tile_bytes, ids, n_items, team, paths, depth, sink, grid,
    # stream
    args = [FAKE, FAKE, FAKE, FAKE, 64, 8, 1024, FAKE, 0, 4, 7, 4, FAKE, 1024, None]
    assert f(*args) == OK                       # no items: nothing launched

    def call(**kw):
        names = ("k", "v", "ks", "vs", "n_blocks", "heads", "tile", "ids", "n", "team", "paths", "depth", "sink",
                 "grid")
        a = list(args)
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)

    for key in ("k", "v", "ids", "sink", "ks"):
        assert call(**{key: None}) == E_NULL, key
    assert call(ks=None, vs=None, paths=1) == OK   # no scale pools: scales are not read
    assert call(ks=None, vs=None) == E_ARG         # paths 7 moves scale tiles that are not there
    assert call(k=FAKE + 8) == E_ARG
    assert call(ks=FAKE + 2) == E_ARG
    for key, val in (("n", -1), ("n", (1 << 30) + 1), ("grid", 0), ("grid", 65537), ("n_blocks", 0),
                     ("heads", 0), ("team", 3), ("team", 8)):
        assert call(**{key: val}) == E_ARG, (key, val)
    assert call(heads=6) == E_ARG               # 6 heads are not a multiple of a 4-wave team
    assert call(heads=6, team=2) == OK
    for tile, paths, depth in ((4096, 7, 4), (512, 0, 4), (1024, 2, 4), (1024, 3, 4), (2048, 6, 4), (8192, 0, 4),
                               (1024, 1, 2), (1024, 7, 3), (1024, 7, 16), (2048, 0, 8), (4096, 0, 2)):
        assert call(tile=tile, paths=paths, depth=depth) == E_UNSUP, (tile, paths, depth)
    for depth in (2, 8):
        assert call(depth=depth) == OK


def test_mxfp4_validation(lib):
    ap = lib.pkv_kv_append_mxfp4
    args = [1, FAKE, FAKE, 8 * 128, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 4, 8, 128, 16, 1024, None]
    bad = list(args)
    bad[13] = 96                        # D
    assert ap(*bad) == E_UNSUP
    bad = list(args)
    bad[6] = None                       # k_scale
    assert ap(*bad) == E_NULL
    bad = list(args)
    bad[4] = FAKE + 8                   # k_pool not 16-byte aligned
    assert ap(*bad) == E_ARG
    bad = list(args)
    bad[11] = 0                         # B = 0
    assert ap(*bad) == OK
    at = lib.pkv_paged_decode_attention_mxfp4
    args = [1, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 8, 32, 32, 128, 16, 1024, 1024,
            0.088, 0, None, 0, None]
    bad = list(args)
    bad[7] = None                       # v_scale
    assert at(*bad) == E_NULL
    bad = list(args)
    bad[16] = 1 << 25                   # n_blocks: code pools of 2^25 * 32 KiB = 1 TiB
    assert at(*bad) == E_UNSUP and b"1 TiB" in lib.pkv_last_error()
    bad = list(args)
    bad[11] = 0                         # B = 0
    assert at(*bad) == OK
    f = lib.pkv_append_decode_attention_mxfp4
    args = [1, FAKE, FAKE, 32 * 128, FAKE, FAKE, 32 * 128, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 8, 32, 32, 128,
            16, 1024, 1024, 0.088, 0, None, 0, None]
    bad = list(args)
    bad[13] = None                      # positions
    assert f(*bad) == E_NULL
    bad = list(args)
    bad[14] = 0                         # B = 0
    assert f(*bad) == OK


def test_copy_blocks_mxfp4_validation(lib):
    f = lib.pkv_copy_blocks_mxfp4
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 8, 128, 16, 64, None]
    bad = list(args)
    bad[8] = 96                         # D
    assert f(*bad) == E_UNSUP
    bad = list(args)
    bad[3] = None                       # v_scale
    assert f(*bad) == E_NULL
    bad = list(args)
    bad[2] = FAKE + 4                   # k_scale not 16-byte aligned
    assert f(*bad) == E_ARG
    bad = list(args)
    bad[6] = 0                          # n = 0: nothing to do
    assert f(*bad) == OK
    bad = list(args)
    bad[6] = -1
    assert f(*bad) == E_ARG


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


@pytest.mark.parametrize("cname,cls", [("pkv_step_desc", pkv.StepDesc), ("pkv_decoder_desc", pkv.DecoderDesc)])
def test_desc_layout_matches_c(tmp_path, cname, cls):
    """The binding's ctypes mirrors of the C structs have the C compiler's size and field offsets."""
    fields = [f[0] for f in cls._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "pkv.h"\nint main(void) {\n'
                   f'  printf("%zu\\n", sizeof({cname}));\n'
                   + "".join(f'  printf("%zu\\n", offsetof({cname}, {f}));\n' for f in fields) + "}\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(cls)
    assert got[1:] == [getattr(cls, f).offset for f in fields]


def test_step_graphs_create_validation(lib):
    """Invalid descriptions are rejected before any HIP call (NULL, with a reason)."""
    d = pkv.StepDesc()
    d.dtype, d.H_q, d.H_kv, d.D, d.block_size, d.n_blocks = 1, 8, 2, 128, 16, 64
    d.positions, d.block_tables, d.bt_stride = FAKE, FAKE, 4
    caps = (ctypes.c_int32 * 3)(1, 2, 4)
    bad = (ctypes.c_int32 * 3)(1, 4, 2)
    P = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert lib.pkv_step_graphs_create(None, P(caps), 3, P(caps), 3) is None
    assert lib.pkv_step_graphs_create(ctypes.byref(d), P(caps), 0, P(caps), 3) is None
    assert lib.pkv_step_graphs_create(ctypes.byref(d), P(bad), 3, P(caps), 3) is None
    assert b"increasing" in lib.pkv_last_error()
    big = (ctypes.c_int32 * 1)(65)                       # > bt_stride * block_size = 64
    assert lib.pkv_step_graphs_create(ctypes.byref(d), P(caps), 3, P(big), 1) is None
    assert b"exceeds" in lib.pkv_last_error()
    d.cow_src = FAKE                                     # cow_dst missing
    assert lib.pkv_step_graphs_create(ctypes.byref(d), P(caps), 3, P(caps), 3) is None
    d.cow_src = None
    d.partition_size, d.workspace, d.workspace_bytes = 16, None, 0
    ctx = (ctypes.c_int32 * 3)(16, 32, 64)              # split into 16-token partitions: needs a workspace
    assert lib.pkv_step_graphs_create(ctypes.byref(d), P(caps), 3, P(ctx), 3) is None
    assert b"workspace" in lib.pkv_last_error()
    assert lib.pkv_step_graphs_launch(None, 1, 1, 0, None) == E_NULL
    lib.pkv_step_graphs_destroy(None)


def test_decoder_create_validation(lib):
    """Invalid decoder descriptions are rejected before any HIP call."""
    d = pkv.DecoderDesc()
    d.dtype, d.H_q, d.H_kv, d.D, d.block_size, d.n_blocks = 1, 8, 2, 128, 16, 64
    d.max_batch, d.bt_stride = 4, 8
    assert lib.pkv_decoder_create(None) is None
    d.max_batch = 0
    assert lib.pkv_decoder_create(ctypes.byref(d)) is None
    d.max_batch = 4
    bc = (ctypes.c_int32 * 2)(2, 3)                      # must end at max_batch = 4
    cc = (ctypes.c_int32 * 2)(64, 128)                   # and at bt_stride * block_size = 128
    d.batch_caps, d.n_batch_caps = ctypes.cast(bc, ctypes.c_void_p), 2
    d.ctx_caps, d.n_ctx_caps = ctypes.cast(cc, ctypes.c_void_p), 2
    assert lib.pkv_decoder_create(ctypes.byref(d)) is None
    assert b"capacity" in lib.pkv_last_error()
    bc[1] = 4
    d.partition_size = 32                                # split needs a workspace
    assert lib.pkv_decoder_create(ctypes.byref(d)) is None
    assert b"workspace" in lib.pkv_last_error()
    assert lib.pkv_decoder_step(None, None, 1, None, None) == E_NULL
    assert lib.pkv_decoder_block_manager(None) is None
    lib.pkv_decoder_destroy(None)


@pytest.mark.parametrize("n,count", [(256, 1), (256, 8), (256, 32), (256, 77), (256, 256), (40, 7), (32, 32)])
def test_cu_mask_layouts(lib, n, count):
    for layout in ("first", "spread"):
        m = pkv.cu_mask(n, count, layout)
        bits = [i for i in range(32 * m.size) if (int(m[i // 32]) >> (i % 32)) & 1]
        assert len(bits) == count and max(bits) < n
        if layout == "first":
            assert bits == list(range(count))
        else:
            assert bits == [j * n // count for j in range(count)]
            gaps = np.diff(bits + [bits[0] + n])
            assert gaps.max() - gaps.min() <= 1            # as even as integers allow


def test_cu_mask_and_stream_validation(lib):
    m = (ctypes.c_uint32 * 8)()
    assert lib.pkv_cu_mask(256, 0, 1, ctypes.cast(m, ctypes.c_void_p), 8) == E_ARG
    assert lib.pkv_cu_mask(256, 257, 1, ctypes.cast(m, ctypes.c_void_p), 8) == E_ARG
    assert lib.pkv_cu_mask(300, 8, 1, ctypes.cast(m, ctypes.c_void_p), 8) == E_ARG
    assert lib.pkv_cu_mask(256, 8, 2, ctypes.cast(m, ctypes.c_void_p), 8) == E_ARG
    assert lib.pkv_cu_mask(256, 8, 1, None, 8) == E_NULL
    zero = (ctypes.c_uint32 * 8)()
    out = ctypes.c_void_p()
    assert lib.pkv_stream_create_cu_masked(ctypes.cast(zero, ctypes.c_void_p), 8, ctypes.byref(out)) == E_ARG
    assert lib.pkv_stream_create_cu_masked(None, 8, ctypes.byref(out)) == E_NULL
    assert lib.pkv_stream_destroy(None) == E_NULL


def test_fp8_entry_point_validation(lib):
    P = ctypes.c_void_p
    # (q_dtype, out, q, qrs, kp, vp, ks, vs, bt, bts, ctx, B, H_q, H_kv, D, bs, nb, maxc, scale, P, ws, wsb, stream)
    base = [1, FAKE, FAKE, 8 * 128, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 2, 8, 8, 128, 16, 64, 100, 0.1, 0,
            None, 0, None]
    def call(kw):
        a = list(base)
        for k, v in kw.items():
            a[k] = v
        return lib.pkv_paged_decode_attention_fp8(*a)
    assert call({0: 9}) == E_UNSUP                 # q dtype
    assert call({6: None}) == E_NULL               # k_scale
    assert call({7: FAKE + 2}) == E_ARG            # v_scale not 4-byte aligned
    assert call({4: FAKE + 8}) == E_ARG            # pool not 16-byte aligned
    assert call({14: 96}) == E_UNSUP               # D
    assert call({11: 0}) == OK                     # B == 0: nothing to do
    # append: (src_dtype, k_new, v_new, rs, kp, vp, ks, vs, bt, bts, pos, B, H_kv, D, bs, nb, stream)
    app = [1, FAKE, FAKE, 8 * 128, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 2, 8, 128, 16, 64, None]
    def append(kw):
        a = list(app)
        for k, v in kw.items():
            a[k] = v
        return lib.pkv_kv_append_fp8(*a)
    assert append({0: 5}) == E_UNSUP
    assert append({7: None}) == E_NULL
    assert append({3: 100}) == E_ARG               # row stride below H_kv * D
    assert append({11: 0}) == OK
    assert lib.pkv_status_string(E_UNSUP) == b"PKV_ERR_UNSUPPORTED"


def test_status_codes_of_the_contract(lib):
    """The boundary's status values: aliased appends -5, HIP errors -6, then the block manager's."""
    names = {-5: b"PKV_ERR_ALIASED_APPEND", -6: b"PKV_ERR_HIP", -7: b"PKV_ERR_OUT_OF_BLOCKS", -8: b"PKV_ERR_SEQUENCE"}
    for code, name in names.items():
        assert lib.pkv_status_string(code) == name
    assert (pkv.PKV_ERR_ALIASED_APPEND, pkv.PKV_ERR_HIP, pkv.PKV_ERR_OUT_OF_BLOCKS, pkv.PKV_ERR_SEQUENCE) == (-5, -6, -7, -8)


def test_check_step_metadata_host_validation(lib):
    """Argument errors are reported before anything touches the GPU."""
    E_ARG = -2
    # exactly one of context_lens and positions
    assert lib.pkv_check_step_metadata(FAKE, 4, None, None, 2, 16, 8, 0, None) == E_ARG
    assert lib.pkv_check_step_metadata(FAKE, 4, FAKE, FAKE, 2, 16, 8, 0, None) == E_ARG
    assert b"exactly one" in lib.pkv_last_error()
    for bt_stride, bs, nb, mx, B in ((0, 16, 8, 0, 2), (4, 0, 8, 0, 2), (4, 16, 0, 0, 2), (4, 16, 8, -1, 2),
                                     (4, 16, 8, 0, -1)):
        assert lib.pkv_check_step_metadata(FAKE, bt_stride, None, FAKE, B, bs, nb, mx, None) == E_ARG
    assert lib.pkv_check_step_metadata(None, 4, None, FAKE, 2, 16, 8, 0, None) == -1     # PKV_ERR_NULL
    assert lib.pkv_check_step_metadata(FAKE, 4, None, FAKE, 0, 16, 8, 0, None) == 0      # B = 0: nothing to check
