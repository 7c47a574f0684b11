"""The library's host block manager (pkv_bm_*) against the oracle's, operation
by operation on seeded streams: same return values, same error kinds, same
block tables, lengths, reference counts and free counts after every call
(bit-exact; both hand out the free block with the smallest key).  Also the
brute-force content model run on the library alone at larger sizes, and the
argument checks of the C ABI.  Host code only: no GPU needed."""
import ctypes

import numpy as np
import pytest

import paged_kv_decode_blocks_amd as pkv
from oracle.block_manager import BlockManager as OracleBM
from oracle.block_manager import BlockManagerError
from tests.bm_model import ContentModel, apply_op, random_ops

KIND = {pkv.PKV_ERR_OUT_OF_BLOCKS: "out_of_blocks", pkv.PKV_ERR_SEQUENCE: "sequence",
        pkv.PKV_ERR_INVALID_ARG: "invalid"}


@pytest.fixture(scope="module", autouse=True)
def lib():
    return pkv.load_library()


def outcome(model, op, live, bt_stride):
    try:
        return ("ok", apply_op(model, op, live, bt_stride))
    except BlockManagerError as e:
        return ("err", e.kind)
    except pkv.PkvError as e:
        return ("err", KIND.get(e.status, e.status))


def same_state(ora: OracleBM, lib: pkv.BlockManager, live):
    assert lib.num_sequences() == ora.num_sequences() == len(live)
    assert lib.num_free_blocks() == ora.num_free_blocks()
    for s in live:
        assert list(lib.block_table(s)) == ora.block_table(s), s
        assert lib.sequence_length(s) == ora.sequence_length(s), s
    for b in range(ora.n_blocks):
        assert lib.block_refcount(b) == ora.block_refcount(b), b


@pytest.mark.parametrize("seed,n_blocks,bs,shuffle,bt_stride", [
    (11, 24, 4, 0, 64), (12, 20, 16, 0, 64), (13, 40, 1, 77, 256), (14, 30, 8, 5, 64), (15, 30, 4, 2**63 + 9, 5),
])
def test_matches_oracle_op_by_op(seed, n_blocks, bs, shuffle, bt_stride):
    ora, lib = OracleBM(n_blocks, bs, shuffle), pkv.BlockManager(n_blocks, bs, shuffle)
    m_ora, m_lib = ContentModel(ora, n_blocks, bs), ContentModel(lib, n_blocks, bs)
    live_ora, live_lib = [], []
    kinds = set()
    for op in random_ops(seed, 350, max_prompt=3 * bs):
        a = outcome(m_ora, op, live_ora, bt_stride)
        b = outcome(m_lib, op, live_lib, bt_stride)
        assert a == b, (op, a, b)
        kinds.add(a[0] if a[0] == "ok" else a[1])
        assert live_ora == live_lib
        same_state(ora, lib, live_lib)
        m_lib.check()
    assert "ok" in kinds and "out_of_blocks" in kinds


@pytest.mark.parametrize("seed,shuffle", [(21, 0), (22, 123456789)])
def test_content_model_large_pool(seed, shuffle):
    """The library alone at a realistic block size and a pool that fills up."""
    n_blocks, bs = 300, 16
    lib = pkv.BlockManager(n_blocks, bs, shuffle)
    model = ContentModel(lib, n_blocks, bs)
    live, fails = [], 0
    for i, op in enumerate(random_ops(seed, 1500, max_prompt=400)):
        try:
            apply_op(model, op, live, bt_stride=128, max_live=40)
        except pkv.PkvError as e:
            assert e.status in (pkv.PKV_ERR_OUT_OF_BLOCKS, pkv.PKV_ERR_INVALID_ARG), e
            fails += 1
        if i % 25 == 0:
            model.check()
    model.check()
    assert fails > 0
    for s in list(live):
        lib.free_sequence(s)
    assert lib.num_free_blocks() == n_blocks and lib.num_sequences() == 0


def test_batch_error_kinds_match_and_change_nothing():
    for mk in (lambda: OracleBM(6, 4), lambda: pkv.BlockManager(6, 4)):
        bm = mk()
        bm.add_sequence(1, 4)
        bm.add_sequence(2, 3)
        before = (list(bm.block_table(1)), list(bm.block_table(2)), bm.num_free_blocks())
        for ids, stride, kind in [([1, 1], 4, "invalid"), ([1, 9], 4, "sequence"), ([1, 2], 1, "invalid")]:
            with pytest.raises((BlockManagerError, pkv.PkvError)) as e:
                bm.append_batch(ids, stride)
            got = e.value.kind if isinstance(e.value, BlockManagerError) else KIND[e.value.status]
            assert got == kind, (ids, stride, got)
            assert (list(bm.block_table(1)), list(bm.block_table(2)), bm.num_free_blocks()) == before
        bm.add_sequence(3, 16)                    # takes the last 4 blocks
        with pytest.raises((BlockManagerError, pkv.PkvError)) as e:
            bm.append_batch([2, 1], 4)            # 2 fits in its block, 1 needs a fresh one: none free
        got = e.value.kind if isinstance(e.value, BlockManagerError) else KIND[e.value.status]
        assert got == "out_of_blocks"
        assert bm.sequence_length(2) == 3 and bm.sequence_length(1) == 4


def test_batch_copy_pointers_required_only_when_copying(lib):
    bm = pkv.BlockManager(8, 4)
    bm.add_sequence(1, 2)
    ids = np.array([1], dtype=np.int64)
    tables = np.zeros((1, 4), dtype=np.int32)
    pos = np.zeros(1, dtype=np.int32)
    P = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert lib.pkv_bm_append_batch(bm._h, P(ids), 1, P(tables), 4, P(pos), None, None, None) == 0
    bm.fork(1, 2)
    before = bm.sequence_length(1)
    assert lib.pkv_bm_append_batch(bm._h, P(ids), 1, P(tables), 4, P(pos), None, None, None) == pkv.PKV_ERR_INVALID_ARG
    assert bm.sequence_length(1) == before and bm.num_free_blocks() == 7


def test_null_and_bad_arguments(lib):
    assert lib.pkv_bm_create(0, 16, 0) is None
    assert lib.pkv_bm_create(4, 0, 0) is None
    assert lib.pkv_bm_add_sequence(None, 1, 1) == -1
    assert lib.pkv_bm_num_free_blocks(None) == -1
    assert lib.pkv_bm_num_sequences(None) == -1
    assert lib.pkv_bm_sequence_length(None, 1) == -1
    lib.pkv_bm_destroy(None)
    bm = pkv.BlockManager(4, 16)
    assert bm.block_refcount(-1) == -1 and bm.block_refcount(4) == -1 and bm.block_refcount(3) == 0
    assert bm.sequence_length(5) == -1
    with pytest.raises(pkv.PkvError) as e:
        bm.block_table(5)
    assert e.value.status == pkv.PKV_ERR_SEQUENCE
    assert lib.pkv_status_string(pkv.PKV_ERR_OUT_OF_BLOCKS) == b"PKV_ERR_OUT_OF_BLOCKS"
    assert lib.pkv_status_string(pkv.PKV_ERR_SEQUENCE) == b"PKV_ERR_SEQUENCE"


def test_batch_tables_reads_without_changing():
    bm = pkv.BlockManager(10, 16, 7)
    bm.add_sequence(4, 40)
    bm.add_sequence(9, 0)
    tables, lens = bm.batch_tables([9, 4], 5)
    assert list(lens) == [0, 40]
    assert list(tables[0]) == [-1] * 5
    assert list(tables[1][:3]) == list(bm.block_table(4)) and list(tables[1][3:]) == [-1, -1]
    assert bm.num_free_blocks() == 7
    with pytest.raises(pkv.PkvError):
        bm.batch_tables([4], 2)
