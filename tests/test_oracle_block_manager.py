"""Pins of the oracle's block manager against things fixed outside it: a
lifecycle worked by hand from the paging rules, the published SplitMix64
outputs, a brute-force content model (every sequence reads back its own
tokens), pool capacity with no fragmentation, all-or-nothing failures, and
planted mistakes that these pins must catch."""
import json
import os

import pytest

from oracle.block_manager import BlockManager, BlockManagerError, splitmix64
from tests.bm_model import ContentModel, apply_op, random_ops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_reference_outputs.json")


def test_splitmix64_matches_published_outputs():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        want = [int(h, 16) for h in c["outputs_hex"]] if "outputs_hex" in c else c["outputs"]
        assert splitmix64(c["seed"], len(want)) == want


def test_seeded_order_follows_published_outputs():
    # seed 1234567 draws 6457827717110365317, 3203168211198807973, 9817491932198370423
    # for blocks 0, 1, 2: ascending draws hand out block 1, then 0, then 2.
    bm = BlockManager(3, 4, shuffle_seed=1234567)
    bm.add_sequence(7, 12)
    assert bm.block_table(7) == [1, 0, 2]


def test_hand_worked_lifecycle():
    """Pool of 6 blocks of 4 tokens, ascending order; each step worked out by
    hand from: a block per started logical block, reclaim when unmapped, whole
    blocks shared by a common prefix, copy before writing a shared partial block."""
    bm = BlockManager(6, 4)
    bm.add_sequence(1, 5)                       # tokens 0..4 -> blocks 0, 1
    assert bm.block_table(1) == [0, 1]
    bm.add_sequence(2, 3)                       # -> block 2
    assert bm.block_table(2) == [2] and bm.num_free_blocks() == 3
    bm.fork(1, 3)                               # 3 maps 0, 1 as well
    assert bm.block_table(3) == [0, 1] and bm.refcount(0) == 2 and bm.refcount(1) == 2
    assert bm.append_token(1) == (5, 1, 3)      # slot 1 of shared block 1: copy it to 3 first
    assert bm.block_table(1) == [0, 3] and bm.refcount(1) == 1 and bm.block_table(3) == [0, 1]
    assert bm.append_token(3) == (5, -1, -1)    # block 1 is now 3's alone: write in place
    assert bm.append_token(1) == (6, -1, -1)
    assert bm.append_token(1) == (7, -1, -1)
    assert bm.append_token(1) == (8, -1, -1)    # starts logical block 2 -> block 4
    assert bm.block_table(1) == [0, 3, 4] and bm.free_blocks() == [5]
    bm.free_sequence(2)                         # block 2 back to the pool
    assert bm.free_blocks() == [2, 5]
    assert bm.add_sequence_shared(4, 9, 1, 8) == 8   # two whole blocks of 1, one fresh (2)
    assert bm.block_table(4) == [0, 3, 2] and bm.refcount(0) == 3 and bm.refcount(3) == 2
    assert bm.append_token(4) == (9, -1, -1)    # block 2 is private
    with pytest.raises(BlockManagerError) as e:
        bm.add_sequence(5, 5)                   # needs 2 blocks, 1 free
    assert e.value.kind == "out_of_blocks"
    assert bm.free_blocks() == [5] and 5 not in bm.tables
    bm.free_sequence(1)                         # block 4 freed; 0 and 3 still mapped
    assert bm.free_blocks() == [4, 5] and bm.refcount(0) == 2 and bm.refcount(3) == 1
    bm.free_sequence(3)
    assert bm.free_blocks() == [1, 4, 5]
    bm.free_sequence(4)
    assert bm.num_free_blocks() == 6


def test_batch_step_worked_by_hand():
    bm = BlockManager(8, 4)
    bm.add_sequence(10, 6)                      # blocks 0, 1 (slots 0, 1 of block 1 used)
    bm.fork(10, 11)
    bm.add_sequence(12, 4)                      # block 2, full
    tables, positions, copies = bm.append_batch([11, 10, 12], 3)
    # 11 writes first into shared block 1: copy to 3; then 10 has block 1 alone; 12 starts block 4
    assert copies == [(1, 3)]
    assert positions == [6, 6, 4]
    assert tables == [[0, 3, -1], [0, 1, -1], [2, 4, -1]]


@pytest.mark.parametrize("seed,n_blocks,bs,shuffle", [(1, 24, 4, 0), (2, 20, 16, 0), (3, 40, 1, 99), (4, 30, 8, 5)])
def test_content_model_random_streams(seed, n_blocks, bs, shuffle):
    bm = BlockManager(n_blocks, bs, shuffle_seed=shuffle)
    model = ContentModel(bm, n_blocks, bs)
    live, ok, failed = [], 0, 0
    for op in random_ops(seed, 400, max_prompt=3 * bs):
        snapshot = (dict(bm.tables), dict(bm.lengths))
        try:
            apply_op(model, op, live, bt_stride=1 << 20)
            ok += 1
        except BlockManagerError as e:
            assert e.kind == "out_of_blocks", e
            assert (bm.tables, bm.lengths) == snapshot      # nothing changed
            failed += 1
        model.check()
    assert ok > 150 and failed > 0


def test_capacity_without_fragmentation():
    """Any free block serves any sequence: after scattered frees, one sequence
    takes exactly all free blocks' tokens, and one more token fails."""
    bm = BlockManager(30, 4, shuffle_seed=3)
    for s in range(10):
        bm.add_sequence(s, 4 * (1 + s % 3) - (s % 2))
    for s in (1, 4, 5, 8):
        bm.free_sequence(s)
    free = bm.num_free_blocks()
    bm.add_sequence(100, 4 * free)
    assert bm.num_free_blocks() == 0
    with pytest.raises(BlockManagerError):
        bm.append_token(100)
    bm.free_sequence(100)
    assert bm.num_free_blocks() == free


def test_errors():
    bm = BlockManager(4, 4)
    bm.add_sequence(1, 3)
    for call, kind in [(lambda: bm.add_sequence(1, 1), "sequence"), (lambda: bm.fork(9, 2), "sequence"),
                       (lambda: bm.fork(1, 1), "sequence"), (lambda: bm.append_token(9), "sequence"),
                       (lambda: bm.free_sequence(9), "sequence"), (lambda: bm.add_sequence(2, -1), "invalid"),
                       (lambda: bm.add_sequence_shared(2, 2, 1, 3), "invalid"),
                       (lambda: bm.add_sequence_shared(2, 9, 1, 4), "invalid"),
                       (lambda: bm.append_batch([1, 1], 4), "invalid"),
                       (lambda: bm.append_batch([1], 0), "invalid")]:
        with pytest.raises(BlockManagerError) as e:
            call()
        assert e.value.kind == kind
        assert bm.tables == {1: [0]} and bm.lengths == {1: 3}


# -- planted mistakes: each must be caught by the pins above -------------------

class NoCopyOnWrite(BlockManager):
    def _append(self, seq_id):
        pos = self.lengths[seq_id]
        if pos % self.block_size == 0:
            self.tables[seq_id].append(self._take_block())
        self.lengths[seq_id] = pos + 1
        return pos, -1, -1


class SharesPartialPrefixBlock(BlockManager):
    def add_sequence_shared(self, seq_id, num_tokens, prefix_id, prefix_tokens):
        whole = -(-prefix_tokens // self.block_size)            # rounds up: shares a partly used block
        self.tables[seq_id] = list(self.tables[prefix_id][:whole])
        self.lengths[seq_id] = num_tokens
        for _ in range(self._blocks_for(num_tokens) - whole):
            self.tables[seq_id].append(self._take_block())
        return whole * self.block_size if whole * self.block_size <= prefix_tokens else (prefix_tokens // self.block_size) * self.block_size


class LargestKeyFirst(BlockManager):
    def _take_block(self):
        free = self.free_blocks()
        if not free:
            raise BlockManagerError("out_of_blocks", "no free block")
        return max(free, key=lambda b: self.key[b])


class NoBlockAtBoundary(BlockManager):
    def _append(self, seq_id):
        pos = self.lengths[seq_id]
        if pos % self.block_size == 0 and pos > 0:
            self.lengths[seq_id] = pos + 1                       # forgets the new block
            return pos, -1, -1
        return super()._append(seq_id)


def _stream_catches(cls):
    for seed in range(1, 6):
        bm = cls(24, 4)
        model = ContentModel(bm, 24, 4)
        live = []
        try:
            for op in random_ops(seed, 300, max_prompt=12):
                try:
                    apply_op(model, op, live, bt_stride=1 << 20)
                except BlockManagerError:
                    pass
                model.check()
        except (AssertionError, IndexError):
            return True
    return False


@pytest.mark.parametrize("cls", [NoCopyOnWrite, SharesPartialPrefixBlock, NoBlockAtBoundary])
def test_planted_mistake_caught_by_content_model(cls):
    assert _stream_catches(cls)


def test_planted_order_mistake_caught_by_worked_example():
    with pytest.raises(AssertionError):
        bm = LargestKeyFirst(3, 4, shuffle_seed=1234567)
        bm.add_sequence(7, 12)
        assert bm.block_table(7) == [1, 0, 2]
    with pytest.raises(AssertionError):
        bm = LargestKeyFirst(6, 4)
        bm.add_sequence(1, 5)
        assert bm.block_table(1) == [0, 1]
