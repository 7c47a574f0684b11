"""Plain reference of the KV pool's paging lifecycle (block allocation, sharing, reclaim).

TEST INFRASTRUCTURE ONLY: the tests may import this module; the product
library never does, and this module never imports the product library.

What it follows
---------------
"从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2: the KV store
is cut into fixed-size physical blocks; each request keeps a page table from
its logical blocks to physical ones, which need not be contiguous; a block is
requested only when a newly generated token needs one, and when a request ends
all its blocks go straight back to one global pool for any other request.
Section 2.3: requests with a common system prompt map the same physical
blocks, so that prefix's KV is stored once.

Readings where the page is silent (each one is also a rule of the C ABI):
  * sharing is counted per block; a block is free exactly when no live
    sequence maps it;
  * a prefix is shared in whole blocks only; a sequence forked from another
    shares every block, its partly filled last block included;
  * a shared block is never written: a sequence about to write into a partly
    filled block that another live sequence maps first moves to a fresh block
    holding a copy of it (copy-on-write); the copy is reported as (old, new);
  * allocation takes the free block with the smallest key; key(i) = i, or with
    a nonzero seed the pair (splitmix64 output number i + 1 for that seed, i);
  * a call that cannot complete raises and changes nothing; a batch step
    reports a bad member (unknown, repeated, or a table too wide) before it
    reports that the pool ran out.

Written for clarity, not speed: the free set is recomputed by a scan, and a
batch step is tried on a deep copy and kept only if every member succeeds.
"""
from __future__ import annotations

import copy
from typing import Dict, List, Optional, Sequence, Tuple

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, count: int) -> List[int]:
    """The first `count` outputs of SplitMix64 started from `seed` (Steele, Lea
    and Flood, OOPSLA 2014): the state advances by the golden-ratio gamma and
    each output is the state passed through the 64-bit mix."""
    out, state = [], seed & _MASK64
    for _ in range(count):
        state = (state + _GOLDEN_GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


class BlockManagerError(Exception):
    """kind is one of 'out_of_blocks', 'sequence', 'invalid'."""

    def __init__(self, kind: str, message: str):
        super().__init__(message)
        self.kind = kind


class BlockManager:
    def __init__(self, n_blocks: int, block_size: int, shuffle_seed: int = 0):
        if n_blocks <= 0 or block_size <= 0:
            raise BlockManagerError("invalid", "sizes must be positive")
        self.n_blocks = n_blocks
        self.block_size = block_size
        if shuffle_seed == 0:
            self.key = list(range(n_blocks))
        else:
            draws = splitmix64(shuffle_seed, n_blocks)
            self.key = [(draws[i], i) for i in range(n_blocks)]
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}

    # -- state ------------------------------------------------------------
    def refcount(self, block: int) -> int:
        return sum(t.count(block) for t in self.tables.values())

    def block_refcount(self, block: int) -> int:
        return self.refcount(block) if 0 <= block < self.n_blocks else -1

    def num_sequences(self) -> int:
        return len(self.tables)

    def free_blocks(self) -> List[int]:
        used = set()
        for t in self.tables.values():
            used.update(t)
        return [b for b in range(self.n_blocks) if b not in used]

    def num_free_blocks(self) -> int:
        return len(self.free_blocks())

    def _take_block(self) -> int:
        free = self.free_blocks()
        if not free:
            raise BlockManagerError("out_of_blocks", "no free block")
        return min(free, key=lambda b: self.key[b])

    def _blocks_for(self, n_tokens: int) -> int:
        return -(-n_tokens // self.block_size)

    def _need(self, seq_id: int):
        if seq_id not in self.tables:
            raise BlockManagerError("sequence", f"sequence {seq_id} does not exist")

    def _new_id(self, seq_id: int):
        if seq_id in self.tables:
            raise BlockManagerError("sequence", f"sequence {seq_id} already exists")

    # -- lifecycle (each call is all-or-nothing: work on a copy, then keep it) --
    def _atomic(self, fn):
        trial = copy.deepcopy(self)
        result = fn(trial)
        self.__dict__.update(trial.__dict__)
        return result

    def add_sequence(self, seq_id: int, num_tokens: int) -> None:
        def run(m):
            if num_tokens < 0:
                raise BlockManagerError("invalid", "negative length")
            m._new_id(seq_id)
            m.tables[seq_id] = []
            m.lengths[seq_id] = num_tokens
            for _ in range(m._blocks_for(num_tokens)):
                m.tables[seq_id].append(m._take_block())
        self._atomic(run)

    def add_sequence_shared(self, seq_id: int, num_tokens: int, prefix_id: int, prefix_tokens: int) -> int:
        def run(m):
            m._need(prefix_id)
            m._new_id(seq_id)
            if not 0 <= prefix_tokens <= min(num_tokens, m.lengths[prefix_id]):
                raise BlockManagerError("invalid", "prefix_tokens out of range")
            whole = prefix_tokens // m.block_size
            m.tables[seq_id] = list(m.tables[prefix_id][:whole])
            m.lengths[seq_id] = num_tokens
            for _ in range(m._blocks_for(num_tokens) - whole):
                m.tables[seq_id].append(m._take_block())
            return whole * m.block_size
        return self._atomic(run)

    def fork(self, parent_id: int, child_id: int) -> None:
        def run(m):
            m._need(parent_id)
            m._new_id(child_id)
            m.tables[child_id] = list(m.tables[parent_id])
            m.lengths[child_id] = m.lengths[parent_id]
        self._atomic(run)

    def _append(self, seq_id: int) -> Tuple[int, int, int]:
        self._need(seq_id)
        pos = self.lengths[seq_id]
        table = self.tables[seq_id]
        src = dst = -1
        if pos % self.block_size == 0:                 # the token starts a new logical block
            table.append(self._take_block())
        elif self.refcount(table[-1]) > 1:             # partly filled block that another sequence maps
            src = table[-1]
            dst = self._take_block()
            table[-1] = dst
        self.lengths[seq_id] = pos + 1
        return pos, src, dst

    def append_token(self, seq_id: int) -> Tuple[int, int, int]:
        """Returns (position, cow_src, cow_dst); the copy pair is (-1, -1) when none is needed."""
        return self._atomic(lambda m: m._append(seq_id))

    def append_batch(self, seq_ids: Sequence[int], bt_stride: int):
        """One token for each sequence, in order.  Returns (tables [B][bt_stride]
        padded with -1, positions [B], list of (cow_src, cow_dst))."""
        def run(m):
            seen = set()
            for s in seq_ids:                          # argument errors first, member by member
                m._need(s)
                if s in seen:
                    raise BlockManagerError("invalid", "a sequence appears twice")
                seen.add(s)
                if m._blocks_for(m.lengths[s] + 1) > bt_stride:
                    raise BlockManagerError("invalid", "table wider than bt_stride")
            positions, copies = [], []
            for s in seq_ids:
                pos, src, dst = m._append(s)
                positions.append(pos)
                if src >= 0:
                    copies.append((src, dst))
            tables = []
            for s in seq_ids:
                t = m.tables[s]
                if len(t) > bt_stride:
                    raise BlockManagerError("invalid", "table wider than bt_stride")
                tables.append(t + [-1] * (bt_stride - len(t)))
            return tables, positions, copies
        return self._atomic(run)

    def free_sequence(self, seq_id: int) -> None:
        def run(m):
            m._need(seq_id)
            del m.tables[seq_id]
            del m.lengths[seq_id]
        self._atomic(run)

    # -- queries ------------------------------------------------------------
    def sequence_length(self, seq_id: int) -> int:
        return self.lengths.get(seq_id, -1)

    def block_table(self, seq_id: int) -> List[int]:
        self._need(seq_id)
        return list(self.tables[seq_id])

    def batch_tables(self, seq_ids: Sequence[int], bt_stride: int):
        tables, lens = [], []
        for s in seq_ids:
            t = self.block_table(s)
            if len(t) > bt_stride:
                raise BlockManagerError("invalid", "table wider than bt_stride")
            tables.append(t + [-1] * (bt_stride - len(t)))
            lens.append(self.lengths[s])
        return tables, lens


def copy_blocks(k_pool, v_pool, pairs: Sequence[Tuple[int, int]]) -> None:
    """Apply copy-on-write pairs to numpy pools [n_blocks][H_kv][bs][D]: block dst takes src's contents."""
    for src, dst in pairs:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]
