"""Brute-force content model and seeded operation streams for block-manager tests.

The model holds no allocation logic of its own.  It keeps, per live sequence,
the list of token labels the sequence logically holds, and a simulated pool
memory (block, slot) -> label that is written only through the block tables a
manager hands out: prompt tokens when a sequence is added, the copy-on-write
pairs the manager reports, and each appended token.  After every operation
each live sequence must read its own labels back through its table, and the
manager's bookkeeping must agree with the tables it reports.  A manager that
writes into a block another sequence still maps, frees a block too early,
hands out a mapped block or mis-sizes a table fails this check.

Managers are driven through one interface (the oracle's and the library's
share method names): add_sequence, add_sequence_shared -> shared tokens,
fork, append_token -> (position, cow_src, cow_dst), free_sequence,
block_table, sequence_length, num_free_blocks, and block_refcount.
"""
from __future__ import annotations

from collections import Counter

import numpy as np


class ContentModel:
    def __init__(self, manager, n_blocks: int, block_size: int):
        self.m = manager
        self.n_blocks = n_blocks
        self.bs = block_size
        self.labels = {}        # seq -> list of token labels
        self.memory = {}        # (block, slot) -> label
        self.fresh = 0

    def _label(self, seq):
        self.fresh += 1
        return ("tok", seq, self.fresh)

    def _write(self, seq, pos, label):
        table = list(self.m.block_table(seq))
        self.memory[(int(table[pos // self.bs]), pos % self.bs)] = label

    def _copy(self, src, dst):
        for slot in range(self.bs):
            if (src, slot) in self.memory:
                self.memory[(dst, slot)] = self.memory[(src, slot)]
            else:
                self.memory.pop((dst, slot), None)

    # -- operations (exceptions from the manager propagate unchanged) --------
    def add_sequence(self, seq, n):
        self.m.add_sequence(seq, n)
        self.labels[seq] = [self._label(seq) for _ in range(n)]
        for p in range(n):
            self._write(seq, p, self.labels[seq][p])

    def add_sequence_shared(self, seq, n, prefix, prefix_tokens):
        shared = self.m.add_sequence_shared(seq, n, prefix, prefix_tokens)
        assert shared % self.bs == 0 and 0 <= shared <= prefix_tokens
        own = list(self.labels[prefix][:prefix_tokens]) + [self._label(seq) for _ in range(n - prefix_tokens)]
        self.labels[seq] = own
        for p in range(shared, n):          # the caller writes everything it did not get for free
            self._write(seq, p, own[p])
        return shared

    def fork(self, parent, child):
        self.m.fork(parent, child)
        self.labels[child] = list(self.labels[parent])

    def append_token(self, seq):
        pos, src, dst = self.m.append_token(seq)
        assert pos == len(self.labels[seq])
        if src >= 0:
            self._copy(int(src), int(dst))
        label = self._label(seq)
        self.labels[seq].append(label)
        self._write(seq, pos, label)
        return pos, src, dst

    def apply_batch(self, seq_ids, tables, positions, cow_pairs):
        """Replay a batch step: copies first, then every sequence's new token."""
        for src, dst in cow_pairs:
            self._copy(int(src), int(dst))
        for b, seq in enumerate(seq_ids):
            assert positions[b] == len(self.labels[seq])
            label = self._label(seq)
            self.labels[seq].append(label)
            p = int(positions[b])
            self.memory[(int(tables[b][p // self.bs]), p % self.bs)] = label

    def free_sequence(self, seq):
        self.m.free_sequence(seq)
        del self.labels[seq]

    # -- the check ------------------------------------------------------------
    def check(self):
        refs = Counter()
        for seq, labels in self.labels.items():
            table = [int(b) for b in self.m.block_table(seq)]
            assert self.m.sequence_length(seq) == len(labels), seq
            assert len(table) == -(-len(labels) // self.bs), (seq, table, len(labels))
            assert len(set(table)) == len(table), (seq, table)
            for b in table:
                assert 0 <= b < self.n_blocks
            refs.update(table)
            for p, want in enumerate(labels):
                got = self.memory.get((table[p // self.bs], p % self.bs))
                assert got == want, (seq, p, got, want)
        for b in range(self.n_blocks):
            assert self.m.block_refcount(b) == refs[b], (b, self.m.block_refcount(b), refs[b])
        assert self.m.num_free_blocks() == self.n_blocks - len(refs)


def random_ops(seed: int, n_ops: int, max_prompt: int):
    """A seeded stream of operations over sequence ids 0, 1, 2, ...  Arguments
    that name live sequences are kept as draws in [0, 1) and resolved against
    the live set when the operation is applied, so every manager in a parity
    test sees the same stream."""
    rng = np.random.default_rng(seed)
    for i in range(n_ops):
        r = rng.random()
        u = float(rng.random())
        v = float(rng.random())
        n = int(rng.integers(0, max_prompt + 1))
        if r < 0.12:
            yield ("add", i, n)
        elif r < 0.18:
            yield ("add_shared", i, n, u, v)
        elif r < 0.26:
            yield ("fork", i, u)
        elif r < 0.36:
            yield ("free", u)
        elif r < 0.46:
            yield ("batch", u, v)
        else:
            yield ("append", u)


def pick(live, u):
    return live[int(u * len(live))]


def apply_op(model: ContentModel, op, live: list, bt_stride: int, max_live: int = 12):
    """Apply one operation through the model; returns what the manager returned
    (None for an op skipped because its preconditions do not hold).  `live` is
    updated only when the manager call succeeds."""
    kind = op[0]
    if kind in ("add", "add_shared", "fork") and len(live) >= max_live:
        kind, op = "free", ("free", op[-1] if isinstance(op[-1], float) else 0.5)
    if kind == "add":
        model.add_sequence(op[1], op[2])
        live.append(op[1])
        return ("add",)
    if not live:
        return None
    if kind == "add_shared":
        _, sid, n, u, v = op
        prefix = pick(live, u)
        plen = model.m.sequence_length(prefix)
        pt = int(v * (plen + 1))
        n = max(n, pt)
        shared = model.add_sequence_shared(sid, n, prefix, pt)
        live.append(sid)
        return ("add_shared", shared)
    if kind == "fork":
        model.fork(pick(live, op[2]), op[1])
        live.append(op[1])
        return ("fork",)
    if kind == "free":
        sid = pick(live, op[1])
        model.free_sequence(sid)
        live.remove(sid)
        return ("free",)
    if kind == "append":
        return ("append",) + tuple(int(x) for x in model.append_token(pick(live, op[1])))
    if kind == "batch":
        _, u, v = op
        k = 1 + int(u * len(live))
        start = int(v * len(live))
        ids = [live[(start + j) % len(live)] for j in range(k)]
        tables, positions, cow = model.m.append_batch(ids, bt_stride)
        tables = [[int(x) for x in row] for row in tables]
        positions = [int(x) for x in positions]
        cow = [(int(a), int(b)) for a, b in cow]
        model.apply_batch(ids, tables, positions, cow)
        return ("batch", tables, positions, cow)
    raise ValueError(kind)
