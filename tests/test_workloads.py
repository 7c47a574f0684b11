"""Seeded generator and byte accounting (CPU only)."""
import hashlib
import json
import os

import numpy as np
import pytest

from workloads import (CONFIGS, NAN_BITS, draw_lengths, get_config, kv_bytes_per_token, make_workload, step_bytes,
                       to_storage)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _digest(w):
    h = hashlib.sha256()
    for a in (w.context_lens, w.block_tables, w.q, w.k_pool, w.v_pool):
        h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    if w.k_new is not None:
        h.update(w.k_new.tobytes())
        h.update(w.v_new.tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_same_seed_same_bytes(name):
    cfg = get_config(name, B=4, lengths=("uniform", 1, 80)) if name != "c1" else get_config(name)
    assert _digest(make_workload(cfg, seed=3)) == _digest(make_workload(cfg, seed=3))
    assert _digest(make_workload(cfg, seed=3)) != _digest(make_workload(cfg, seed=4))


def _is_poison(a, dtype):
    bits = a.view(np.uint32 if dtype == "f32" else np.uint16)
    return bits == NAN_BITS[dtype]


@pytest.mark.parametrize("name", ["c1", "c3"])
def test_poison_layout(name):
    cfg = get_config(name) if name == "c1" else get_config(name, B=6)
    w = make_workload(cfg, seed=1)
    bs = cfg.block_size
    used = set()
    for b in range(cfg.B):
        hist = int(w.history_lens[b])
        nb = -(-int(w.context_lens[b]) // bs)
        ids = w.block_tables[b, :nb]
        assert np.all(w.block_tables[b, nb:] == -1)
        used.update(int(i) for i in ids)
        for pool in (w.k_pool, w.v_pool):
            seq = pool[ids].transpose(0, 2, 1, 3).reshape(nb * bs, cfg.H_kv, cfg.D)
            assert not np.any(_is_poison(seq[:hist], cfg.dtype))
            assert np.all(_is_poison(seq[hist:], cfg.dtype))       # incl. the append slot
    assert len(used) == sum(-(-int(n) // bs) for n in w.context_lens)   # no block shared
    unused = np.array(sorted(set(range(w.n_blocks)) - used), dtype=np.int64)
    if unused.size:
        assert np.all(_is_poison(w.k_pool[unused], cfg.dtype))


def test_config_shapes_and_lengths():
    w = make_workload(get_config("c1"))
    assert list(w.context_lens) == [5, 37] and list(w.positions) == [4, 36]
    assert w.n_blocks == 8 and w.k_pool.shape == (8, 2, 16, 64) and w.k_pool.dtype == np.float32
    n = draw_lengths(get_config("c3", B=2000), np.random.default_rng(0))
    assert n.min() >= 128 and n.max() <= 2048
    assert list(draw_lengths(get_config("c3", B=5), np.random.default_rng(9))) == \
        list(make_workload(get_config("c3", B=5, H_q=1, H_kv=1, D=8), seed=9).context_lens)
    c4 = get_config("c4")
    rng_lens = draw_lengths(get_config("c4", B=4000), np.random.default_rng(0))
    assert rng_lens.min() >= 512 and rng_lens.max() <= 4096
    # log-uniform: the median sits near the geometric mean sqrt(512*4096) ~ 1448
    assert 1300 < np.median(rng_lens) < 1600
    assert c4.kv_std == 0.5 and c4.partition_size == 512
    c5 = get_config("c5")
    assert c5.G == 8 and c5.partition_size == 1024


def test_pool_factor():
    cfg = get_config("c2", B=2, H_q=2, H_kv=2)
    w = make_workload(cfg, seed=0)
    assert w.meta["required_blocks"] == 2 * 64 and w.n_blocks == 2 * 128


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    bits = to_storage(x, "bf16")
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... 0x3F82)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]


def test_step_bytes_c2_matches_hand_count():
    cfg = get_config("c2")
    b = step_bytes(cfg, np.full(8, 1024), append=False)
    assert b["total"] == 134_416_416
    ba = step_bytes(cfg, np.full(8, 1024), append=True)
    assert ba["kv_history"] == 8 * 1023 * 16384 and ba["append"] == 2 * 8 * 16384


def test_worked_transfer_example_pins_kv_bytes_per_token():
    g = json.load(open(os.path.join(GOLDEN, "kv_transfer_worked_example.json")))
    dims = g["model_dims_not_on_the_page"]
    per_tok = kv_bytes_per_token(dims["kv_heads"], dims["head_dim"], dims["elem_bytes"], layers=dims["layers"])
    pr = g["printed"]
    assert per_tok == pr["bytes_per_token_MB"] * 2 ** 20
    ms = pr["tokens"] * per_tok / (pr["links"] * pr["link_GB_per_s"] * 2 ** 30) * 1e3
    assert abs(ms - pr["latency_ms"]) <= g["tolerance_ms"]
