"""The climbing-score inputs are strong enough to expose a wrong rescale (CPU only).

tests/test_gpu_softmax_edges.py relies on workloads.make_peaked_workload to make
the kernels' lazy rescaling run with live accumulators.  Here, on the CPU:

* the generator's inputs do climb: a wave's lazily moved reference maximum
  jumps by more than 8 binary orders at least twice inside every 512-token
  partition, for 1-block chunks over 4 waves;
* a plain float64 emulation of a wave-split online softmax whose reference
  maximum moves lazily (the scheme the grouped kernels use), merged by
  log-sum-exp, reproduces the oracle on them; and each planted mistake in its
  rescale -- accumulators not scaled, the running sum not scaled, alpha
  inverted -- misses the oracle by far more than the (2e-3, 1e-2) bound.
The emulation is written here from the softmax's definition; it shares nothing
with the HIP kernels, and the planted mistakes live only in this file.
"""
import numpy as np
import pytest

import oracle
from workloads import get_config, make_peaked_workload

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def climb():
    cfg = get_config("c5", B=2, H_q=4, H_kv=2, lengths=("fixed", (1500, 2600)), pool=("factor", 1.2),
                     partition_size=0)
    w = make_peaked_workload(cfg, 3)
    kf = oracle.decode("bf16", w.k_pool)
    vf = oracle.decode("bf16", w.v_pool)
    ref = oracle.paged_decode_attention("bf16", w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    return w, kf, vf, ref


def rows(w, pool, b, g):
    n = int(w.context_lens[b])
    t = np.arange(n)
    return pool[w.block_tables[b, t // 16], g, t % 16]


def lazy_softmax(s2, V, waves=4, slack=8.0, mistake=None):
    """Output of one head: tokens in 16-token chunks dealt round-robin to `waves` waves;
    each wave keeps (m, l, acc) with m moved only when a chunk's maximum exceeds it by more
    than `slack` (binary orders); the waves merge by log-sum-exp."""
    n = s2.size
    states = []
    for wv in range(waves):
        m, l, acc = -np.inf, 0.0, np.zeros(V.shape[1])
        for c in range(wv, -(-n // 16), waves):
            sl = slice(16 * c, min(16 * c + 16, n))
            mloc = s2[sl].max()
            if mloc > m + slack:
                alpha = 2.0 ** (m - mloc) if np.isfinite(m) else 0.0
                if mistake == "inverted" and np.isfinite(m):
                    alpha = 2.0 ** (mloc - m)
                if mistake != "sum":
                    l *= alpha
                if mistake != "acc":
                    acc = acc * alpha
                m = mloc
            p = 2.0 ** (s2[sl] - m)
            l += p.sum()
            acc = acc + p @ V[sl]
        if l > 0:
            states.append((m, l, acc))
    M = max(s[0] for s in states)
    L = sum(s[1] * 2.0 ** (s[0] - M) for s in states)
    O = sum(s[2] * 2.0 ** (s[0] - M) for s in states)
    return O / L


def test_generator_inputs_climb(climb):
    from tests.test_gpu_softmax_edges import lazy_jumps
    w, kf, _, _ = climb
    for b in range(2):
        for h in (0, 2):                                   # even heads of each group climb
            q = oracle.decode("bf16", w.q[b, h])
            s2 = float(w.scale) * (rows(w, kf, b, h // 2) @ q) * LOG2E
            for length, jumps in lazy_jumps(s2, 512, 1, 4):
                if length >= 512:
                    assert jumps >= 2


@pytest.mark.parametrize("mistake", [None, "acc", "sum", "inverted"])
def test_only_a_correct_rescale_matches_the_oracle(climb, mistake):
    w, kf, vf, ref = climb
    worst = 0.0
    for b in range(2):
        for h in range(4):
            g = h // 2
            q = oracle.decode("bf16", w.q[b, h])
            s2 = float(w.scale) * (rows(w, kf, b, g) @ q) * LOG2E
            with np.errstate(over="ignore", invalid="ignore"):
                out = lazy_softmax(s2, rows(w, vf, b, g), mistake=mistake)
            err = np.abs(out - ref[b, h]) / np.maximum(np.abs(ref[b, h]), 0.2)
            worst = max(worst, float(np.nan_to_num(err, nan=np.inf).max()))
    if mistake is None:
        assert worst < 1e-12
    else:
        assert worst > 0.1, f"planted mistake '{mistake}' went unseen (max rel err {worst:.2e})"
