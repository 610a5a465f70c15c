"""Property-based pins (hypothesis) for the oracle's layout and probe statistics on small,
adversarial tables, and for the arithmetic fact the full-size exact-sum checks rest on."""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from gen import synth, workloads as W  # noqa: E402
from oracle import emb_oracle as O  # noqa: E402
from tests.test_oracle_probe_stats import brute_force  # noqa: E402

FAST = settings(max_examples=60, deadline=None, derandomize=True, database=None)


@st.composite
def key_sets(draw):
    n = draw(st.integers(1, 120))
    raw = draw(st.lists(st.integers(0, (1 << 48) - 1), min_size=n, max_size=n, unique=True))
    fields = draw(st.lists(st.integers(0, 2), min_size=n, max_size=n))
    keys = np.array([(f << 48) | r for f, r in zip(fields, raw)], dtype=np.uint64)
    lf = draw(st.sampled_from([0.3, 0.5, 0.8, 1.0]))
    return keys, lf


@FAST
@given(key_sets())
def test_closed_form_layout_equals_textbook_insertion(ks):
    keys, lf = ks
    nh = O.n_home_slots(keys.size, lf)
    _, slot = O.layout_closed_form(keys, nh)
    ins = O.layout_by_insertion([int(k) for k in keys], nh)
    assert [ins[int(k)] for k in keys] == slot.tolist()


@FAST
@given(key_sets(), st.integers(0, 2**32 - 1), st.sampled_from([1, 4, 15]))
def test_scan_buckets_equal_the_walk(ks, seed, per_bucket):
    keys, lf = ks
    r = np.random.default_rng(seed)
    ot = O.Table(keys, [8, 8, 8], "f32", False, 1 + (seed & 1), lf, 0.1,
                 np.zeros(keys.size * 8, np.float32))
    # bags of field 0..2: resident keys, absent keys, the EMPTY key
    pool = np.concatenate([keys, (np.arange(5, dtype=np.uint64) << np.uint64(48)) | np.uint64(12345),
                           np.array([O.EMPTY], dtype=np.uint64)])
    q = pool[r.integers(0, pool.size, size=30)]
    lens = r.multinomial(q.size, np.ones(6) / 6)
    off = np.concatenate([[0], np.cumsum(lens)])
    assert np.array_equal(ot.scan_buckets(q.view(np.int64), off, per_bucket),
                          brute_force(ot, q.view(np.int64), off, per_bucket))


@settings(max_examples=30, deadline=None, derandomize=True, database=None)
@given(st.integers(0, 2**32 - 1), st.integers(1, 1 << 17))
def test_dyadic_gradients_sum_exactly_in_fp32_in_any_order(seed, n):
    """Every element of synth.dyadic_grad is a multiple of 2^-7 in [-1, 1]; a sum of up to 2^17
    of them is a multiple of 2^-7 below 2^17 in magnitude, which fp32 holds exactly, so every
    partial sum in any order is exact."""
    w = W.scaled(W.F100, n_keys=1000, batch=64)
    g = synth.dyadic_grad(w, seed % 7).astype(np.float32).reshape(-1)
    assert np.all(g * 128 == np.round(g * 128)) and np.abs(g).max() <= 1
    r = np.random.default_rng(seed)
    x = g[r.integers(0, g.size, size=n)]
    exact = float(np.sum(x.astype(np.float64)))
    sub = x[r.permutation(n)][: min(n, 4096)]       # a sequential fp32 sum in a random order
    acc = np.float32(0)
    for v in sub:
        acc = np.float32(acc + v)
    assert float(acc) == float(np.sum(sub.astype(np.float64)))
    assert float(np.sum(x, dtype=np.float32)) == exact   # numpy's pairwise fp32 sum
