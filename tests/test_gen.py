"""Statistics and determinism of the seeded synthetic generators (CPU only)."""
import numpy as np
import pytest

from gen import synth, workloads as W

SMALL_F26 = W.scaled(W.F26, n_keys=260_000, batch=2048)
SMALL_F40 = W.scaled(W.F40_VARDIM, n_keys=2_000_000, batch=8192)
SMALL_F100 = W.scaled(W.F100, n_keys=1_000_000, batch=512)


def test_deterministic_and_batch_dependent():
    a = synth.batch(SMALL_F26, 3)
    b = synth.batch(SMALL_F26, 3)
    c = synth.batch(SMALL_F26, 4)
    assert np.array_equal(a["keys"], b["keys"]) and np.array_equal(a["grad"], b["grad"])
    assert not np.array_equal(a["offsets"], c["offsets"])
    r1, _ = synth.initial_state(W.TINY)
    r2, _ = synth.initial_state(W.TINY)
    assert np.array_equal(r1, r2)


@pytest.mark.parametrize("w", [W.TINY, SMALL_F26, SMALL_F40, SMALL_F100])
def test_keys_are_distinct_and_carry_their_field(w):
    k = synth.resident_keys(w)
    assert k.size == w.n_keys == synth.field_key_counts(w).sum()
    assert np.unique(k).size == k.size
    fid = (k >> np.uint64(48)).astype(np.int64)
    want = np.zeros(k.size, dtype=np.int64) if w.field0_only else np.repeat(
        np.arange(w.n_fields), synth.field_key_counts(w))
    assert np.array_equal(fid, want)


@pytest.mark.parametrize("w", [W.TINY, SMALL_F26, SMALL_F40])
def test_csr_shape_and_bag_fields(w):
    bt = synth.batch(w, 0)
    off = bt["offsets"].astype(np.int64)
    assert off[0] == 0 and off[-1] == bt["keys"].size and np.all(np.diff(off) >= 0)
    assert off.size == w.batch * w.n_fields + 1
    j = np.repeat(np.arange(off.size - 1), np.diff(off))
    fid = (bt["keys"].view(np.uint64) >> np.uint64(48)).astype(np.int64)
    want = np.zeros_like(j) if w.field0_only else j % w.n_fields
    assert np.array_equal(fid, want)
    assert bt["grad"].shape == (w.batch, int(synth.field_dims(w).sum()))
    assert bt["grad"].dtype == (np.float16 if w.grad_dtype == "f16" else np.float32)
    assert set(np.unique(bt["keys"].view(np.uint64))) <= set(synth.resident_keys(w).tolist())


def test_bag_length_distributions():
    L = synth.bag_lengths(SMALL_F26, 0)
    assert L.min() >= 1
    # E[max(1, Pois(3))] = 3 + P(X=0) = 3 + e^-3
    assert abs(L.mean() - (3 + np.exp(-3))) < 0.03
    L2 = synth.bag_lengths(SMALL_F100, 0)
    assert abs(L2.mean() - 5) < 0.05 and L2.min() == 0
    assert np.all(synth.bag_lengths(W.TINY, 0) == 4)


def test_zipf_rank_frequency_slope():
    r = np.random.default_rng(0)
    ranks = synth.zipf_ranks(r, 2_000_000, 100_000, 1.05)
    assert ranks.min() >= 1 and ranks.max() <= 100_000
    cnt = np.bincount(ranks, minlength=101)[1:101].astype(np.float64)
    slope = np.polyfit(np.log(np.arange(1, 101)), np.log(cnt), 1)[0]
    assert abs(slope + 1.05) < 0.05
    # truncated law: P(1) = 1 / H_{N,alpha}
    H = (np.arange(1, 100_001, dtype=np.float64) ** -1.05).sum()
    assert abs(cnt[0] / 2_000_000 - 1 / H) < 0.01 / H * 10


def test_longtail_batch_is_exactly_ninety_percent_tail():
    bt = synth.batch(SMALL_F40, 0, with_grad=False)
    k = bt["keys"].view(np.uint64)
    fid = (k >> np.uint64(48)).astype(np.int64)
    for f in range(0, SMALL_F40.n_fields, 7):
        kk = k[fid == f]
        if kk.size == 0:
            continue
        _, c = np.unique(kk, return_counts=True)
        tail = (c <= 2).sum()
        assert tail == 9 * (c.size - tail)                 # 90 % / 10 % split, exactly
        assert c.sum() == kk.size


def test_var_dims_and_fp16_state():
    d = synth.field_dims(W.F40_VARDIM)
    assert set(d.tolist()) <= set(W.DIM_CHOICES) and len(set(d.tolist())) > 2
    rows, master = synth.initial_state(W.scaled(W.F100, n_keys=10_000, batch=8))
    assert rows.dtype == np.float16 and master.dtype == np.float32
    assert rows.tobytes() == master.astype(np.float16).tobytes()
    assert abs(master.std() - 0.01) < 5e-4
    off = synth.row_offsets(SMALL_F40)
    assert off[-1] == (synth.field_dims(SMALL_F40).astype(np.int64)
                       * synth.field_key_counts(SMALL_F40)).sum()
