"""Pins for the oracle's probe statistics (CPU only).

The statistic is the number of 15-slot buckets each probe reads (collision monitoring by
sampling, JD ads article, section 4.3).  The oracle computes it in vectorised form from the
table's slots; here it is checked against a slot-by-slot walk over the probed array built by
textbook sequential insertion, and against the displacement (slot - home), which the layout
tests pin to linear-probing theory.
"""
import numpy as np
import pytest

from oracle import emb_oracle as O


def walk_buckets(arr, n_home, key, per_bucket):
    """Scan from the key's home slot one slot at a time until the key or an EMPTY slot; return
    the number of distinct buckets the visited slots fall in."""
    k = int(key)
    s = O.home_of(O.hash64(k), n_home)
    seen = set()
    while True:
        seen.add(s // per_bucket)
        v = int(arr[s])
        if v == k or v == O.EMPTY:
            return len(seen)
        s += 1


def small_table(n_keys, n_fields, n_tables, lf, seed):
    r = np.random.default_rng(seed)
    fid = r.integers(0, n_fields, size=n_keys).astype(np.uint64)
    raw = np.unique(r.integers(0, 1 << 40, size=n_keys * 2, dtype=np.int64))[:n_keys]
    raw = r.permutation(raw).astype(np.uint64)
    keys = (fid << np.uint64(48)) | raw
    dims = np.full(n_fields, 8)
    rows = np.zeros(n_keys * 8, dtype=np.float32)
    return O.Table(keys, dims, "f32", False, n_tables, lf, 0.1, rows), r


def brute_force(ot, keys, offsets, per_bucket):
    """Per occurrence: 0 without a scan (EMPTY key, or another field than the bag's), else the
    buckets the slot-by-slot walk reads in the occurrence's table."""
    bag = O.bag_of_occurrence(offsets)
    out = []
    arrays = []
    for t in range(ot.n_tables):
        m = ot.tab == t
        # slots from sequential insertion, independent of the closed form the oracle uses
        ins = O.layout_by_insertion([int(k) for k in ot.keys[m]], ot.n_home[t])
        slots = np.array([ins[int(k)] for k in ot.keys[m]], dtype=np.int64)
        arrays.append(O.key_array(ot.keys[m], slots, ot.n_home[t]))
    for i, k in enumerate(np.asarray(keys).view(np.uint64)):
        k = int(k)
        if k == O.EMPTY or (k >> 48) != int(bag[i] % ot.F):
            out.append(0)
            continue
        t = (k & 1) if ot.n_tables == 2 else 0
        out.append(walk_buckets(arrays[t], ot.n_home[t], k, per_bucket))
    return np.array(out, dtype=np.int64)


def mixed_batch(ot, r, n_bags):
    """Bags of resident keys, absent keys, the EMPTY key and keys of another field."""
    F = ot.F
    bags = []
    for j in range(n_bags):
        f = j % F
        mine = ot.keys[(ot.keys >> np.uint64(48)) == np.uint64(f)]
        other = ot.keys[(ot.keys >> np.uint64(48)) != np.uint64(f)]
        b = list(mine[r.integers(0, mine.size, size=r.integers(0, 6))]) if mine.size else []
        if j % 3 == 0:
            b.append(np.uint64((f << 48) | int(r.integers(1 << 41, 1 << 42))))  # absent
        if j % 5 == 0:
            b.append(np.uint64(O.EMPTY))
        if j % 7 == 0 and other.size:
            b.append(other[0])                                            # wrong field
        bags.append(b)
    lens = np.array([len(b) for b in bags])
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    keys = np.array([k for b in bags for k in b], dtype=np.uint64).view(np.int64)
    return keys, off


@pytest.mark.parametrize("n_keys,n_fields,n_tables,lf,per_bucket",
                         [(300, 1, 1, 0.5, 15), (600, 3, 1, 0.95, 15), (500, 2, 2, 1.0, 15),
                          (400, 1, 1, 1.0, 4), (200, 2, 1, 0.8, 1)])
def test_scan_buckets_matches_slot_by_slot_walk(n_keys, n_fields, n_tables, lf, per_bucket):
    ot, r = small_table(n_keys, n_fields, n_tables, lf, seed=n_keys + n_tables)
    keys, off = mixed_batch(ot, r, 40 * n_fields)
    got = ot.scan_buckets(keys, off, per_bucket)
    want = brute_force(ot, keys, off, per_bucket)
    assert np.array_equal(got, want)
    assert (got == 0).any() and (got >= 1).any()


def test_one_slot_buckets_give_displacement_plus_one():
    # with buckets of one slot a hit reads slot - home + 1 buckets
    ot, r = small_table(3000, 4, 1, 0.9, seed=3)
    F = ot.F
    f = (ot.keys >> np.uint64(48)).astype(np.int64)
    order = np.argsort(f, kind="stable")           # every key once, each in a bag of its field
    counts = np.bincount(f, minlength=F)
    off = np.concatenate([[0], np.cumsum(counts)])
    got = ot.scan_buckets(ot.keys[order].view(np.int64), off, per_bucket=1)
    assert np.array_equal(got, ot.slot[order] - ot.home[order] + 1)


def test_full_bucket_table_at_load_factor_one_has_long_scans():
    # at load factor 1.0 clusters are long: many scans leave the home bucket, none at 0.05
    dense, r = small_table(3000, 1, 1, 1.0, seed=4)
    sparse, _ = small_table(3000, 1, 1, 0.05, seed=4)
    off = np.array([0, 3000])
    for ot, lo, hi in ((dense, 0.2, 1.0), (sparse, 0.0, 0.05)):
        b = ot.scan_buckets(ot.keys.view(np.int64), off)
        assert lo <= np.mean(b > 1) <= hi
