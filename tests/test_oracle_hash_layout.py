"""Pins for the oracle's hash and table layout (CPU only).

The pages give no hash or probing scheme (the Tencent talk only says the keys
are rehashed into one big table that is prebuilt off-GPU), so the oracle's
choices are pinned by mathematics: the hash is checked against an
independently derived inverse and for mixing quality; the layout is checked by
a textbook sequential insertion, brute-force search and linear-probing theory.
"""
import numpy as np
import pytest

from oracle import emb_oracle as O

M64 = (1 << 64) - 1


def inverse_hash(y: int) -> int:
    """Undo the mix step by step: x ^ (x >> 32) is its own inverse on 64 bits,
    and multiplication by an odd constant is undone by its inverse mod 2**64."""
    inv = pow(O.MIX, -1, 1 << 64)
    x = y ^ (y >> 32)
    x = (x * inv) & M64
    x ^= x >> 32
    x = (x * inv) & M64
    x ^= x >> 32
    return x


def test_mix_constant_is_golden_ratio_fraction():
    # floor(2**64 / phi) computed from phi = (1 + sqrt 5) / 2 with integer arithmetic
    from math import isqrt
    s5 = isqrt(5 << 256)                   # sqrt(5) * 2**128
    phi = ((1 << 128) + s5) // 2           # phi * 2**128
    assert ((1 << 64) << 128) // phi == O.MIX
    assert O.MIX & 1


def test_hash_fixed_point_and_inverse():
    assert O.hash64(0) == 0
    r = np.random.default_rng(7)
    for k in r.integers(0, 1 << 63, size=2000, dtype=np.int64).tolist() + [1, 2, M64 - 1, 1 << 48]:
        assert inverse_hash(O.hash64(k)) == k


def test_hash_numpy_matches_python_ints():
    r = np.random.default_rng(8)
    k = r.integers(0, 1 << 63, size=5000, dtype=np.int64).view(np.uint64) * np.uint64(2) + np.uint64(1)
    h = O.hash64_array(k)
    assert all(int(a) == O.hash64(int(b)) for a, b in zip(h, k))


def test_hash_is_injective_on_a_million_keys():
    r = np.random.default_rng(9)
    k = np.unique(r.integers(0, 1 << 62, size=1_000_000, dtype=np.int64).view(np.uint64))
    assert np.unique(O.hash64_array(k)).size == k.size


def test_hash_avalanche_in_high_half():
    # flipping one input bit should flip about half of the 32 high output bits
    r = np.random.default_rng(10)
    k = r.integers(0, 1 << 63, size=4000, dtype=np.int64).view(np.uint64)
    h0 = O.hash64_array(k) >> np.uint64(32)
    for bit in (0, 1, 17, 31, 32, 47, 48, 55, 63):
        h1 = O.hash64_array(k ^ np.uint64(1 << bit)) >> np.uint64(32)
        flips = np.array([bin(int(x)).count("1") for x in (h0 ^ h1)])
        assert 14.0 < flips.mean() < 18.0, (bit, flips.mean())


def test_home_is_uniform():
    from scipy.stats import chisquare
    r = np.random.default_rng(11)
    k = r.integers(0, 1 << 48, size=400_000, dtype=np.int64).view(np.uint64)
    home = O.home_of(O.hash64_array(k), 1000)
    assert home.min() >= 0 and home.max() < 1000
    assert chisquare(np.bincount(home, minlength=1000)).pvalue > 1e-4


def test_home_range_reduction_matches_definition():
    for h, n in [(0, 5), (M64, 5), (M64, 1), (1 << 63, 10), (123456789 << 32, 1_600_000_000)]:
        assert O.home_of(h, n) == ((h >> 32) * n) >> 32
        assert 0 <= O.home_of(h, n) < n


def test_n_home_slots():
    assert O.n_home_slots(1 << 22, 0.5) == 1 << 23
    assert O.n_home_slots(50_000_000, 0.6) == 83_333_334
    assert O.n_home_slots(0, 0.5) == 1


@pytest.mark.parametrize("n,lf", [(1, 0.5), (7, 0.9), (300, 0.5), (500, 0.95), (2000, 0.6)])
def test_closed_form_equals_sequential_insertion(n, lf):
    r = np.random.default_rng(n)
    keys = np.unique(r.integers(0, 1 << 50, size=n, dtype=np.int64)).view(np.uint64)
    nh = O.n_home_slots(keys.size, lf)
    want = O.layout_by_insertion(keys.tolist(), nh)
    home, slot = O.layout_closed_form(keys, nh)
    assert [want[int(k)] for k in keys] == slot.tolist()


def test_crowded_table_clusters_and_spills():
    # far more keys than home slots: one long cluster running past n_home
    keys = np.arange(1, 201, dtype=np.uint64) * np.uint64(0x1234567)
    nh = 10
    want = O.layout_by_insertion(keys.tolist(), nh)
    _, slot = O.layout_closed_form(keys, nh)
    assert [want[int(k)] for k in keys] == slot.tolist()
    assert slot.max() >= 199


@pytest.mark.parametrize("lf", [0.5, 0.6, 0.9])
def test_probe_brute_force(lf):
    r = np.random.default_rng(int(lf * 100))
    keys = np.unique(r.integers(0, 1 << 48, size=3000, dtype=np.int64)).view(np.uint64)
    nh = O.n_home_slots(keys.size, lf)
    home, slot = O.layout_closed_form(keys, nh)
    arr = O.key_array(keys, slot, nh)
    assert arr[-1] == np.uint64(O.EMPTY)
    for k, s in zip(keys[:500], slot[:500]):
        # the probe returns the one position where a full scan finds the key
        assert np.nonzero(arr == k)[0].tolist() == [s]
        assert O.probe(arr, nh, int(k)) == s
    absent = r.integers(1 << 49, 1 << 50, size=300, dtype=np.int64).view(np.uint64)
    for k in absent:
        assert not np.any(arr == k)
        assert O.probe(arr, nh, int(k)) == O.MISS
    assert O.probe(arr, nh, O.EMPTY) == O.MISS


def test_layout_invariants():
    r = np.random.default_rng(12)
    keys = np.unique(r.integers(0, 1 << 48, size=50_000, dtype=np.int64)).view(np.uint64)
    nh = O.n_home_slots(keys.size, 0.6)
    home, slot = O.layout_closed_form(keys, nh)
    assert np.all(slot >= home)
    assert np.unique(slot).size == keys.size
    occ = np.zeros(int(slot.max()) + 1, dtype=bool)
    occ[slot] = True
    # every slot between a key's home and its slot is occupied
    cs = np.concatenate([[0], np.cumsum(occ)])
    assert np.all(cs[slot + 1] - cs[home] == slot - home + 1)
    # along the array, (home, key) increases strictly
    o = np.argsort(slot)
    hk = list(zip(home[o].tolist(), keys[o].tolist()))
    assert all(a < b for a, b in zip(hk, hk[1:]))


@pytest.mark.parametrize("lf,want", [(0.5, 0.5), (0.6, 0.75)])
def test_mean_displacement_matches_linear_probing_theory(lf, want):
    # successful-search cost of linear probing is (1 + 1/(1-a))/2 probes, i.e.
    # a mean displacement of (1/(1-a) - 1)/2 (Knuth, TAOCP vol. 3, 6.4)
    r = np.random.default_rng(13)
    keys = np.unique(r.integers(0, 1 << 48, size=400_000, dtype=np.int64)).view(np.uint64)
    nh = O.n_home_slots(keys.size, lf)
    home, slot = O.layout_closed_form(keys, nh)
    assert abs((slot - home).mean() - want) < 0.03 * want + 0.01


def test_validation_errors():
    with pytest.raises(O.OracleError):
        O.validate_keys(np.array([1, 2, 1], dtype=np.uint64), 1)
    with pytest.raises(O.OracleError):
        O.validate_keys(np.array([O.EMPTY], dtype=np.uint64), 1)
    with pytest.raises(O.OracleError):
        O.validate_keys(np.array([(3 << 48) | 5], dtype=np.uint64), 3)
    O.validate_keys(np.array([(2 << 48) | 5], dtype=np.uint64), 3)


def test_multiple_hash_partition():
    r = np.random.default_rng(14)
    keys = np.unique(r.integers(0, 1 << 48, size=1000, dtype=np.int64)).view(np.uint64)
    t = O.table_of(keys, 2)
    assert set(np.unique(t).tolist()) <= {0, 1}
    assert np.all(t == (keys & np.uint64(1)).astype(np.int64))
    assert np.all(O.table_of(keys, 1) == 0)


@pytest.mark.parametrize("n,lf,chunk", [(1, 0.5, 1 << 24), (2000, 0.6, 97), (60_000, 0.5, 1000),
                                        (60_000, 0.95, 4096), (200_000, 1.0, 1 << 24)])
def test_sampled_slots_equal_full_layout(n, lf, chunk):
    """The counting form used for very large tables agrees with the sorted closed form (itself
    pinned by sequential insertion), including clusters that run across the chunks it walks."""
    r = np.random.default_rng(n + chunk)
    keys = np.unique(r.integers(0, 1 << 48, size=n, dtype=np.int64)).view(np.uint64)
    r.shuffle(keys)
    nh = O.n_home_slots(keys.size, lf)
    home, slot = O.layout_closed_form(keys, nh)
    sample = np.unique(r.integers(0, keys.size, size=min(keys.size, 3000)))
    hs, ss, rank = O.slots_of_sample(keys, nh, sample, chunk=chunk)
    assert np.array_equal(hs, home[sample])
    assert np.array_equal(ss, slot[sample])
    # rank = position in (home, key) order
    order = np.lexsort((keys, home))
    pos = np.empty(keys.size, dtype=np.int64)
    pos[order] = np.arange(keys.size)
    assert np.array_equal(rank, pos[sample])


def test_sampled_slots_on_a_crowded_table_by_insertion():
    # many keys per home slot: the same-home rank r carries most of the slot
    keys = np.arange(1, 301, dtype=np.uint64) * np.uint64(0x9E37)
    nh = 17
    want = O.layout_by_insertion(keys.tolist(), nh)
    sample = np.arange(0, 300, 7)
    _, ss, _ = O.slots_of_sample(keys, nh, sample, chunk=5)
    assert ss.tolist() == [want[int(k)] for k in keys[sample]]
