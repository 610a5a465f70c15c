"""Pins for the oracle's forward pooling, dedup, gradient reduction and Adagrad (CPU only).

Each check ties the oracle to something other than itself: plain loops on
tiny inputs, torch's CPU embedding_bag and autograd (the library routine the
JD article's section 4.2.1 builds on), a dense incidence-matrix product,
torch.optim.Adagrad, closed forms and invariants.
"""
import os

import numpy as np
import pytest
import torch

from oracle import emb_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make_table(n_keys=200, dims=(4,), row_dtype="f32", has_master=False, n_tables=1, lf=0.5,
               seed=0, acc_init=0.1, raw_hi=1 << 40):
    r = np.random.default_rng(seed)
    F = len(dims)
    keys = []
    for f in range(F):
        raw = np.unique(r.integers(0, raw_hi, size=n_keys, dtype=np.int64))[: n_keys // F]
        keys.append((np.uint64(f) << np.uint64(48)) | raw.view(np.uint64))
    keys = np.concatenate(keys)
    width = np.asarray(dims)[(keys >> np.uint64(48)).astype(np.int64)]
    draw = r.standard_normal(int(width.sum())).astype(np.float32) * np.float32(0.5)
    rows = draw if row_dtype == "f32" else draw.astype(np.float16)
    master = draw if has_master else None
    return O.Table(keys, dims, row_dtype, has_master, n_tables, lf, acc_init, rows,
                   master=master)


def make_batch(t: O.Table, B=16, mean=3, seed=1, miss_frac=0.0):
    r = np.random.default_rng(seed)
    F = t.F
    L = r.poisson(mean, size=(B, F))
    offsets = np.concatenate([[0], np.cumsum(L.reshape(-1))]).astype(np.int64)
    keys = np.empty(int(offsets[-1]), dtype=np.uint64)
    for j in range(B * F):
        f = j % F
        pool = t.keys[t.field == f]
        n = int(offsets[j + 1] - offsets[j])
        keys[offsets[j]:offsets[j + 1]] = pool[r.integers(0, pool.size, size=n)]
    if miss_frac:
        m = r.random(keys.size) < miss_frac
        keys[m] ^= np.uint64(1 << 47)          # absent raw ids of the same field
    width = int(t.dims.sum())
    grad = r.standard_normal((B, width))
    return keys.view(np.int64), offsets, grad


# ------------------------------------------------------------------ forward
def test_pool_matches_plain_loops_with_misses_duplicates_and_empty_bags():
    t = make_table(n_keys=300, dims=(4, 8, 4), seed=3)
    keys, offsets, _ = make_batch(t, B=20, mean=2, seed=4, miss_frac=0.1)
    keys = keys.copy()
    keys[0] = -1                              # EMPTY as a batch key: a miss
    out, n_miss = t.forward(keys, offsets, "f32")
    rows_by_key = {int(k): t.row64(i) for i, k in enumerate(t.keys)}
    plain = O.pool_plain(rows_by_key, keys.view(np.uint64), offsets)
    assert n_miss == sum(1 for k in keys.view(np.uint64) if int(k) not in rows_by_key)
    for j, v in enumerate(plain):
        b, f = divmod(j, t.F)
        blk = out[b, t.col[f]:t.col[f] + t.dims[f]]
        if v is None:
            assert np.all(blk == 0)
        else:
            np.testing.assert_array_equal(blk, v.astype(np.float32))


def test_pool_equals_torch_embedding_bag_fp64():
    t = make_table(n_keys=500, dims=(16,), seed=5)
    keys, offsets, _ = make_batch(t, B=64, mean=4, seed=6)
    out, _ = t.forward(keys, offsets, "f32")
    W = torch.from_numpy(t.rows.reshape(-1, 16).astype(np.float64))
    idx = torch.from_numpy(t.key_index(keys))
    ref = torch.nn.functional.embedding_bag(idx, W, torch.from_numpy(offsets[:-1]), mode="sum")
    np.testing.assert_array_equal(out, ref.numpy().astype(np.float32))


def test_pool_is_linear_in_rows_and_additive_over_bag_splits():
    t1 = make_table(n_keys=200, dims=(8,), seed=7)
    t2 = make_table(n_keys=200, dims=(8,), seed=7)
    t2.rows[:] = np.random.default_rng(8).standard_normal(t2.rows.size).astype(np.float32)
    a = 0.75
    t3 = make_table(n_keys=200, dims=(8,), seed=7)
    t3.rows[:] = (a * t1.rows.astype(np.float64) + t2.rows).astype(np.float32)
    keys, offsets, _ = make_batch(t1, B=30, mean=5, seed=9)
    p1, _ = t1.forward(keys, offsets, "f32")
    p2, _ = t2.forward(keys, offsets, "f32")
    p3, _ = t3.forward(keys, offsets, "f32")
    np.testing.assert_allclose(p3, a * p1.astype(np.float64) + p2, rtol=1e-5, atol=1e-5)
    # splitting every bag in two and adding the halves gives the same pool
    mid = (offsets[:-1] + offsets[1:]) // 2
    split = np.empty(2 * (offsets.size - 1) + 1, dtype=np.int64)
    split[0::2] = offsets
    split[1::2] = mid
    # the split batch is read as a two-sample batch per original sample
    halves, _ = t1.forward(keys, split, "f32")
    np.testing.assert_allclose(halves[0::2] + halves[1::2].astype(np.float64), p1, rtol=1e-6,
                               atol=1e-6)


def test_bag_field_mismatch_is_a_miss():
    t = make_table(n_keys=100, dims=(4, 4), seed=10)
    k0 = t.keys[t.field == 0][0]
    keys = np.array([k0, k0], dtype=np.uint64).view(np.int64)
    offsets = np.array([0, 1, 2])             # bag 0 is field 0, bag 1 is field 1
    out, n_miss = t.forward(keys, offsets, "f32")
    assert n_miss == 1
    np.testing.assert_array_equal(out[0, 0:4], t.row64(int(np.nonzero(t.keys == k0)[0][0])).astype(np.float32))
    assert np.all(out[0, 4:8] == 0)


def test_pool_fp16_rounds_once_from_float64():
    # a sum just above a rounding midpoint must round up (single rounding)
    t = make_table(n_keys=20, dims=(8,), row_dtype="f16", seed=11)
    x = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert float(O.f16(np.array([x]))[0]) == 1.0 + 2.0 ** -10
    assert float(O.f16(np.array([1.0 + 2.0 ** -11]))[0]) == 1.0       # tie to even
    assert float(O.f16(np.array([2.0 ** -24]))[0]) == 2.0 ** -24         # subnormal kept


def test_pool_sampled_bags_match_full():
    t = make_table(n_keys=400, dims=(4, 8), seed=12, row_dtype="f16", has_master=True)
    keys, offsets, _ = make_batch(t, B=25, mean=3, seed=13)
    out, _ = t.forward(keys, offsets, "f16")
    res, _ = t.forward(keys, offsets, "f16", bags=np.arange(0, 50, 7))
    for j, v in res.items():
        b, f = divmod(j, t.F)
        np.testing.assert_array_equal(out[b, t.col[f]:t.col[f] + t.dims[f]], v)


# ------------------------------------------------------------------ dedup / reduce
def test_touched_matches_counter_and_is_sorted_by_table_then_slot():
    t = make_table(n_keys=300, dims=(4, 4), n_tables=2, seed=14)
    keys, offsets, _ = make_batch(t, B=40, mean=4, seed=15, miss_frac=0.05)
    u, tab, slot, cnt = t.touched(keys, offsets)
    kidx, _, _ = t.lookup(keys, offsets)
    want = O.dedup_counts_plain(kidx[kidx >= 0].tolist())
    assert sorted(zip(u.tolist(), cnt.tolist())) == want
    assert cnt.sum() == (kidx >= 0).sum()
    assert u.size <= min(keys.size, t.keys.size)
    pairs = list(zip(tab.tolist(), slot.tolist()))
    assert pairs == sorted(pairs) and len(set(pairs)) == len(pairs)


def test_row_grads_equal_incidence_product_and_autograd():
    t = make_table(n_keys=120, dims=(6,), seed=16)
    keys, offsets, grad = make_batch(t, B=30, mean=5, seed=17)
    g = t.row_grads(keys, offsets, grad)
    # dense incidence: A[j, u] = number of times key u occurs in bag j;  g = A^T G
    kidx = t.key_index(keys)
    bag = O.bag_of_occurrence(offsets)
    A = np.zeros((offsets.size - 1, t.keys.size))
    np.add.at(A, (bag, kidx), 1.0)
    dense = A.T @ grad
    for u, v in g.items():
        np.testing.assert_allclose(v, dense[u], rtol=1e-12, atol=1e-12)
    assert set(g) == set(np.nonzero(A.sum(0))[0].tolist())
    # autograd of embedding_bag(sum) in float64
    W = torch.zeros(t.keys.size, 6, dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.embedding_bag(torch.from_numpy(kidx), W,
                                            torch.from_numpy(offsets[:-1]), mode="sum")
    out.backward(torch.from_numpy(grad))
    for u, v in g.items():
        np.testing.assert_allclose(v, W.grad[u].numpy(), rtol=1e-12, atol=1e-12)


def test_row_grads_var_dim_uses_each_fields_block():
    t = make_table(n_keys=200, dims=(8, 16, 32), seed=18, row_dtype="f16", has_master=True)
    keys, offsets, grad = make_batch(t, B=12, mean=3, seed=19)
    g = t.row_grads(keys, offsets, grad)
    kidx = t.key_index(keys)
    bag = O.bag_of_occurrence(offsets)
    for u, v in g.items():
        f = int(t.field[u])
        assert v.size == t.dims[f]
        occ = np.nonzero(kidx == u)[0]
        want = sum(grad[bag[i] // t.F, t.col[f]:t.col[f] + t.dims[f]] for i in occ)
        np.testing.assert_allclose(v, want, rtol=1e-12)


# ------------------------------------------------------------------ Adagrad
def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "adagrad_single_step.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return rows


@pytest.mark.parametrize("row", _golden_rows())
def test_adagrad_single_step_golden(row):
    w0, g, acc0, lr, eps, acc_new, w_new = row
    t = make_table(n_keys=2, dims=(1,), seed=20, acc_init=acc0)
    t.rows[0] = np.float32(w0)
    t.adagrad_rows({0: np.array([g])}, lr, eps)
    # lr and eps pass through fp32 (the library takes them as float); results are fp32
    assert abs(float(t.acc[0]) - acc_new) <= 1e-7 * abs(acc_new) + 1e-20
    assert abs(float(t.rows[0]) - w_new) <= 2e-7 * abs(w_new)


def test_adagrad_sign_update_when_acc_and_eps_are_zero():
    t = make_table(n_keys=64, dims=(4,), seed=21, acc_init=0.0)
    before = t.rows.copy()
    r = np.random.default_rng(22)
    g = {u: r.standard_normal(4) for u in range(0, 32)}
    t.adagrad_rows(g, 0.25, 0.0)
    for u, gu in g.items():
        want = before[4 * u:4 * u + 4].astype(np.float64) - 0.25 * np.sign(gu)
        np.testing.assert_allclose(t.rows[4 * u:4 * u + 4], want, rtol=1e-7, atol=1e-7)


def test_adagrad_invariants_and_untouched_rows():
    t = make_table(n_keys=128, dims=(8,), seed=23)
    rows0, acc0 = t.rows.copy(), t.acc.copy()
    r = np.random.default_rng(24)
    g = {u: r.standard_normal(8) * 10 for u in range(0, 60, 2)}
    g[1] = np.zeros(8)                        # a zero gradient leaves the row bit-identical
    t.adagrad_rows(g, 0.05, 1e-8)
    for u in range(t.keys.size):
        a, b = 8 * u, 8 * u + 8
        if u in g:
            assert np.all(t.acc[a:b] >= acc0[a:b])
            assert np.all(np.abs(t.rows[a:b].astype(np.float64) - rows0[a:b]) < 0.05 + 1e-6)
        if u not in g or u == 1:
            assert t.rows[a:b].tobytes() == rows0[a:b].tobytes()
            assert t.acc[a:b].tobytes() == acc0[a:b].tobytes()


def test_adagrad_equals_torch_optim_adagrad_dense_step():
    t = make_table(n_keys=64, dims=(4,), seed=25)
    keys, offsets, grad = make_batch(t, B=10, mean=3, seed=26)
    P = torch.tensor(t.rows.reshape(-1, 4).astype(np.float64), requires_grad=True)
    opt = torch.optim.Adagrad([P], lr=float(np.float32(0.05)), eps=float(np.float32(1e-8)),
                              initial_accumulator_value=0.1)
    kidx = t.key_index(keys)
    out = torch.nn.functional.embedding_bag(torch.from_numpy(kidx), P,
                                            torch.from_numpy(offsets[:-1]), mode="sum")
    out.backward(torch.from_numpy(grad))
    opt.step()
    t.backward(keys, offsets, grad, 0.05, 1e-8)
    np.testing.assert_allclose(t.rows.reshape(-1, 4), P.detach().numpy(), rtol=2e-7, atol=1e-9)
    st = opt.state[P]["sum"].numpy()
    np.testing.assert_allclose(t.acc.reshape(-1, 4), st, rtol=2e-7)


def test_adagrad_two_steps_compose():
    t = make_table(n_keys=16, dims=(3,), seed=27)
    w0 = t.rows[:3].astype(np.float64)
    g1, g2 = np.array([0.3, -1.0, 2.0]), np.array([-0.7, 0.1, 0.0])
    lr, eps = float(np.float32(0.05)), float(np.float32(1e-8))
    t.adagrad_rows({0: g1}, 0.05, 1e-8)
    t.adagrad_rows({0: g2}, 0.05, 1e-8)
    a1 = 0.1 + g1 ** 2
    w1 = w0 - lr * g1 / (np.sqrt(a1) + eps)
    a2 = a1 + g2 ** 2
    w2 = w1 - lr * g2 / (np.sqrt(a2) + eps)
    np.testing.assert_allclose(t.rows[:3], w2, rtol=1e-6)
    np.testing.assert_allclose(t.acc[:3], a2, rtol=1e-6)


def test_fp16_master_and_no_master_paths():
    tm = make_table(n_keys=64, dims=(8,), seed=28, row_dtype="f16", has_master=True)
    tn = make_table(n_keys=64, dims=(8,), seed=28, row_dtype="f16", has_master=False)
    r = np.random.default_rng(29)
    for step in range(3):
        g = {u: r.standard_normal(8) for u in range(0, 64, 3)}
        rows_before = tn.rows.copy()
        acc_before = tn.acc.copy()
        tm.adagrad_rows(g, 0.05, 1e-8)
        tn.adagrad_rows(g, 0.05, 1e-8)
        # master invariant: the stored row is the fp16 rounding of the master copy
        assert tm.rows.tobytes() == tm.master.astype(np.float16).tobytes()
        # no master: the fp16 row itself is updated and re-rounded
        for u, gu in g.items():
            a, b = 8 * u, 8 * u + 8
            acc_new = acc_before[a:b].astype(np.float64) + gu * gu
            d = float(np.float32(0.05)) * gu / (np.sqrt(acc_new) + float(np.float32(1e-8)))
            want = (rows_before[a:b].astype(np.float64) - d).astype(np.float16)
            assert tn.rows[a:b].tobytes() == want.tobytes()


def test_backward_end_to_end_matches_pieces():
    t = make_table(n_keys=300, dims=(4, 8), n_tables=2, seed=30, row_dtype="f16", has_master=True)
    t2 = make_table(n_keys=300, dims=(4, 8), n_tables=2, seed=30, row_dtype="f16", has_master=True)
    keys, offsets, grad = make_batch(t, B=20, mean=3, seed=31, miss_frac=0.05)
    grad = grad.astype(np.float16)
    u, tab, slot, cnt = t.backward(keys, offsets, grad, 0.05, 1e-8)
    g = t2.row_grads(keys, offsets, grad)
    assert set(g) == set(u.tolist())
    t2.adagrad_rows(g, 0.05, 1e-8)
    assert t.rows.tobytes() == t2.rows.tobytes()
    assert t.acc.tobytes() == t2.acc.tobytes()
