"""Pins of the oracle's FTRL-Proximal step against what the published method fixes, independent of
the oracle's own closed form:

* with no regularisation and a linear state consistent with the weights, FTRL-Proximal is online
  gradient descent with per-coordinate rates alpha / (beta + sqrt(n)) (McMahan et al. 2013, the
  equivalence stated with Algorithm 1);
* every iterate is the minimiser of the FTRL-Proximal objective (linear loss terms, proximal terms
  centred on the past iterates, L1 and L2 penalties), found here by a generic bounded scalar
  minimiser;
* the L1 term keeps a coordinate exactly at zero while the summed gradient stays within l1;
* the first step from zero state with no regularisation has length alpha whatever the gradient;
* storage rules shared with the Adagrad step (fp16 row = RNE of the fp32 master, untouched rows).
"""
import numpy as np
import pytest
from scipy.optimize import minimize_scalar

from oracle import emb_oracle as O


def one_row_table(D, w0, n0, z0=None, row_dtype="f32", master=None):
    keys = np.array([(0 << 48) | 12345], dtype=np.uint64)
    return O.Table(keys, [D], row_dtype, master is not None, 1, 0.5, n0,
                   np.asarray(w0, dtype=np.float32 if row_dtype == "f32" else np.float16),
                   master=master, ftrl=True, linear=z0)


def test_no_regularisation_equals_adaptive_gradient_descent():
    rng = np.random.default_rng(1)
    D, alpha, beta = 8, 0.05, 1.0
    w = rng.normal(0, 0.01, D)
    n = np.full(D, 0.1)
    # linear state consistent with the weights: z = -w (beta + sqrt(n)) / alpha
    z0 = (-w * (beta + np.sqrt(n)) / alpha).astype(np.float32)
    T = one_row_table(D, w.astype(np.float32), 0.1, z0)
    w = T.rows.astype(np.float64)
    n = T.acc.astype(np.float64)
    for _ in range(20):
        g = rng.normal(0, 1, D)
        T.ftrl_rows({0: g}, alpha, beta, 0.0, 0.0)
        n = n + g * g
        w = w - alpha * g / (beta + np.sqrt(n))
        np.testing.assert_allclose(T.rows, w, rtol=2e-5, atol=1e-7)
        np.testing.assert_allclose(T.acc, n, rtol=1e-6)


@pytest.mark.parametrize("l1,l2,beta", [(0.05, 0.1, 1.0), (0.5, 0.0, 0.5), (0.0, 1.0, 0.0),
                                        (2.0, 0.3, 1.0)])
def test_every_iterate_minimises_the_ftrl_objective(l1, l2, beta):
    rng = np.random.default_rng(7)
    D, alpha, n0 = 6, 0.1, 0.1
    w0 = rng.normal(0, 0.5, D).astype(np.float32)
    T = one_row_table(D, w0, n0)
    hist_w = [T.rows.astype(np.float64).copy()]
    hist_n = [T.acc.astype(np.float64).copy()]
    gsum = np.zeros(D)
    for t in range(8):
        g = rng.normal(0, 1, D)
        T.ftrl_rows({0: g}, alpha, beta, l1, l2)
        gsum += g
        hist_w.append(T.rows.astype(np.float64).copy())
        hist_n.append(T.acc.astype(np.float64).copy())
        sig = [(np.sqrt(hist_n[s]) - np.sqrt(hist_n[s - 1])) / alpha for s in range(1, t + 2)]
        base = (beta + np.sqrt(hist_n[0])) / alpha + l2
        for i in range(D):
            def obj(x):
                v = gsum[i] * x + l1 * abs(x) + 0.5 * base[i] * x * x
                for s in range(1, t + 2):
                    v += 0.5 * sig[s - 1][i] * (x - hist_w[s - 1][i]) ** 2
                return v
            # the minimiser lies where the objective's slope changes sign: within |z| / quadratic
            r = minimize_scalar(obj, bounds=(-50.0, 50.0), method="bounded",
                                options={"xatol": 1e-12})
            assert abs(T.rows[i] - r.x) <= 1e-5 * max(1.0, abs(r.x)) + 2e-7, (t, i, T.rows[i], r.x)


def test_l1_keeps_a_coordinate_exactly_zero_until_the_summed_gradient_exceeds_it():
    D, alpha, beta, l1 = 4, 0.1, 1.0, 1.0
    T = one_row_table(D, np.zeros(D, np.float32), 0.0)
    g = np.array([0.3, -0.3, 0.0, 0.45])
    for step in range(2):
        T.ftrl_rows({0: g}, alpha, beta, l1, 0.0)
        assert np.all(T.rows == 0.0)                 # |sum g| <= 0.9 < l1
    T.ftrl_rows({0: g}, alpha, beta, l1, 0.0)    # third step: |sum g| = 0.9, 0.9, 0, 1.35
    assert T.rows[0] == 0 and T.rows[1] == 0 and T.rows[2] == 0
    assert T.rows[3] < 0                          # z = 1.35 > l1: weight opposite to z


def test_first_step_from_zero_state_has_length_alpha():
    D, alpha = 5, 0.07
    T = one_row_table(D, np.zeros(D, np.float32), 0.0)
    g = np.array([1e-3, -2.0, 5.0, -1e-6, 0.5])
    T.ftrl_rows({0: g}, alpha, 0.0, 0.0, 0.0)
    np.testing.assert_allclose(T.rows, -alpha * np.sign(g), rtol=1e-6)


def test_fp16_master_storage_and_untouched_rows():
    rng = np.random.default_rng(3)
    keys = np.array([5, 6, 7], dtype=np.uint64)
    D = 16
    master = rng.normal(0, 0.1, 3 * D).astype(np.float32)
    T = O.Table(keys, [D], "f16", True, 1, 0.5, 0.1, master.astype(np.float16), master=master,
                ftrl=True)
    before = [x.copy() for x in T.state_of(2)] + [T.linear[2 * D:].copy()]
    for _ in range(3):
        T.ftrl_rows({0: rng.normal(0, 1, D), 1: rng.normal(0, 1, D)}, 0.05, 1.0, 0.01, 0.1)
    assert T.rows.tobytes() == O.f16(T.master).tobytes()
    after = [x for x in T.state_of(2)] + [T.linear[2 * D:]]
    for x, y in zip(before, after):
        assert x.tobytes() == y.tobytes()
    # a touched row whose linear state is zero and whose gradient is zero gets weight zero: the
    # FTRL weight is a function of (z, n) once the row is touched
    T2 = O.Table(keys[:1], [D], "f32", False, 1, 0.5, 0.1, master[:D], ftrl=True)
    T2.ftrl_rows({0: np.zeros(D)}, 0.05, 1.0, 0.0, 0.0)
    assert np.all(T2.rows == 0)


def test_first_step_moves_the_fp32_master_copy_by_alpha():
    """With beta = 0, no regularisation and a fresh accumulator, sigma = |g| / alpha makes the first
    step land exactly alpha away from the weight it reads against the gradient's sign.  The master
    holds 1 + 2^-12, which its fp16 row rounds to 1.0, so reading the row would miss the 2^-12."""
    keys = np.array([9], dtype=np.uint64)
    m = np.full(8, 1.0 + 2.0 ** -12, dtype=np.float32)
    T = O.Table(keys, [8], "f16", True, 1, 0.5, 0.0, m.astype(np.float16), master=m, ftrl=True)
    assert np.all(T.rows == 1.0)
    g = np.array([1.0, -1.0, 3.0, -0.5, 2.0, -2.0, 0.25, -8.0])
    T.ftrl_rows({0: g}, 0.25, 0.0, 0.0, 0.0)
    assert T.master.tobytes() == (m.astype(np.float64) - 0.25 * np.sign(g)).astype(np.float32).tobytes()
