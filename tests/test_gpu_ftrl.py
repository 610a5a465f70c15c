"""GPU parity of the FTRL-Proximal update (sparse_ftrl_bwd) against the oracle: forward outputs and
the unique set bit-exact, rows, masters, accumulators and linear states within the budgets derived
in parity_util over consecutive steps, untouched state bit-identical.  Covers fp32 and fp16 rows,
with and without master, mixed widths over two tables, a strong L1 term that leaves most weights at
exactly zero, a supplied non-zero linear state, and the PASS write-backs and carry with the linear
state."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ad_recommendation_amd import emb  # noqa: E402
from gen import synth, workloads as W  # noqa: E402
from oracle import emb_oracle as O  # noqa: E402
from tests import parity_util as P  # noqa: E402
from tests.test_gpu_parity import DT, gpu_step, width_class  # noqa: E402

pytestmark = pytest.mark.gpu

BETA, L1, L2 = 1.0, 0.01, 0.1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    emb.lib()
    yield


def run_ftrl(w, steps=3, l1=L1, l2=L2, beta=BETA, linear=None, flags=0):
    dims = synth.field_dims(w)
    keys = synth.resident_keys(w)
    rows, master = synth.initial_state(w)
    say(f"[ftrl] {w.name}: {keys.size} keys, l1={l1} l2={l2} beta={beta}")
    T = emb.Table(dims, DT[w.row_dtype], w.has_master, w.n_tables, w.load_factor, w.acc_init,
                  keys, rows, None, master, flags=emb.FLAG_FTRL | flags)
    if linear is not None:
        T.fill_linear(0, keys.size, linear)
    T.flash()
    ot = O.Table(keys, dims, w.row_dtype, w.has_master, w.n_tables, w.load_factor, w.acc_init,
                 rows, master=master, ftrl=True, linear=linear)
    bud = P.Budget(ot)
    prm = (w.lr, beta, l1, l2)
    for s in range(steps):
        bt = synth.batch(w, s)
        kk, off, grad = bt["keys"], bt["offsets"], bt["grad"]
        res = gpu_step(T, kk, off, grad, w.out_dtype, w.grad_dtype, 0.0, 0.0, ftrl=prm)
        kidx, tab, slot = ot.lookup(kk, off)
        assert np.array_equal(res["slot"], slot)
        out_o, nm = ot.forward(kk, off, w.out_dtype)
        assert nm == res["n_miss"]
        P.check_pooled(res["out"], out_o, P.pooled_scale(ot, kk, off, bud), w.out_dtype)
        u, utab, uslot, ucnt = bud.oracle_step_ftrl(ot, kk, off, grad, *prm)
        assert res["n_unique"] == u.size
        if T.info["unique_by_width"]:
            order = np.argsort(width_class(w, dims)[ot.field[u]], kind="stable")
            u, ucnt = u[order], ucnt[order]
        got = emb.table_rowref_keys(T.h, res["unique"]) if u.size else np.zeros(0, np.int64)
        assert np.array_equal(got.view(np.uint64), ot.keys[u])
        assert np.array_equal(res["count"], ucnt)
        say(f"[ftrl] {w.name} step {s}: nnz={kk.size} unique={u.size}")
    return T, ot, bud, keys


def check_all(T, ot, bud, keys):
    emb.pass_writeback(T.h)
    r, a, m = T.export(keys)
    z = T.export_linear(keys)
    P.check_state(ot, bud, keys, r, a, m, z)
    return r, a, m, z


@pytest.mark.parametrize("w", [W.TINY, W.scaled(W.F26, n_keys=500_000, batch=512),
                               W.scaled(W.F100, n_keys=200_000, batch=64),
                               W.scaled(W.F40_VARDIM, n_keys=400_000, batch=256),
                               W.scaled(W.F64_PASS, n_keys=400_000, batch=64)],
                         ids=lambda w: w.name)
def test_ftrl_parity(w):
    T, ot, bud, keys = run_ftrl(w)
    check_all(T, ot, bud, keys)
    say(f"[ftrl] {w.name}: ok")


@pytest.mark.parametrize("w", [W.TINY, W.scaled(W.F40_VARDIM, n_keys=400_000, batch=256)],
                         ids=lambda w: w.name)
def test_ftrl_strong_l1_gives_exact_zeros(w):
    T, ot, bud, keys = run_ftrl(w, l1=1.0)
    r, _, _, _ = check_all(T, ot, bud, keys)
    # where the oracle's |z'| is clear of the threshold, zero weights are zero on both sides
    touched = bud.row > 0
    zero_o = ot.rows == 0
    assert zero_o[touched].mean() > 0.3
    clear = np.abs(np.abs(ot.linear.astype(np.float64)) - 1.0) > 10 * bud.lin
    sel = touched & zero_o & clear
    # rows come back in key order; the oracle holds them in the same packing
    assert np.all(r[sel] == 0)


def test_ftrl_with_supplied_linear_state():
    w = W.scaled(W.F26, n_keys=200_000, batch=256)
    rows, _ = synth.initial_state(w)
    z = np.random.default_rng(42).normal(0, 0.5, rows.size).astype(np.float32)
    T, ot, bud, keys = run_ftrl(w, linear=z)
    check_all(T, ot, bud, keys)


def test_ftrl_state_in_pass_lifecycle():
    """Touched write-back of an FTRL table equals its full write-back (the linear state included),
    and carry copies the linear state into the next table."""
    w = W.scaled(W.F100, n_keys=100_000, batch=64)
    dims = synth.field_dims(w)
    keys = synth.resident_keys(w)
    rows, master = synth.initial_state(w)
    mk = lambda fl: emb.Table(dims, DT[w.row_dtype], w.has_master, w.n_tables, w.load_factor,
                              w.acc_init, keys, rows, None, master, flags=emb.FLAG_FTRL | fl)
    A, B = mk(emb.FLAG_TRACK_TOUCHED), mk(0)
    A.flash()
    B.flash()
    prm = (w.lr, BETA, L1, L2)
    for s in range(2):
        bt = synth.batch(w, s)
        for T in (A, B):
            gpu_step(T, bt["keys"], bt["offsets"], bt["grad"], w.out_dtype, w.grad_dtype, 0, 0,
                     want_unique=False, ftrl=prm)
    A.writeback_touched()
    emb.pass_writeback(B.h)
    for x, y in zip(A.export(keys), B.export(keys)):
        if x is not None:
            assert x.tobytes() == y.tobytes()
    assert A.export_linear(keys).tobytes() == B.export_linear(keys).tobytes()
    C = mk(0)
    assert C.carry_from(A) == keys.size
    assert C.export_linear(keys).tobytes() == A.export_linear(keys).tobytes()
