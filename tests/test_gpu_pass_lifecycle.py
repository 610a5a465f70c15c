"""PASS lifecycle on the GPU: the end-of-PASS write-back of only the touched rows, the incremental
export list, and carrying state into the next PASS's table.

Each PASS's table holds the deduplicated keys of its own batches plus some others, built from one
store of initial state (the workload's); the second PASS's table takes the first one's state for
the keys they share.  The oracle runs every batch of both PASSes on one table over all keys, so
after the second PASS each key's state must equal the oracle's: keys of the second PASS as read
from its table, keys only in the first PASS from the first table's image.  The touched write-back
is also compared bit for bit with the full write-back of a twin table that ran the same steps."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ad_recommendation_amd import emb  # noqa: E402
from gen import synth, workloads as W  # noqa: E402
from tests import parity_util as P  # noqa: E402
from tests.test_gpu_parity import DT, gpu_step  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    emb.lib()
    yield


def pass_table(w, dims, keys, rows, master, roff, idx, flags=0, with_state=True):
    T = emb.Table(dims, DT[w.row_dtype], w.has_master, w.n_tables, w.load_factor, w.acc_init,
                  keys[idx], P.take(rows, roff, idx) if with_state else None, None,
                  P.take(master, roff, idx) if with_state else None, flags=flags)
    return T


def pass_keys(w, keys, batches, seed):
    """Indices (ascending) of a PASS's key set: its batches' deduplicated keys plus 10% others."""
    used = np.unique(np.concatenate([b["keys"] for b in batches]))
    sorter = np.argsort(keys)
    pos = sorter[np.searchsorted(keys, used, sorter=sorter)]
    assert np.array_equal(keys[pos], used)
    extra = np.random.default_rng(seed).choice(keys.size, keys.size // 10, replace=False)
    return np.union1d(pos, extra)


def units_of(T, ks):
    gran = T.field_dim // int(T.info["granule"])
    return int(gran[(np.asarray(ks, dtype=np.uint64) >> np.uint64(48)).astype(np.int64)].sum())


def run_step(T, w, bt):
    return gpu_step(T, bt["keys"], bt["offsets"], bt["grad"], w.out_dtype, w.grad_dtype, w.lr, w.eps)


@pytest.mark.parametrize("w", [W.TINY, W.scaled(W.F40_VARDIM, n_keys=400_000, batch=256),
                               W.scaled(W.F100, n_keys=200_000, batch=64)],
                         ids=lambda w: w.name)
def test_two_pass_lifecycle_against_oracle(w):
    dims = synth.field_dims(w)
    keys = synth.resident_keys(w)
    rows, master = synth.initial_state(w)
    roff = synth.row_offsets(w)
    batches = [synth.batch(w, s) for s in range(4)]
    idx1 = pass_keys(w, keys, batches[:2], 11)
    idx2 = pass_keys(w, keys, batches[2:], 12)
    say(f"[lifecycle] {w.name}: PASS 1 {idx1.size} keys, PASS 2 {idx2.size} keys, "
        f"shared {np.intersect1d(idx1, idx2).size}")
    ot = P.oracle_table(w, keys, rows, master, dims)
    bud = P.Budget(ot)

    # PASS 1: a tracking table and a twin written back whole
    A = pass_table(w, dims, keys, rows, master, roff, idx1, emb.FLAG_TRACK_TOUCHED)
    A_full = pass_table(w, dims, keys, rows, master, roff, idx1)
    A.flash()
    A_full.flash()
    touched = set()
    for s in range(2):
        ra = run_step(A, w, batches[s])
        run_step(A_full, w, batches[s])
        touched.update(emb.table_rowref_keys(A.h, ra["unique"]).tolist())
        bud.oracle_step(ot, batches[s]["keys"], batches[s]["offsets"], batches[s]["grad"], w.lr, w.eps)
    n_units = A.writeback_touched()
    emb.pass_writeback(A_full.h)
    tk = np.array(sorted(touched), dtype=np.int64)
    assert n_units == units_of(A, tk)
    k1 = keys[idx1]
    ra_, aa_, ma_ = A.export(k1)
    rf_, af_, mf_ = A_full.export(k1)
    assert ra_.tobytes() == rf_.tobytes() and aa_.tobytes() == af_.tobytes()
    if w.has_master:
        assert ma_.tobytes() == mf_.tobytes()
    # incremental export: exactly the touched keys, in rowref order
    dirty = emb.table_dirty_keys(A.h, clear=True)
    assert np.array_equal(np.sort(dirty), tk)
    rr, _ = emb.table_key_rowref(A.h, dirty)
    assert np.all(np.diff(rr.astype(np.int64)) > 0)
    assert emb.table_dirty_keys(A.h).size == 0
    P.check_state(ot, bud, k1.view(np.uint64), ra_, aa_, ma_)
    A_full.close()
    say(f"[lifecycle] {w.name}: PASS 1 written back ({n_units} units)")

    # PASS 2: built from the store, then the keys shared with PASS 1 take its state
    B = pass_table(w, dims, keys, rows, master, roff, idx2, emb.FLAG_TRACK_TOUCHED)
    shared = np.intersect1d(idx1, idx2)
    assert B.carry_from(A) == shared.size
    B.flash()
    for s in range(2, 4):
        run_step(B, w, batches[s])
        bud.oracle_step(ot, batches[s]["keys"], batches[s]["offsets"], batches[s]["grad"], w.lr, w.eps)
    B.writeback_touched()
    k2 = keys[idx2]
    rb, ab, mb = B.export(k2)
    P.check_state(ot, bud, k2.view(np.uint64), rb, ab, mb)
    only1 = keys[np.setdiff1d(idx1, idx2)]
    if only1.size:
        r1, a1, m1 = A.export(only1)
        P.check_state(ot, bud, only1.view(np.uint64), r1, a1, m1)
    say(f"[lifecycle] {w.name}: ok")
    A.close()
    B.close()


@pytest.mark.parametrize("ws_kind", ["min", "large"])
def test_touched_writeback_repeats_and_pieces(ws_kind):
    """Three write-backs in one PASS (after step 0, after step 1, with nothing new): each moves only
    the rows updated since the one before, and the image ends bit-identical to a full write-back.
    The smallest workspace splits the first write-back (over 200k rows of the 26-field workload)
    into several pieces."""
    w = W.F26
    dims = synth.field_dims(w)
    keys = synth.resident_keys(w)
    rows, master = synth.initial_state(w)
    A = emb.Table(dims, DT[w.row_dtype], w.has_master, w.n_tables, w.load_factor, w.acc_init,
                  keys, rows, None, master, flags=emb.FLAG_TRACK_TOUCHED)
    A_full = emb.Table(dims, DT[w.row_dtype], w.has_master, w.n_tables, w.load_factor,
                       w.acc_init, keys, rows, None, master)
    A.flash()
    A_full.flash()
    wmin = emb.writeback_workspace_bytes(A.h)
    ws = torch.empty(wmin if ws_kind == "min" else 256 << 20, dtype=torch.uint8, device="cuda")
    got = []
    union = set()
    for s in range(2):
        bt = synth.batch(w, s)
        ra = run_step(A, w, bt)
        run_step(A_full, w, bt)
        step_keys = emb.table_rowref_keys(A.h, ra["unique"])
        n = A.writeback_touched(ws)
        assert n == units_of(A, step_keys)
        got.append(n)
        union.update(step_keys.tolist())
        say(f"[lifecycle] F26 step {s}: {n} units written back ({ws_kind} workspace)")
    assert got[0] > 2 * 32768   # more than one piece with the smallest workspace
    assert A.writeback_touched(ws) == 0
    emb.pass_writeback(A_full.h)
    r1, a1, _ = A.export(keys)
    r2, a2, _ = A_full.export(keys)
    assert r1.tobytes() == r2.tobytes() and a1.tobytes() == a2.tobytes()
    # both write-backs were dirty-marked; the list holds the union of the two steps' rows
    assert np.array_equal(np.sort(emb.table_dirty_keys(A.h)), np.array(sorted(union), dtype=np.int64))
    # a new flash clears the device bitmap: nothing to write back
    A.flash()
    assert A.writeback_touched(ws) == 0
    A.close()
    A_full.close()
