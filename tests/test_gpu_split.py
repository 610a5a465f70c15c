"""The split entry points (lookup_probe + pool_fwd, sparse_bwd_dedup + sparse_*_apply) with the
deduplication on a second stream, overlapping the pooling: every output bit-identical to the fused
calls on a twin table over consecutive steps (pooled output, rowrefs, slots, misses, unique rows,
counts, exported rows, accumulators, masters and linear states), the tiny workload also checked
against the oracle, and the misuse the host refuses (an apply without its dedup, twice, after a
flash or a touched write-back, or with other sizes), and caller-made rowrefs outside the table
acting exactly as misses."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ad_recommendation_amd import emb  # noqa: E402
from gen import synth, workloads as W  # noqa: E402
from tests import parity_util as P  # noqa: E402
from tests.test_gpu_parity import DT, TDT, gpu_step  # noqa: E402

pytestmark = pytest.mark.gpu

FTRL = (0.05, 1.0, 0.01, 0.1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    emb.lib()
    yield


def split_step(T, keys, offsets, grad, out_dtype, grad_dtype, lr, eps, ftrl=None):
    """One step through the split calls: probe, then pooling on the caller's stream while the
    dedup runs on a second stream, then the update after both."""
    dev = "cuda"
    F = T.n_fields
    k = torch.from_numpy(np.ascontiguousarray(keys)).to(dev)
    o = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int32)).to(dev)
    n_bags, nnz = o.numel() - 1, k.numel()
    out = torch.full((n_bags // F, T.out_width), float("nan"), dtype=TDT[out_dtype], device=dev)
    rowref = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    slot = torch.empty(max(nnz, 1), dtype=torch.int64, device=dev)
    n_miss = torch.zeros(1, dtype=torch.int64, device=dev)
    g = torch.from_numpy(np.ascontiguousarray(grad)).to(dev)
    ws = torch.empty(max(1, emb.bwd_workspace_bytes(T.h, n_bags, nnz)), dtype=torch.uint8, device=dev)
    uniq = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    cnt = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    nu = torch.full((1,), -1, dtype=torch.int64, device=dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    emb.lookup_probe(T.h, k, o, n_bags, nnz, rowref, slot, n_miss, stream=main)
    probed = torch.cuda.Event()
    probed.record(main)
    side.wait_event(probed)
    emb.sparse_bwd_dedup(T.h, rowref, o, n_bags, nnz, ws, stream=side)
    deduped = torch.cuda.Event()
    deduped.record(side)
    emb.pool_fwd(T.h, rowref, o, n_bags, nnz, out, DT[out_dtype], stream=main)
    main.wait_event(deduped)
    if ftrl is None:
        emb.sparse_adagrad_apply(T.h, n_bags, nnz, g, DT[grad_dtype], lr, eps, ws, uniq, cnt, nu,
                                 stream=main)
    else:
        emb.sparse_ftrl_apply(T.h, n_bags, nnz, g, DT[grad_dtype], *ftrl, ws, uniq, cnt, nu,
                              stream=main)
    torch.cuda.synchronize()
    U = int(nu.item())
    return {
        "out": out.cpu().numpy(),
        "rowref": rowref.cpu().numpy().view(np.uint32)[:nnz],
        "slot": slot.cpu().numpy()[:nnz],
        "n_miss": int(n_miss.item()),
        "n_unique": U,
        "unique": uniq.cpu().numpy().view(np.uint32)[:U],
        "count": cnt.cpu().numpy()[:U],
    }


def twin_tables(w, flags=0):
    dims = synth.field_dims(w)
    keys = synth.resident_keys(w)
    rows, master = synth.initial_state(w)
    Ts = []
    for _ in range(2):
        T = emb.Table(dims, DT[w.row_dtype], w.has_master, w.n_tables, w.load_factor, w.acc_init,
                      keys, rows, None, master, flags=flags)
        T.flash()
        Ts.append(T)
    return Ts, keys, rows, master, dims


def same_bits(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("w, ftrl", [
    (W.TINY, False),
    (W.scaled(W.F26, n_keys=500_000, batch=512), False),
    (W.scaled(W.F100, n_keys=400_000, batch=128), False),
    (W.scaled(W.F40_VARDIM, n_keys=400_000, batch=256), False),
    (W.scaled(W.F64_PASS, n_keys=1_000_000, batch=256), False),
    (W.scaled(W.F100, n_keys=400_000, batch=128), True),
], ids=["tiny", "f26", "f100", "f40", "f64", "f100-ftrl"])
def test_split_calls_bit_identical_to_fused(w, ftrl):
    (A, B), keys, rows, master, dims = twin_tables(w, emb.FLAG_FTRL if ftrl else 0)
    say(f"[split] {w.name} ftrl={ftrl}: {keys.size} keys")
    for s in range(2):
        bt = synth.batch(w, s)
        kk, off, grad = bt["keys"], bt["offsets"], bt["grad"]
        fa = FTRL if ftrl else None
        ra = gpu_step(A, kk, off, grad, w.out_dtype, w.grad_dtype, w.lr, w.eps, ftrl=fa)
        rb = split_step(B, kk, off, grad, w.out_dtype, w.grad_dtype, w.lr, w.eps, ftrl=fa)
        for name in ("out", "rowref", "slot", "unique", "count"):
            assert same_bits(ra[name], rb[name]), (name, s)
        assert ra["n_miss"] == rb["n_miss"] and ra["n_unique"] == rb["n_unique"]
        say(f"[split] {w.name} step {s}: nnz={kk.size} unique={rb['n_unique']} identical")
    for T in (A, B):
        emb.pass_writeback(T.h)
    ea, eb = A.export(keys), B.export(keys)
    for x, y in zip(ea, eb):
        if x is not None or y is not None:
            assert same_bits(x, y)
    if ftrl:
        assert same_bits(A.export_linear(keys), B.export_linear(keys))
    A.close()
    B.close()


def test_split_calls_match_the_oracle():
    w = W.TINY
    (T, _), keys, rows, master, dims = twin_tables(w)
    ot = P.oracle_table(w, keys, rows, master, dims)
    bud = P.Budget(ot)
    for s in range(2):
        bt = synth.batch(w, s)
        kk, off, grad = bt["keys"], bt["offsets"], bt["grad"]
        res = split_step(T, kk, off, grad, w.out_dtype, w.grad_dtype, w.lr, w.eps)
        out_o, nm = ot.forward(kk, off, w.out_dtype)
        assert nm == res["n_miss"]
        P.check_pooled(res["out"], out_o, P.pooled_scale(ot, kk, off, bud), w.out_dtype)
        u, _, _, ucnt = bud.oracle_step(ot, kk, off, grad, w.lr, w.eps)
        assert res["n_unique"] == u.size
        got = emb.table_rowref_keys(T.h, res["unique"])
        assert np.array_equal(got.view(np.uint64), ot.keys[u])
        assert np.array_equal(res["count"], ucnt)
    emb.pass_writeback(T.h)
    r, a, m = T.export(keys)
    P.check_state(ot, bud, keys, r, a, m)
    T.close()


def test_apply_needs_its_dedup():
    w = W.TINY
    (T, _), keys, _, _, _ = twin_tables(w)
    bt = synth.batch(w, 0)
    dev = "cuda"
    k = torch.from_numpy(bt["keys"]).to(dev)
    o = torch.from_numpy(bt["offsets"]).to(dev)
    g = torch.from_numpy(bt["grad"]).to(dev)
    n_bags, nnz = o.numel() - 1, k.numel()
    rowref = torch.empty(nnz, dtype=torch.int32, device=dev)
    ws = torch.empty(emb.bwd_workspace_bytes(T.h, n_bags, nnz), dtype=torch.uint8, device=dev)
    ws2 = torch.empty_like(ws)
    emb.lookup_probe(T.h, k, o, n_bags, nnz, rowref)

    def apply(wsx=ws, nb=n_bags, nz=nnz):
        emb.sparse_adagrad_apply(T.h, nb, nz, g, emb.EMB_F32, w.lr, w.eps, wsx)

    with pytest.raises(emb.EmbError) as e:
        apply()                                   # no dedup yet
    assert e.value.code == -6
    emb.sparse_bwd_dedup(T.h, rowref, o, n_bags, nnz, ws)
    with pytest.raises(emb.EmbError) as e:
        apply(wsx=ws2)                            # another workspace
    assert e.value.code == -6
    emb.sparse_bwd_dedup(T.h, rowref, o, n_bags, nnz, ws)
    with pytest.raises(emb.EmbError) as e:
        apply(nz=nnz - 4, nb=n_bags - 1)          # other sizes
    assert e.value.code == -6
    emb.sparse_bwd_dedup(T.h, rowref, o, n_bags, nnz, ws)
    apply()
    with pytest.raises(emb.EmbError) as e:
        apply()                                   # one apply per dedup
    assert e.value.code == -6
    emb.sparse_bwd_dedup(T.h, rowref, o, n_bags, nnz, ws)
    T.flash()
    with pytest.raises(emb.EmbError) as e:
        apply()                                   # a flash came in between
    assert e.value.code == -6
    torch.cuda.synchronize()
    T.close()


def test_touched_writeback_cancels_a_pending_dedup():
    w = W.TINY
    (T, _), keys, _, _, _ = twin_tables(w, emb.FLAG_TRACK_TOUCHED)
    bt = synth.batch(w, 0)
    dev = "cuda"
    k = torch.from_numpy(bt["keys"]).to(dev)
    o = torch.from_numpy(bt["offsets"]).to(dev)
    g = torch.from_numpy(bt["grad"]).to(dev)
    n_bags, nnz = o.numel() - 1, k.numel()
    rowref = torch.empty(nnz, dtype=torch.int32, device=dev)
    ws = torch.empty(max(emb.bwd_workspace_bytes(T.h, n_bags, nnz),
                         emb.writeback_workspace_bytes(T.h)), dtype=torch.uint8, device=dev)
    emb.lookup_probe(T.h, k, o, n_bags, nnz, rowref)
    emb.sparse_bwd_dedup(T.h, rowref, o, n_bags, nnz, ws)
    emb.pass_writeback_touched(T.h, ws)           # may overwrite the sorted pairs
    with pytest.raises(emb.EmbError) as e:
        emb.sparse_adagrad_apply(T.h, n_bags, nnz, g, emb.EMB_F32, w.lr, w.eps, ws)
    assert e.value.code == -6
    emb.sparse_bwd_dedup(T.h, rowref, o, n_bags, nnz, ws)
    emb.sparse_adagrad_apply(T.h, n_bags, nnz, g, emb.EMB_F32, w.lr, w.eps, ws)
    torch.cuda.synchronize()
    T.close()


def test_rowrefs_outside_the_table_count_as_misses():
    """pool_fwd and sparse_bwd_dedup take rowrefs from the caller: any value at or above the
    table's rowref space must act exactly like EMB_ROWREF_MISS (the kernels' own bounds checks;
    nothing outside the rows is read)."""
    w = W.TINY
    (A, B), keys, _, _, _ = twin_tables(w)
    space = int(A.info["rowref_space"])
    bt = synth.batch(w, 0)
    dev = "cuda"
    k = torch.from_numpy(bt["keys"]).to(dev)
    o = torch.from_numpy(bt["offsets"]).to(dev)
    g = torch.from_numpy(bt["grad"]).to(dev)
    n_bags, nnz = o.numel() - 1, k.numel()
    rowref = torch.empty(nnz, dtype=torch.int32, device=dev)
    emb.lookup_probe(A.h, k, o, n_bags, nnz, rowref)
    torch.cuda.synchronize()
    rr = rowref.cpu().numpy().view(np.uint32).copy()
    bad = np.array([space, space + 123, 0xFFFFFFFE, 0x80000000], dtype=np.uint32)
    pos = np.arange(0, nnz, max(1, nnz // 16))[:16]
    outside, missed = rr.copy(), rr.copy()
    outside[pos] = bad[np.arange(pos.size) % bad.size]
    missed[pos] = emb.ROWREF_MISS
    res = []
    for T, r in ((A, outside), (B, missed)):
        rt = torch.from_numpy(r.view(np.int32)).to(dev)
        out = torch.full((n_bags, 16), float("nan"), dtype=torch.float32, device=dev)
        emb.pool_fwd(T.h, rt, o, n_bags, nnz, out, emb.EMB_F32)
        ws = torch.empty(emb.bwd_workspace_bytes(T.h, n_bags, nnz), dtype=torch.uint8, device=dev)
        uniq = torch.empty(nnz, dtype=torch.int32, device=dev)
        cnt = torch.empty(nnz, dtype=torch.int32, device=dev)
        nu = torch.zeros(1, dtype=torch.int64, device=dev)
        emb.sparse_bwd_dedup(T.h, rt, o, n_bags, nnz, ws)
        emb.sparse_adagrad_apply(T.h, n_bags, nnz, g, emb.EMB_F32, w.lr, w.eps, ws, uniq, cnt, nu)
        torch.cuda.synchronize()
        U = int(nu.item())
        res.append((out.cpu().numpy(), uniq.cpu().numpy()[:U], cnt.cpu().numpy()[:U]))
        emb.pass_writeback(T.h)
    for x, y in zip(res[0], res[1]):
        assert same_bits(x, y)
    for x, y in zip(A.export(keys), B.export(keys)):
        if x is not None or y is not None:
            assert same_bits(x, y)
    A.close()
    B.close()
