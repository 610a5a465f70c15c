"""The C-ABI library on the CPU: it loads, exports every declared symbol, builds the same table
layout as the oracle (bit-exact slots), and rejects bad input with the documented codes.  No
device work runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

from ad_recommendation_amd import emb
from gen import synth, workloads as W
from oracle import emb_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "emb.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = emb.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(emb.exported_symbols()) == set(names)


def _table(w, **kw):
    keys = synth.resident_keys(w)
    rows, master = synth.initial_state(w)
    T = emb.Table(synth.field_dims(w), emb.EMB_F16 if w.row_dtype == "f16" else emb.EMB_F32,
                  w.has_master, w.n_tables, w.load_factor, w.acc_init, keys, rows, None, master,
                  **kw)
    return T, keys, rows, master


@pytest.mark.parametrize("w", [W.TINY, W.scaled(W.F26, n_keys=300_000, batch=64),
                               W.scaled(W.F40_VARDIM, n_keys=400_000, batch=64),
                               W.scaled(W.F100, n_keys=200_000, batch=16)])
def test_layout_slots_bit_exact_with_oracle(w):
    T, keys, rows, master = _table(w)
    ot = O.Table(keys, synth.field_dims(w), w.row_dtype, w.has_master, w.n_tables, w.load_factor,
                 w.acc_init, rows, master=master)
    rr, sl = emb.table_key_rowref(T.h, keys)
    assert np.array_equal(sl, ot.slot)
    assert T.info["n_home"][:w.n_tables] == ot.n_home
    # rowrefs: ascending in (table, slot); distinct; map back to their keys
    order = np.lexsort((ot.slot, ot.tab))
    assert np.all(np.diff(rr[order].astype(np.int64)) > 0)
    assert np.array_equal(emb.table_rowref_keys(T.h, rr), keys.view(np.int64))
    # the host image holds every key's initial row and state
    sample = keys[:: max(1, keys.size // 500)]
    r2, a2, m2 = T.export(sample)
    idx = ot.key_index(sample)
    want_r = np.concatenate([ot.state_of(int(i))[0] for i in idx])
    assert r2.tobytes() == want_r.tobytes()
    assert np.all(a2 == np.float32(w.acc_init))
    if w.has_master:
        assert m2.tobytes() == np.concatenate([ot.state_of(int(i))[2] for i in idx]).tobytes()
    assert abs(T.info["mean_displacement"] - (ot.slot - ot.home).mean()) < 1e-9
    assert T.info["max_displacement"] == int((ot.slot - ot.home).max())


def test_absent_keys_miss_on_host_probe():
    T, keys, _, _ = _table(W.TINY)
    absent = (keys[:100] ^ np.uint64(1 << 47))
    rr, sl = emb.table_key_rowref(T.h, absent)
    assert np.all(rr == emb.ROWREF_MISS) and np.all(sl == -1)
    rr, sl = emb.table_key_rowref(T.h, np.array([-1], dtype=np.int64))
    assert rr[0] == emb.ROWREF_MISS


def _err(fn, *a, **k):
    with pytest.raises(emb.EmbError) as e:
        fn(*a, **k)
    return e.value.name


def test_create_errors():
    k = np.arange(1, 101, dtype=np.int64)
    r = np.zeros(100 * 8, dtype=np.float32)
    mk = emb.table_create_from_prebuilt
    assert _err(mk, [8], emb.EMB_F32, False, 1, 0.5, 0.1, np.r_[k, k[:1]], np.zeros(101 * 8, np.float32)) == "EMB_EDUPKEY"
    assert _err(mk, [8], emb.EMB_F32, False, 1, 0.5, 0.1, np.r_[k, [-1]], np.zeros(101 * 8, np.float32)) == "EMB_ESENTINEL"
    assert _err(mk, [8], emb.EMB_F32, False, 1, 0.5, 0.1, np.r_[k, [(1 << 48) | 3]], np.zeros(101 * 8, np.float32)) == "EMB_ERANGE"
    assert _err(mk, [8], emb.EMB_F32, False, 1, 0.0, 0.1, k, r) == "EMB_EINVAL"
    assert _err(mk, [8], emb.EMB_F32, False, 1, 1.5, 0.1, k, r) == "EMB_EINVAL"
    assert _err(mk, [12], emb.EMB_F32, False, 1, 0.5, 0.1, k, None) == "EMB_EINVAL"
    assert _err(mk, [512], emb.EMB_F32, False, 1, 0.5, 0.1, k, None) == "EMB_EINVAL"
    assert _err(mk, [8], emb.EMB_F32, True, 1, 0.5, 0.1, k, r) == "EMB_EINVAL"
    assert _err(mk, [8], emb.EMB_F32, False, 3, 0.5, 0.1, k, r) == "EMB_EINVAL"
    # null key pointer with a positive count
    d = (ctypes.c_int32 * 1)(8)
    desc = emb.EmbTableDesc(1, d, 0, 0, 1, 0.5, 0.1, 0)
    h = ctypes.c_void_p()
    assert emb.lib().table_create_from_prebuilt(ctypes.byref(desc), None, 5, None, None, None,
                                                ctypes.byref(h)) == -1


def test_rows_null_and_master_from_rows():
    k = (np.arange(1, 51, dtype=np.int64))
    T = emb.Table([8], emb.EMB_F32, False, 1, 0.5, 0.25, k)
    r, a, _ = T.export(k[:3])
    assert np.all(r == 0) and np.all(a == np.float32(0.25))
    rows16 = (np.arange(50 * 8) % 7 - 3).astype(np.float16) / np.float16(8)
    T2 = emb.Table([8], emb.EMB_F16, True, 1, 0.5, 0.1, k, rows16)
    r, a, m = T2.export(k)
    assert r.tobytes() == rows16.tobytes() and m.tobytes() == rows16.astype(np.float32).tobytes()
    master = np.random.default_rng(0).standard_normal(50 * 8).astype(np.float32)
    T3 = emb.Table([8], emb.EMB_F16, True, 1, 0.5, 0.1, k, None, None, master)
    r, a, m = T3.export(k)
    assert r.tobytes() == master.astype(np.float16).tobytes()      # fp16 RNE of the master copy
    assert m.tobytes() == master.tobytes()


def test_host_fp16_rounding_matches_numpy_on_hard_cases():
    vals = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24, 2 ** -25, 3 * 2 ** -26, 2 ** -14 - 2 ** -26,
                     65504, 65520, 65519.99, -0.0, 6.1e-5, 5.96e-8, 1e-9, -2.5e-6], dtype=np.float32)
    k = np.arange(1, 3, dtype=np.int64)
    m = np.zeros(16, dtype=np.float32)
    m[:vals.size] = vals
    T = emb.Table([8], emb.EMB_F16, True, 1, 0.5, 0.1, k, None, None, m)
    r, _, _ = T.export(k)
    with np.errstate(over="ignore"):
        assert r.tobytes() == m.astype(np.float16).tobytes()


def test_call_errors_without_device_work():
    T, keys, _, _ = _table(W.TINY)
    L = emb.lib()
    nul = None
    A = 1 << 20   # a fake, 16-byte aligned "device" address: no call below reaches the device
    # lookup arguments are checked before the table state
    assert L.lookup_pool_fwd(T.h, A, A, 4, 4, A, 7, A, nul, nul, nul) == -1       # bad out dtype
    assert L.lookup_pool_fwd(T.h, nul, A, 4, 4, A, 0, A, nul, nul, nul) == -1     # null keys
    assert L.lookup_pool_fwd(T.h, A, A, -1, 4, A, 0, A, nul, nul, nul) == -1      # negative size
    assert L.lookup_pool_fwd(T.h, A, A, 4, 4, A + 8, 0, A, nul, nul, nul) == -1   # misaligned out
    assert L.lookup_pool_fwd(T.h, A, A, 0, 4, A, 0, A, nul, nul, nul) == -1       # occurrences, no bags
    assert L.lookup_pool_fwd(T.h, A, A, 4, 4, A, 0, A, nul, nul, nul) == -6       # before flash
    assert L.sparse_adagrad_bwd(T.h, A, A, 4, 4, A, 0, 0.1, 1e-8, A, 16, nul, nul, nul, nul) == -5  # ws too small
    assert L.sparse_adagrad_bwd(T.h, A, A, 4, 4, A, 0, 0.1, 1e-8, A, 1 << 20, nul, A, nul, nul) == -1  # count w/o unique
    assert L.sparse_adagrad_bwd(T.h, A, A, 4, 4, A + 4, 0, 0.1, 1e-8, A, 1 << 20, nul, nul, nul, nul) == -1  # misaligned grad
    assert L.sparse_adagrad_bwd(T.h, A, A, 4, 4, A, 0, 0.1, 1e-8, A, 1 << 20, nul, nul, nul, nul) == -6
    # the split halves check the same way
    assert L.lookup_probe(T.h, nul, A, 4, 4, A, nul, nul, nul) == -1               # null keys
    assert L.lookup_probe(T.h, A, A, 4, 4, nul, nul, nul, nul) == -1               # null rowref
    assert L.lookup_probe(T.h, A, A, 4, 4, A, nul, nul, nul) == -6                 # before flash
    assert L.pool_fwd(T.h, A, A, 4, 4, A, 7, nul) == -1                            # bad out dtype
    assert L.pool_fwd(T.h, A, A, 4, 4, nul, 0, nul) == -1                          # null output
    assert L.pool_fwd(T.h, A, A, 4, 4, A, 0, nul) == -6                            # before flash
    assert L.sparse_bwd_dedup(T.h, A, nul, 4, 4, A, 1 << 20, nul) == -1            # null offsets
    assert L.sparse_bwd_dedup(T.h, A, A, 4, 4, A, 16, nul) == -5                   # ws too small
    assert L.sparse_bwd_dedup(T.h, A, A, 4, 4, A, 1 << 20, nul) == -6              # before flash
    assert L.sparse_adagrad_apply(T.h, 4, 4, nul, 0, 0.1, 1e-8, A, 1 << 20, nul, nul, nul, nul) == -1  # null grad
    assert L.sparse_adagrad_apply(T.h, 4, 4, A, 0, 0.1, 1e-8, A, 1 << 20, nul, nul, nul, nul) == -6
    assert L.sparse_ftrl_apply(T.h, 4, 4, A, 0, 0.0, 1.0, 0.0, 0.0, A, 1 << 20, nul, nul, nul, nul) == -1  # alpha 0
    assert L.pass_flash(T.h, 256, 16, nul) == -5                                    # arena too small
    assert L.pass_flash(T.h, 100, 1 << 40, nul) == -1                               # misaligned
    assert L.pass_writeback(T.h, nul) == -6
    assert emb.lib().emb_last_error()


def test_multifield_bag_count_must_divide():
    w = W.scaled(W.F26, n_keys=26_000, batch=4)
    T, _, _, _ = _table(w)
    assert emb.lib().lookup_pool_fwd(T.h, 8, 8, 27, 4, 8, 0, 8, None, None, None) == -1


def test_workspace_size_grows_with_batch():
    T, _, _, _ = _table(W.TINY)
    a = emb.bwd_workspace_bytes(T.h, 256, 1024)
    b = emb.bwd_workspace_bytes(T.h, 256 * 64, 1024 * 64)
    assert 0 < a < b and b >= 16 * 1024 * 64


@pytest.mark.parametrize("w", [W.scaled(W.F26, n_keys=120_000, batch=16),
                               W.scaled(W.F40_VARDIM, n_keys=160_000, batch=16),
                               W.scaled(W.F100, n_keys=90_000, batch=16)])
def test_fill_state_in_pieces_equals_create_with_state(w):
    """Streaming a PASS's state into the image field by field gives the same image as handing it
    all over at create."""
    T_all, keys, rows, master = _table(w)
    rdt = emb.EMB_F16 if w.row_dtype == "f16" else emb.EMB_F32
    T = emb.Table(synth.field_dims(w), rdt, w.has_master, w.n_tables, w.load_factor, w.acc_init,
                  keys)
    foff = synth.field_key_offsets(w)
    acc_all = np.full(rows.size, 0.25, dtype=np.float32)
    roff = synth.row_offsets(w)
    for f in range(w.n_fields):
        r_f, m_f = synth.field_state(w, f)
        a, b = int(foff[f]), int(foff[f + 1])
        if w.has_master and f % 2:        # odd fields: rows derived from the master copy
            T.fill_state(a, b - a, None, acc_all[roff[a]:roff[b]], m_f)
        else:
            T.fill_state(a, b - a, r_f, acc_all[roff[a]:roff[b]], m_f)
    r1, a1, m1 = T_all.export(keys)
    r2, a2, m2 = T.export(keys)
    assert np.array_equal(r1.view(np.uint8), r2.view(np.uint8))
    assert np.all(a2 == 0.25)
    if w.has_master:
        assert np.array_equal(m1.view(np.uint32), m2.view(np.uint32))


def test_fill_state_errors():
    w = W.scaled(W.F100, n_keys=20_000, batch=4)
    T_all, keys, rows, master = _table(w)
    T = emb.Table(synth.field_dims(w), emb.EMB_F16, True, 1, w.load_factor, w.acc_init, keys)
    with pytest.raises(emb.EmbError) as e:
        T.fill_state(keys.size - 1, 2, rows[:128])
    assert e.value.name == "EMB_EINVAL"
    with pytest.raises(emb.EmbError) as e:
        T.fill_state(-1, 1, rows[:64])
    assert e.value.name == "EMB_EINVAL"
    T.fill_state(0, 0)                    # empty range: nothing to do
    w2 = W.scaled(W.F26, n_keys=20_000, batch=4)
    T2, keys2, rows2, _ = _table(w2)
    with pytest.raises(emb.EmbError) as e:
        T2.fill_state(0, 1, None, None, np.zeros(16, dtype=np.float32))
    assert e.value.name == "EMB_EINVAL"


@pytest.mark.parametrize("w", [W.TINY, W.scaled(W.F26, n_keys=300_000, batch=64),
                               W.scaled(W.F40_VARDIM, n_keys=400_000, batch=64),
                               W.scaled(W.F100, n_keys=200_000, batch=16)])
def test_bench_plan_mirrors_the_library(w):
    """bench.py's byte model re-derives the backward's sort and piece plans; the workspace size
    those plans imply must equal the library's bwd_workspace_bytes for every batch size."""
    import bench
    T, _, _, _ = _table(w)
    dims = synth.field_dims(w)
    space, classed = T.info["rowref_space"], bool(T.info["unique_by_width"])
    al = lambda x: (x + 255) & ~255  # noqa: E731
    for nnz in (1, 1000, 325_000, 1_500_000, 5_000_000, 32_768_000, 50_331_648):
        ipt, tiles, bits = bench.sort_plan(nnz, space, classed)
        pw, n_pieces = bench.piece_plan(nnz, int(dims.max()), w.row_dtype == "f16", classed)
        bins = (1 << bits) + 1
        tg = 16 if tiles >= 512 * 16 else tiles // 512 if tiles >= 512 else 1
        groups = -(-tiles // tg)
        npc = max(n_pieces, 1)
        want = (4 * al(4 * (nnz + 1)) + al(4 * bins * max(tiles, 1)) + al(4 * bins * max(groups, 1))
                + al(4 * bins) + al(64) + al(4 * (tiles + 1)) + 2 * al(4 * npc * int(dims.max()))
                + al(4 * npc) + al(8 * npc))
        assert emb.bwd_workspace_bytes(T.h, w.n_fields, nnz) == want, nnz


def test_product_path_never_imports_the_oracle():
    """The binding and the package load without the oracle (no CPU fallback path exists)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import ad_recommendation_amd; "
            "from ad_recommendation_amd import emb; emb.lib(); "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "assert not bad, bad; print('ok')" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_mixed_width_state_arrays_are_padded_by_a_widest_row():
    # each state array of a mixed-width table is followed by one widest row, so a rowref that
    # names a row narrower than its bag's field cannot reach the next array or the metadata
    w = W.scaled(W.F40_VARDIM, n_keys=20_000, batch=8)
    keys = synth.resident_keys(w)
    dims = synth.field_dims(w)
    T = emb.Table(dims, emb.EMB_F16, True, w.n_tables, w.load_factor, w.acc_init, keys)
    E, D = T.info["total_elems"], int(dims.max())
    # rows (2 B), accumulator (4 B) and master (4 B), each padded, then 256-byte alignment
    assert T.info["state_bytes"] >= (E + D) * (2 + 4 + 4)
    F = emb.Table([16] * 4, emb.EMB_F32, False, 1, 0.5, 0.1,
                  (np.arange(1000, dtype=np.uint64) | (np.uint64(1) << np.uint64(48))))
    assert F.info["state_bytes"] < (F.info["total_elems"] * 8) + 1024   # fixed width: no pad


def test_bench_algorithmic_bytes_follow_the_byte_model():
    """B_alg and B_min of one step, on a hand-made batch whose counts are known: 2 fields of width
    8 (fp16 rows, fp32 master, fp16 output and gradient), 2 samples, 7 occurrences of 3 rows, with
    one row crossing no piece.  The sort's passes are not part of B_alg."""
    import bench
    from dataclasses import replace
    w = replace(W.scaled(W.F100, n_keys=100, batch=2), n_fields=2, dim=8)
    st = {"nnz": 7, "U": 3, "bags": 4, "occ_elems": 7 * 8, "bag_elems": 4 * 8,
          "u_elems_inside": 3 * 8, "u_elems_cross": 0, "u_cross": 0, "n_pieces": 1, "pdim": 8,
          "classed": False}
    # forward: per occurrence key 8 + probe 12 + rowref 4 + row 8*2; per bag offset 4 + out 8*2
    fwd = 7 * (8 + 12 + 4 + 16) + 4 * (4 + 16)
    # backward: per occurrence rowref 4 + gradient 8*2; per bag offset 4; per row its state
    # read and written (row 2, acc 4, master 4 bytes per element, twice) plus rowref and count
    bwd = 7 * (4 + 16) + 4 * 4 + 3 * 8 * (2 * 2 + 8 + 8) + 12 * 3
    assert bench.b_alg_bytes(st, w) == fwd + bwd
    # compulsory bytes: each datum once -- one probe hit and one row read per distinct row
    bmin = 7 * 12 + 3 * 12 + 3 * 8 * 2 + 4 * (4 + 16) + 4 * (4 + 16) + 7 * 4 + 3 * 8 * (2 * 2 + 8 + 8)
    assert bench.b_min_bytes(st, w) == bmin
    assert bench.b_alg_bytes(st, w, ftrl=True) == fwd + bwd + 3 * 8 * 8
    assert "sort_scatter" in bench.SORT_KERNELS and "update_pieces" not in bench.SORT_KERNELS
