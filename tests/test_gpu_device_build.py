"""The layout built on the GPU (table_create_on_device) against the oracle and the host build.

Against the oracle: every key's slot must be the oracle's (ordered linear probing in closed form,
per table), and rowrefs must follow (table, slot) order -- the rank itself on one-table,
fixed-width tables.  Against the host build: after both tables are flashed, their arenas must be
byte-identical (key buckets, rowref prefixes, rows, accumulators, masters, field metadata), and so
must the host-side lookups and statistics.  Cases: every workload's shape at reduced size, load
factor 1.0 (long probe runs), tiny tables where many keys share a home, two tables, an empty key
set, and duplicate keys.  (At 150M and 800M keys the device-built layout is checked on sampled
keys by the PASS-scale tests.)"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ad_recommendation_amd import emb  # noqa: E402
from gen import synth, workloads as W  # noqa: E402
from oracle import emb_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    emb.lib()
    yield


def build_both(dims, rdt, master, n_tables, lf, keys, flags=0):
    ws = torch.empty(max(256, emb.table_build_workspace_bytes(dims, n_tables, lf, keys.size)),
                     dtype=torch.uint8, device="cuda")
    D = emb.Table(dims, rdt, master, n_tables, lf, 0.1, keys, flags=flags, device_ws=ws)
    del ws
    H = emb.Table(dims, rdt, master, n_tables, lf, 0.1, keys, flags=flags)
    return D, H


def assert_oracle_layout(T, keys, n_tables, lf, fixed_width):
    """Slots of every key equal the oracle's; rowrefs ascend with (table, slot)."""
    k = np.asarray(keys).view(np.uint64)
    if k.size == 0:
        return
    rr, sl = emb.table_key_rowref(T.h, k)
    tab = O.table_of(k, n_tables)
    slot_o = np.empty(k.size, dtype=np.int64)
    for t in range(n_tables):
        m = np.nonzero(tab == t)[0]
        if m.size:
            _, slot_o[m] = O.layout_closed_form(k[m], O.n_home_slots(m.size, lf))
    assert np.array_equal(sl, slot_o)
    order = np.lexsort((slot_o, tab))
    assert np.all(np.diff(rr[order].astype(np.int64)) > 0)
    if fixed_width and n_tables == 1:
        assert np.array_equal(rr[order].astype(np.int64), np.arange(k.size))


def assert_same(D, H, keys):
    for k in ("arena_bytes", "key_bytes", "n_keys", "rowref_space", "n_home", "n_buckets",
              "n_keys_t", "max_displacement", "unique_by_width"):
        assert D.info[k] == H.info[k], k
    assert abs(D.info["mean_displacement"] - H.info["mean_displacement"]) < 1e-9
    rd, sd = emb.table_key_rowref(D.h, keys)
    rh, shh = emb.table_key_rowref(H.h, keys)
    assert np.array_equal(rd, rh) and np.array_equal(sd, shh)
    D.flash()
    H.flash()
    torch.cuda.synchronize()
    assert torch.equal(D.arena, H.arena)


@pytest.mark.parametrize("w", [W.TINY, W.scaled(W.F26, n_keys=1_000_000, batch=16),
                               W.scaled(W.F100, n_keys=500_000, batch=16),
                               W.scaled(W.F40_VARDIM, n_keys=600_000, batch=16),
                               W.scaled(W.F64_PASS, n_keys=2_000_000, batch=16)],
                         ids=lambda w: w.name)
def test_device_build_matches_host_build(w):
    keys = synth.resident_keys(w)
    dims = synth.field_dims(w)
    rdt = emb.EMB_F16 if w.row_dtype == "f16" else emb.EMB_F32
    say(f"[device build] {w.name}: {keys.size} keys")
    D, H = build_both(dims, rdt, w.has_master, w.n_tables, w.load_factor, keys)
    assert_oracle_layout(D, keys, w.n_tables, w.load_factor, bool(np.all(dims == dims[0])))
    assert_same(D, H, keys)
    # state filled afterwards lands in the same places
    rows, master = synth.initial_state(w)
    D.fill_state(0, keys.size, rows, None, master)
    H.fill_state(0, keys.size, rows, None, master)
    D.flash()
    H.flash()
    torch.cuda.synchronize()
    assert torch.equal(D.arena, H.arena)


@pytest.mark.parametrize("n,lf,nt", [(1, 0.5, 1), (2, 1.0, 2), (40, 1.0, 1), (1000, 1.0, 2),
                                     (5000, 0.9, 1), (300_000, 1.0, 1), (0, 0.5, 1), (0, 0.5, 2)])
def test_device_build_edge_shapes(n, lf, nt):
    rng = np.random.default_rng(n + 17)
    raw = rng.choice(1 << 40, size=n, replace=False).astype(np.uint64)
    keys = (raw | (rng.integers(0, 3, size=n).astype(np.uint64) << np.uint64(48))).astype(np.uint64)
    keys = np.unique(keys)
    dims = [8, 24, 64]
    D, H = build_both(dims, emb.EMB_F16, True, nt, lf, keys, flags=emb.FLAG_FTRL)
    assert_oracle_layout(D, keys, nt, lf, False)
    assert_same(D, H, keys)


def test_device_build_rejects_duplicates():
    keys = np.array([5, 9, 11, 9], dtype=np.uint64)
    ws = torch.empty(emb.table_build_workspace_bytes([8], 1, 0.5, keys.size), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(emb.EmbError) as e:
        emb.Table([8], emb.EMB_F32, False, 1, 0.5, 0.1, keys, device_ws=ws)
    assert e.value.name == "EMB_EDUPKEY"
    with pytest.raises(emb.EmbError) as e:
        emb.Table([8], emb.EMB_F32, False, 1, 0.5, 0.1, keys, device_ws=ws[: 1024])
    assert e.value.name == "EMB_ENOSPACE"
