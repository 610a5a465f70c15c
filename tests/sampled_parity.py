"""Sampled parity for tables too large for the whole-table oracle, over one or more consecutive
steps on the same table (each step's update is seen by the next).

The oracle checks samples it can compute one by one:
  * slots and rowrefs of 20,000 sampled occurrences per step, bit-exact, from per-home key counts
    (``oracle.slots_of_sample``) rather than a sort of the whole key set;
  * the number of distinct rows touched, bit-exact; the unique list's order;
  * the occurrence counts and the updated state (rows, accumulators, masters, FTRL linear state)
    of the step's picked rows: its hot rows -- the 64 most frequent keys and every key with more
    than 63 update pieces' worth of occurrences, whose segments may span more than 64 pieces and
    make the fixup read piece flags in a second round -- and 1 % of the other touched keys;
  * the pooled output of 1 sample in 64 (all of its bags) at the first step;
  * sampled untouched keys bit-identical after the first step.
The update oracle is one table over the picked keys of every step, fed each batch with every other
key's occurrences dropped (all bags and the full upstream gradient kept), which leaves those keys'
gradient sums as they are; it replays the steps in order, so later steps start from the oracle's
own state.  A step run with dyadic gradients (every element a multiple of 2^-7 in [-1, 1]) has
exact fp32 gradient sums on both sides: the accumulators of its hot rows, when every earlier update
of those rows was exact too, must then be within 2 ulp of the oracle's.
"""
from __future__ import annotations

import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from gen import synth
from oracle import emb_oracle as O
from tests import parity_util as P

ACC_EXACT_REL = 2.0 ** -22          # 2 ulp of an fp32 value, relative


def say(*a):
    print("[sampled]", *a, flush=True)
    sys.stdout.flush()


def positions(keys, want, chunk=1 << 24):
    """Index in `keys` of each of the sorted distinct keys `want` (each must occur once), in one
    pass over `keys` without sorting it."""
    pos = np.full(want.size, -1, dtype=np.int64)
    low = np.uint64((1 << 28) - 1)
    maybe = np.zeros(1 << 28, dtype=bool)            # filter on the low 28 bits first
    maybe[(want & low).astype(np.intp)] = True
    for a in range(0, keys.size, chunk):
        kc = keys[a:a + chunk]
        c = np.nonzero(maybe[(kc & low).astype(np.intp)])[0]
        i = np.minimum(np.searchsorted(want, kc[c]), want.size - 1)
        hit = want[i] == kc[c]
        pos[i[hit]] = a + c[hit]
    assert np.all(pos >= 0)
    return pos


def initial_rows(w, pos):
    """Initial rows (and fp32 master copies, when the workload keeps them) of the resident keys at
    positions `pos`, packed in that order with each key's field width; each field that holds one
    of them is regenerated once (fields on a thread pool).
    Returns (rows, master or None, offsets [n + 1] into both)."""
    dims = synth.field_dims(w).astype(np.int64)
    foff = synth.field_key_offsets(w)
    fld = np.searchsorted(foff, pos, side="right") - 1
    width = dims[fld]
    roff = np.concatenate([[0], np.cumsum(width)])
    out = np.empty(int(roff[-1]), dtype=np.float16 if w.row_dtype == "f16" else np.float32)
    mst = np.empty(int(roff[-1]), dtype=np.float32) if w.has_master else None

    def one(f):
        sel = np.nonzero(fld == f)[0]
        if sel.size:
            D = int(dims[f])
            r_f, m_f = synth.field_state(w, f)
            dst = (roff[sel][:, None] + np.arange(D)[None, :]).reshape(-1)
            src = ((pos[sel] - foff[f])[:, None] * D + np.arange(D)[None, :]).reshape(-1)
            out[dst] = r_f[src]
            if mst is not None:
                mst[dst] = m_f[src]
    with ThreadPoolExecutor(max(1, min(8, synth.worker_count()))) as ex:
        list(ex.map(one, range(w.n_fields)))
    return out, mst, roff


def piece_width(w, nnz, classed):
    """Occurrences per update piece of the library's backward for a batch of nnz occurrences."""
    import bench
    dims = synth.field_dims(w)
    return bench.piece_plan(nnz, int(dims.max()), w.row_dtype == "f16", classed)[0]


def hot_index(bcount, pw, n_top=64):
    """Indices of a batch's hot keys (by their occurrence counts): the n_top most frequent, and
    every key with more than 63 pieces' worth of occurrences."""
    top = np.argsort(-bcount, kind="stable")[:n_top]
    long_rows = np.nonzero(bcount > 63 * pw)[0]
    return np.unique(np.concatenate([top, long_rows]))


def restrict(bkeys, offsets, keep_sorted):
    """The batch with only the occurrences of keys in `keep_sorted` kept, every bag kept."""
    lens = np.diff(offsets.astype(np.int64))
    m = np.isin(bkeys, keep_sorted)
    bag_of = np.repeat(np.arange(lens.size, dtype=np.int64), lens)
    off = np.concatenate([[0], np.cumsum(np.bincount(bag_of[m], minlength=lens.size))])
    return bkeys[m].view(np.int64), off


class SampledRun:
    """Sampled checks of consecutive GPU steps on one table.  Construct it with the steps'
    batches before the first step (the samples are drawn up front), then call ``after_step`` once
    per step, after the step's write-back and before the next step."""

    def __init__(self, w, keys, batches, *, classed=False, unique_by_width=False, ftrl=None,
                 rowref_keys=None, seed=7):
        self.w = w
        self.keys = keys
        self.batches = batches
        self.ftrl = ftrl
        self.rowref_keys = rowref_keys
        self.unique_by_width = unique_by_width
        self.dims = synth.field_dims(w)
        self.simple = w.n_tables == 1 and np.all(self.dims == self.dims[0])
        r = np.random.default_rng(seed)
        self.st = []
        for s, bt in enumerate(batches):
            bkeys = bt["keys"].view(np.uint64)
            bk, bcount = np.unique(bkeys, return_counts=True)
            pw = piece_width(w, bkeys.size, classed)
            hot = hot_index(bcount, pw)
            rnd = np.unique(r.integers(0, bk.size, size=max(1, bk.size // 100)))
            pick = np.union1d(hot, rnd)
            occ = np.unique(r.integers(0, bkeys.size, size=20_000))
            self.st.append({"bk": bk, "bcount": bcount, "pick": pick, "hot": hot, "occ": occ,
                            "pw": pw, "long": int((bcount > 63 * pw).sum())})
            say(f"step {s}: {bkeys.size} lookups, {bk.size} distinct keys, piece width {pw}, "
                f"{hot.size} hot keys (max count {int(bcount.max())}, {self.st[-1]['long']} "
                f"beyond 63 pieces), {pick.size} picked")
        # pooled check at the first step: 1 sample in 64, all of its bags
        bt0 = batches[0]
        F = w.n_fields
        off64 = bt0["offsets"].astype(np.int64)
        lens = np.diff(off64)
        self.samp = np.arange(0, w.batch, 64)
        bag_ids = (self.samp[:, None] * F + np.arange(F)[None, :]).reshape(-1)
        sl = lens[bag_ids]
        self.sub_off = np.concatenate([[0], np.cumsum(sl)])
        sub_idx = np.repeat(off64[bag_ids], sl) + (np.arange(self.sub_off[-1]) -
                                                  np.repeat(self.sub_off[:-1], sl))
        self.sub_keys = bt0["keys"].view(np.uint64)[sub_idx]
        self.fwd_keys = np.unique(self.sub_keys)
        self.n_bags_sub = bag_ids.size
        # every key a check needs, located and regenerated once
        self.upd_keys = np.unique(np.concatenate([st["bk"][st["pick"]] for st in self.st]))
        occ_keys = [bt["keys"].view(np.uint64)[st["occ"]] for bt, st in zip(batches, self.st)]
        self.want = np.unique(np.concatenate(occ_keys + [self.upd_keys, self.fwd_keys]))
        t0 = time.perf_counter()
        self.wpos = positions(keys, self.want)
        say(f"{self.want.size} sampled keys located in {time.perf_counter() - t0:.0f}s")
        touched_any = np.unique(np.concatenate([st["bk"] for st in self.st]))
        upos = np.unique(r.integers(0, keys.size, size=5000))      # untouched candidates
        self.upos = upos[~np.isin(keys[upos], touched_any)]
        t0 = time.perf_counter()
        self.init, self.init_m, self.roff = initial_rows(w, np.concatenate([self.wpos, self.upos]))
        say(f"initial rows of {self.wpos.size + self.upos.size} keys regenerated in "
            f"{time.perf_counter() - t0:.0f}s")
        # oracle slots and ranks of every wanted key, per table
        t0 = time.perf_counter()
        nw = self.wpos.size
        ktab = O.table_of(keys, w.n_tables)
        self.slot_o = np.empty(nw, dtype=np.int64)
        self.rank_o = np.empty(nw, dtype=np.int64)
        for t in range(w.n_tables):
            mt = ktab == t
            keys_t = keys[mt] if w.n_tables > 1 else keys
            pos_in_t = (np.cumsum(mt) - 1)[self.wpos] if w.n_tables > 1 else self.wpos
            sel = np.nonzero(ktab[self.wpos] == t)[0]
            nh = O.n_home_slots(keys_t.size, w.load_factor)
            _, sl_t, rk_t = O.slots_of_sample(keys_t, nh, pos_in_t[sel])
            self.slot_o[sel] = sl_t
            self.rank_o[sel] = rk_t
        del ktab
        say(f"oracle slots of {nw} keys in {time.perf_counter() - t0:.0f}s")
        # the update oracle over the picked keys of every step
        usel = np.searchsorted(self.want, self.upd_keys)
        self.ot = O.Table(self.upd_keys, self.dims, w.row_dtype, w.has_master, w.n_tables,
                          w.load_factor, w.acc_init, P.take(self.init, self.roff, usel),
                          master=P.take(self.init_m, self.roff, usel), ftrl=ftrl is not None)
        self.bud = P.Budget(self.ot)
        self.exact_rows = np.ones(self.upd_keys.size, dtype=bool)   # every update so far exact

    def after_step(self, s, res, export, *, lr=None, eps=None, exact_grad=False,
                   export_linear=None):
        w, st, bt = self.w, self.st[s], self.batches[s]
        lr = w.lr if lr is None else lr
        eps = w.eps if eps is None else eps
        bkeys = bt["keys"].view(np.uint64)
        bk, bcount = st["bk"], st["bcount"]
        assert res["n_miss"] == 0
        assert res["n_unique"] == bk.size
        uq = res["unique"].astype(np.int64)
        if self.unique_by_width:
            epl = 8 if w.row_dtype == "f16" else 4
            wcls = np.ceil(np.log2(-(-self.dims.astype(np.int64) // epl))).astype(np.int64)
            ucls = wcls[(self.rowref_keys(res["unique"]).view(np.uint64) >>
                         np.uint64(48)).astype(np.int64)]
            assert np.all(np.diff(ucls) >= 0)
            assert np.all(np.diff(uq)[np.diff(ucls) == 0] > 0)
        else:
            assert np.all(np.diff(uq) > 0)
        # slots and rowrefs of the sampled occurrences
        occ = st["occ"]
        at = np.searchsorted(self.want, bkeys[occ])
        assert np.array_equal(res["slot"][occ], self.slot_o[at])
        pick_keys = bk[st["pick"]]
        if self.simple:
            assert np.array_equal(res["rowref"][occ].astype(np.int64), self.rank_o[at])
            pr = self.rank_o[np.searchsorted(self.want, pick_keys)]
            u_at = np.searchsorted(uq, pr)
            assert np.array_equal(uq[u_at], pr)
        else:
            assert np.array_equal(self.rowref_keys(res["rowref"][occ]).view(np.uint64), bkeys[occ])
            ukeys = self.rowref_keys(res["unique"]).view(np.uint64)
            order = np.argsort(ukeys)
            u_at = order[np.searchsorted(ukeys[order], pick_keys)]
            assert np.array_equal(ukeys[u_at], pick_keys)
        assert np.array_equal(res["count"][u_at], bcount[st["pick"]])
        say(f"step {s}: {occ.size} slots, {pick_keys.size} unique rows and counts match "
            f"(hot rows up to {int(bcount[st['hot']].max())} occurrences)")

        if s == 0:
            self._check_pooled(res)

        # update of the picked keys: the oracle replays this step on the batch restricted to the
        # keys it holds
        keys_r, off_r = restrict(bkeys, bt["offsets"], self.upd_keys)
        idx_pick = self.ot.key_index(pick_keys)
        prev_acc = {int(i): self.ot.acc[self.ot.roff[i]:self.ot.roff[i + 1]].copy() for i in
                    self.ot.key_index(bk[st["hot"]])}
        t0 = time.perf_counter()
        if self.ftrl is None:
            self.bud.oracle_step(self.ot, keys_r, off_r, bt["grad"], lr, eps)
        else:
            self.bud.oracle_step_ftrl(self.ot, keys_r, off_r, bt["grad"], *self.ftrl)
        say(f"step {s}: oracle update of {self.upd_keys.size} held keys over {keys_r.size} "
            f"occurrences in {time.perf_counter() - t0:.0f}s")
        rows_g, acc_g, mst_g = export(pick_keys)
        P.check_state(self.ot, self.bud, pick_keys, rows_g, acc_g,
                      mst_g if w.has_master else None,
                      None if self.ftrl is None else export_linear(pick_keys))
        # exact gradient sums: the hot rows' accumulators within 2 ulp
        touched_now = self.ot.key_index(bk)
        touched_now = touched_now[touched_now >= 0]
        if exact_grad:
            hot_keys = bk[st["hot"]]
            hidx = self.ot.key_index(hot_keys)
            ok = self.exact_rows[hidx]
            if ok.any():
                pos_in_pick = np.searchsorted(pick_keys, hot_keys[ok])
                wo = np.concatenate([[0], np.cumsum(self.ot.width[idx_pick])])
                for j, i in zip(pos_in_pick, hidx[ok]):
                    a, b = int(self.ot.roff[i]), int(self.ot.roff[i + 1])
                    g_acc = acc_g[wo[j]:wo[j + 1]].astype(np.float64)
                    o_acc = self.ot.acc[a:b].astype(np.float64)
                    assert np.all(np.abs(g_acc - o_acc) <= ACC_EXACT_REL * np.abs(o_acc)), \
                        f"hot key {int(self.ot.keys[i]):#x}: accumulator off by " \
                        f"{np.max(np.abs(g_acc - o_acc) / np.abs(o_acc)):.3g} relative"
                    assert np.all(o_acc >= prev_acc[int(i)].astype(np.float64))
                say(f"step {s}: {int(ok.sum())} hot rows' accumulators within 2 ulp "
                    f"(exact gradient sums)")
        else:
            self.exact_rows[touched_now] = False
        say(f"step {s}: {pick_keys.size} updated rows within budget")

        if s == 0:
            # untouched resident keys: bit-identical to their initial state
            nw = self.wpos.size
            usel = np.arange(nw, nw + self.upos.size)
            ru, au, mu = export(self.keys[self.upos])
            assert np.all(au == np.float32(w.acc_init))
            assert ru.tobytes() == P.take(self.init, self.roff, usel).tobytes()
            if self.init_m is not None:
                assert mu.tobytes() == P.take(self.init_m, self.roff, usel).tobytes()
            if self.ftrl is not None:
                assert np.all(export_linear(self.keys[self.upos]) == 0)
            say(f"{self.upos.size} untouched rows bit-identical")

    def _check_pooled(self, res):
        w = self.w
        fsel = np.searchsorted(self.want, self.fwd_keys)
        ot = O.Table(self.fwd_keys, self.dims, w.row_dtype, w.has_master, w.n_tables,
                     w.load_factor, w.acc_init, P.take(self.init, self.roff, fsel),
                     master=P.take(self.init_m, self.roff, fsel))
        out_o, miss_o = ot.forward(self.sub_keys.view(np.int64), self.sub_off, w.out_dtype)
        assert miss_o == 0
        P.check_pooled(res["out"][self.samp], out_o,
                       P.pooled_scale(ot, self.sub_keys.view(np.int64), self.sub_off),
                       w.out_dtype)
        say(f"{self.samp.size} sampled samples ({self.n_bags_sub} bags) pooled within tolerance")
