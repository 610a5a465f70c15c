"""Plain CPU oracle for one training step of a GPU-resident sparse embedding layer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the GPU path is checked against.  Only the test-suite, the
package's smoke entry and the benchmark's CPU-baseline leg may import it; the
product path never does.  It shares no code with the HIP/C++ library.

What it computes, and the passage each step follows (sources are the four web
pages this project is built from):

* Key layout -- a key is int64, the low 48 bits hold the raw id and the high
  16 bits the id of the table/field it belongs to, so every field lives in one
  unified hash table (Tencent PCG GPU training talk, "compute optimisation",
  unified hash table paragraph).
* Insert-free prebuilt table -- the whole hash-table structure is prepared
  off-GPU from the PASS's deduplicated keys and copied in bulk; there is no
  insert (Tencent talk, "optimisations of each stage", flash paragraph).
  The pages give no hash, probing scheme or layout.  The reading used here:
  a 64-bit multiply/xor-shift mix, a multiply-shift range reduction to a home
  slot, and ordered linear probing without wrap-around (keys sorted by
  (home, key) and placed at max(home, previous slot + 1)), which makes every
  key's slot a pure function of the key set.
* Multiple Hash -- the table may be decomposed into two smaller tables; here
  a key lives in table (key & 1) (Tencent talk, space optimisation).
* Dynamic embedding -- row width varies with the field (Tencent talk, space
  optimisation).
* Forward -- sum pooling of each CSR bag, as EmbeddingBag(mode='sum') over
  flat ids and offsets (JD article, section 4.2.1).
* Backward -- the gradient of a row is the sum of the upstream gradient slices
  of every occurrence of its key (sum-pooling derivative), and each touched row
  gets an element-wise Adagrad step: the squared gradient is added to a
  per-element accumulator that then scales the learning rate; rows and state
  of features absent from the batch are left untouched (JD article, 3.2.1).
* Mixed precision -- rows stored in fp16 with an fp32 weight copy used for the
  update, fp32 optimizer state (JD article, 3.2.3 and 5.2).
* FTRL -- the JD article (3.2.1) names FTRL as the Adagrad variant used for
  sparse features and says no more.  The reading taken: per-coordinate
  FTRL-Proximal as published by McMahan et al., "Ad Click Prediction: a View
  from the Trenches" (KDD 2013), Algorithm 1, with the squared-gradient sum n
  being the same per-element accumulator Adagrad keeps, a per-element linear
  state z (zero unless supplied), and the weight read from the stored row (or
  its fp32 master copy) so that rows may start from a random initialisation.

All sums are taken in float64 and rounded once to the stored type.
"""
from __future__ import annotations

import math
from collections import Counter
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

EMPTY = 0xFFFF_FFFF_FFFF_FFFF          # marks a free slot; field id 0xFFFF is therefore reserved
FIELD_SHIFT = 48
RAW_MASK = (1 << 48) - 1
MIX = 0x9E3779B97F4A7C15              # floor(2**64 / golden ratio), Knuth's multiplicative constant
M64 = (1 << 64) - 1
MISS = -1


# =========================================================================== hashing
def hash64(k: int) -> int:
    """64-bit mix of a key (Python integers, arithmetic mod 2**64).

    x = (k ^ (k >> 32)) * MIX;  x = (x ^ (x >> 32)) * MIX;  x ^= x >> 32.
    Each step is invertible, so distinct keys never share a hash value."""
    x = k & M64
    x = ((x ^ (x >> 32)) * MIX) & M64
    x = ((x ^ (x >> 32)) * MIX) & M64
    x ^= x >> 32
    return x


def hash64_array(keys: np.ndarray) -> np.ndarray:
    """hash64 over a uint64 array (numpy uint64 multiplication wraps mod 2**64)."""
    x = np.asarray(keys).view(np.uint64).copy()
    with np.errstate(over="ignore"):
        x ^= x >> np.uint64(32)
        x *= np.uint64(MIX)
        x ^= x >> np.uint64(32)
        x *= np.uint64(MIX)
        x ^= x >> np.uint64(32)
    return x


def n_home_slots(n_keys: int, load_factor: float) -> int:
    """Home-slot count of a table: ceil(N / load_factor), at least 1 (IEEE double division)."""
    return max(1, int(math.ceil(float(n_keys) / float(load_factor))))


def home_of(h, n_home: int):
    """Multiply-shift range reduction of the high 32 hash bits onto [0, n_home)."""
    if isinstance(h, np.ndarray):
        hi = (h >> np.uint64(32)).astype(np.uint64)
        return ((hi * np.uint64(n_home)) >> np.uint64(32)).astype(np.int64)
    return ((h >> 32) * n_home) >> 32


# =========================================================================== validation / routing
class OracleError(ValueError):
    pass


def validate_keys(keys: np.ndarray, n_fields: int) -> None:
    """A prebuilt key set must be distinct, avoid the EMPTY marker and name a known field."""
    k = np.asarray(keys).view(np.uint64)
    if np.any(k == np.uint64(EMPTY)):
        raise OracleError("EMPTY sentinel used as a key")
    if np.any((k >> np.uint64(FIELD_SHIFT)) >= np.uint64(n_fields)):
        raise OracleError("field id out of range")
    if np.unique(k).size != k.size:
        raise OracleError("duplicate key")


def table_of(keys: np.ndarray, n_tables: int) -> np.ndarray:
    """Multiple Hash routing: table (key & 1) when the table is split in two, else 0."""
    k = np.asarray(keys).view(np.uint64)
    if n_tables == 1:
        return np.zeros(k.shape, dtype=np.int64)
    return (k & np.uint64(1)).astype(np.int64)


# =========================================================================== layout
def layout_by_insertion(keys: Sequence[int], n_home: int) -> Dict[int, int]:
    """Ordered linear probing, built the textbook way: take the keys in
    (home, key) order and insert each at the first free slot at or after its
    home, never wrapping.  Returns {key: slot}.  Plain Python; small tables."""
    homes = {int(k): home_of(hash64(int(k)), n_home) for k in keys}
    occupied = set()
    slot_of = {}
    for k in sorted(homes, key=lambda kk: (homes[kk], kk)):
        s = homes[k]
        while s in occupied:
            s += 1
        occupied.add(s)
        slot_of[k] = s
    return slot_of


def layout_closed_form(keys: np.ndarray, n_home: int) -> Tuple[np.ndarray, np.ndarray]:
    """Same layout in closed form.  With keys sorted by (home, key), the i-th
    key lands at slot_i = max(home_i, slot_{i-1} + 1), i.e.
    slot_i = i + max_{j <= i}(home_j - j).  Returns (home, slot), both int64 and
    aligned with ``keys``."""
    k = np.asarray(keys).view(np.uint64)
    home = home_of(hash64_array(k), n_home)
    order = np.lexsort((k, home))
    hs = home[order]
    i = np.arange(hs.size, dtype=np.int64)
    slots_sorted = i + np.maximum.accumulate(hs - i) if hs.size else hs
    slot = np.empty_like(home)
    slot[order] = slots_sorted
    return home, slot


def slots_of_sample(keys: np.ndarray, n_home: int, sample: np.ndarray,
                    chunk: int = 1 << 24) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The layout of ``layout_closed_form`` for a few keys of a very large one-table key set,
    without sorting the set.

    In (home, key) order the i-th key sits at slot_i = max_{j <= i}(home_j + i - j).  Grouping
    the j by their home x, the best j of a group is its first, whose rank is P(x) = #{keys with
    home < x}; an x that no key has never beats the max (the first key at or after it does at
    least as well).  So a key of home h that is preceded by r keys of the same home has
    rank i = P(h) + r and slot = P(h) + r + max_{0 <= x <= h}(x - P(x)).
    Only counts of keys per home are needed.  Returns (home, slot, rank) of keys[sample]."""
    k = np.asarray(keys).view(np.uint64)
    sample = np.asarray(sample, dtype=np.int64)
    home = np.empty(k.size, dtype=np.int64)
    for a in range(0, k.size, chunk):
        home[a:a + chunk] = home_of(hash64_array(k[a:a + chunk]), n_home)
    counts = np.bincount(home, minlength=n_home)
    hs = home[sample]
    ks = k[sample]
    # r: keys of the same home with a smaller key (candidates found chunk by chunk)
    wanted = np.zeros(n_home, dtype=bool)
    wanted[hs] = True
    cand = np.concatenate([a + np.nonzero(wanted[home[a:a + chunk]])[0]
                           for a in range(0, k.size, chunk)])
    del wanted              # ascending positions, the sample among them
    order = np.lexsort((k[cand], home[cand]))      # candidates in (home, key) order
    place = np.empty(cand.size, dtype=np.int64)
    place[order] = np.arange(cand.size)
    first = np.searchsorted(home[cand][order], hs, side="left")
    r = place[np.searchsorted(cand, sample)] - first
    # P(h) and max_{x <= h}(x - P(x)), walking the home range in chunks
    P_at = np.empty(hs.size, dtype=np.int64)
    Q_at = np.empty(hs.size, dtype=np.int64)
    by_home = np.argsort(hs, kind="stable")
    hs_sorted = hs[by_home]
    p_run, q_run, s = 0, -(1 << 62), 0
    for a in range(0, n_home, chunk):
        b = min(n_home, a + chunk)
        c = counts[a:b]
        P = p_run + np.concatenate([[0], np.cumsum(c)[:-1]])
        Q = np.maximum(np.maximum.accumulate(np.arange(a, b, dtype=np.int64) - P), q_run)
        e = int(np.searchsorted(hs_sorted, b, side="left"))
        sel = by_home[s:e]
        P_at[sel] = P[hs[sel] - a]
        Q_at[sel] = Q[hs[sel] - a]
        s = e
        p_run = int(P[-1] + c[-1])
        q_run = int(Q[-1])
    rank = P_at + r
    return hs, rank + Q_at, rank


def key_array(keys: np.ndarray, slot: np.ndarray, n_home: int) -> np.ndarray:
    """The probed array: EMPTY everywhere except each key at its slot, with at
    least one EMPTY past the last key so every scan ends."""
    n = max(n_home, int(slot.max()) + 1 if slot.size else 0) + 1
    arr = np.full(n, EMPTY, dtype=np.uint64)
    arr[slot] = np.asarray(keys).view(np.uint64)
    return arr


def probe(arr: np.ndarray, n_home: int, k: int) -> int:
    """Look a key up: scan from its home slot until the key or an EMPTY slot."""
    k = int(k) & M64
    if k == EMPTY:
        return MISS
    s = home_of(hash64(k), n_home)
    while int(arr[s]) != EMPTY:
        if int(arr[s]) == k:
            return s
        s += 1
    return MISS


# =========================================================================== fp helpers
def f16(x: np.ndarray) -> np.ndarray:
    """Round to fp16, nearest-even, subnormals kept (numpy's conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# =========================================================================== table
class Table:
    """The prebuilt table with its rows and optimizer state, kept per key in
    the order the caller supplied the keys.

    dims[f] is field f's row width; rows are packed in key order with width
    dims[field(key)].  row_dtype is "f32" or "f16"; fp16 tables may keep an fp32
    master copy.  The Adagrad accumulator is fp32 per element."""

    def __init__(self, keys: np.ndarray, dims: Sequence[int], row_dtype: str, has_master: bool,
                 n_tables: int, load_factor: float, acc_init: float,
                 rows: np.ndarray, acc: Optional[np.ndarray] = None,
                 master: Optional[np.ndarray] = None, ftrl: bool = False,
                 linear: Optional[np.ndarray] = None):
        self.keys = np.ascontiguousarray(np.asarray(keys).view(np.uint64))
        self.dims = np.asarray(dims, dtype=np.int64)
        self.F = int(self.dims.size)
        validate_keys(self.keys, self.F)
        self.row_dtype = row_dtype
        self.has_master = bool(has_master and row_dtype == "f16")
        self.n_tables = n_tables
        self.load_factor = load_factor
        self.field = (self.keys >> np.uint64(FIELD_SHIFT)).astype(np.int64)
        self.width = self.dims[self.field]
        self.roff = np.concatenate([[0], np.cumsum(self.width)]).astype(np.int64)
        total = int(self.roff[-1])
        rdt = np.float32 if row_dtype == "f32" else np.float16
        self.rows = np.array(rows, dtype=rdt, copy=True).reshape(-1)
        assert self.rows.size == total
        self.acc = (np.full(total, acc_init, dtype=np.float32) if acc is None
                    else np.array(acc, dtype=np.float32, copy=True).reshape(-1))
        if self.has_master:
            self.master = (self.rows.astype(np.float32) if master is None
                           else np.array(master, dtype=np.float32, copy=True).reshape(-1))
        else:
            self.master = None
        # FTRL linear state z, fp32 per element
        if ftrl:
            self.linear = (np.zeros(total, dtype=np.float32) if linear is None
                           else np.array(linear, dtype=np.float32, copy=True).reshape(-1))
        else:
            self.linear = None
        # per-table layout
        self.tab = table_of(self.keys, n_tables)
        self.n_home = []
        self.home = np.empty(self.keys.size, dtype=np.int64)
        self.slot = np.empty(self.keys.size, dtype=np.int64)
        self._sorted = []   # per table: (sorted keys, key index in input order)
        for t in range(n_tables):
            idx = np.nonzero(self.tab == t)[0]
            nh = n_home_slots(idx.size, load_factor)
            self.n_home.append(nh)
            h, s = layout_closed_form(self.keys[idx], nh)
            self.home[idx] = h
            self.slot[idx] = s
            o = np.argsort(self.keys[idx], kind="stable")
            self._sorted.append((self.keys[idx][o], idx[o]))
        self.col = np.concatenate([[0], np.cumsum(self.dims)]).astype(np.int64)  # pooled column offsets

    # ------------------------------------------------------------------ lookup
    def key_index(self, qkeys: np.ndarray) -> np.ndarray:
        """Index (into the prebuilt key list) of each queried key, MISS if absent.
        Exact search of the key set, table by table (the set the probe must find)."""
        q = np.asarray(qkeys).view(np.uint64)
        out = np.full(q.shape, MISS, dtype=np.int64)
        qt = table_of(q, self.n_tables)
        for t in range(self.n_tables):
            sk, si = self._sorted[t]
            m = np.nonzero(qt == t)[0]
            if sk.size == 0 or m.size == 0:
                continue
            pos = np.searchsorted(sk, q[m])
            pos_c = np.minimum(pos, sk.size - 1)
            hit = sk[pos_c] == q[m]
            out[m[hit]] = si[pos_c[hit]]
        out[q == np.uint64(EMPTY)] = MISS
        return out

    def lookup(self, keys: np.ndarray, offsets: np.ndarray):
        """Resolve every occurrence of a batch.  An occurrence whose key is absent,
        or whose field id differs from its bag's field (bag j belongs to field
        j mod F), is a miss.  Returns (key index, table, slot), MISS for misses."""
        kidx = self.key_index(keys)
        bag = bag_of_occurrence(offsets)
        bag_field = bag % self.F
        ok = kidx >= 0
        ok[ok] &= self.field[kidx[ok]] == bag_field[ok]
        kidx = np.where(ok, kidx, MISS)
        tab = np.where(ok, self.tab[np.maximum(kidx, 0)], MISS)
        slot = np.where(ok, self.slot[np.maximum(kidx, 0)], MISS)
        return kidx, tab, slot

    def row64(self, i: int) -> np.ndarray:
        return self.rows[self.roff[i]:self.roff[i + 1]].astype(np.float64)

    # ------------------------------------------------------------------ probe statistics
    def scan_buckets(self, keys: np.ndarray, offsets: np.ndarray, per_bucket: int = 15):
        """Buckets each occurrence's probe reads, for collision monitoring by sampling (JD
        article, 4.3).  The probed array is cut into buckets of ``per_bucket`` consecutive slots
        (slot s lies in bucket s // per_bucket).  A scan runs for every occurrence whose key is
        not EMPTY and whose field is its bag's field; it starts at the key's home slot and stops
        at the key, or at the first EMPTY slot at or after home when the key is absent, and
        reads every bucket from the home slot's to the stop slot's.  Occurrences with no scan
        read 0 buckets.  Returns int64 [nnz]."""
        q = np.asarray(keys).view(np.uint64)
        bag_field = bag_of_occurrence(offsets) % self.F
        scanned = (q != np.uint64(EMPTY)) & ((q >> np.uint64(FIELD_SHIFT)).astype(np.int64) ==
                                             bag_field)
        kidx = self.key_index(q)
        qt = table_of(q, self.n_tables)
        out = np.zeros(q.size, dtype=np.int64)
        for t in range(self.n_tables):
            sel = np.nonzero(scanned & (qt == t))[0]
            if sel.size == 0:
                continue
            home = home_of(hash64_array(q[sel]), self.n_home[t])
            occ = np.sort(self.slot[self.tab == t])
            # last slot of the run of consecutive occupied slots that holds each occupied slot
            brk = np.nonzero(np.diff(occ) != 1)[0]
            run_last = np.repeat(occ[np.concatenate([brk, [occ.size - 1]])],
                                 np.diff(np.concatenate([[-1], brk, [occ.size - 1]]))) \
                if occ.size else occ
            p = np.searchsorted(occ, home)
            pc = np.minimum(p, max(occ.size - 1, 0))
            inside = (p < occ.size) & (occ[pc] == home) if occ.size else np.zeros(sel.size, bool)
            first_empty = np.where(inside, run_last[pc] + 1 if occ.size else home, home)
            hit = kidx[sel] >= 0
            stop = np.where(hit, self.slot[np.maximum(kidx[sel], 0)], first_empty)
            out[sel] = stop // per_bucket - home // per_bucket + 1
        return out

    # ------------------------------------------------------------------ forward
    def forward(self, keys: np.ndarray, offsets: np.ndarray, out_dtype: str,
                bags: Optional[np.ndarray] = None):
        """Sum pooling (EmbeddingBag mode='sum'): out[b, col_f:col_f+D_f] is the
        float64 sum of the rows of bag j = b*F + f, misses adding nothing,
        rounded once to out_dtype.  With ``bags`` only those bags are computed
        and a dict {bag: pooled vector} is returned.  Returns (out, n_miss)."""
        offsets = np.asarray(offsets, dtype=np.int64)
        n_bags = offsets.size - 1
        if n_bags % self.F:
            raise OracleError("bag count is not a multiple of the field count")
        B = n_bags // self.F
        kidx, _, _ = self.lookup(keys, offsets)
        n_miss = int((kidx < 0).sum())
        cast = f32 if out_dtype == "f32" else f16
        if bags is not None:
            res = {}
            for j in np.asarray(bags, dtype=np.int64):
                f = int(j % self.F)
                acc = np.zeros(int(self.dims[f]), dtype=np.float64)
                for i in range(offsets[j], offsets[j + 1]):
                    if kidx[i] >= 0:
                        acc += self.row64(int(kidx[i]))
                res[int(j)] = cast(acc)
            return res, n_miss
        out = np.zeros((B, int(self.col[-1])), dtype=np.float64)
        bag = bag_of_occurrence(offsets)
        for f in range(self.F):
            D = int(self.dims[f])
            sel = np.nonzero((bag % self.F == f) & (kidx >= 0))[0]
            if sel.size == 0:
                continue
            # gather each occurrence's row (float64) and add it into its sample's block
            ro = self.roff[kidx[sel]]
            gathered = self.rows[ro[:, None] + np.arange(D)[None, :]].astype(np.float64)
            np.add.at(out, (bag[sel] // self.F, slice(int(self.col[f]), int(self.col[f]) + D)),
                      gathered)
        return cast(out), n_miss

    # ------------------------------------------------------------------ backward
    def touched(self, keys: np.ndarray, offsets: np.ndarray):
        """Deduplicated touched rows of a batch: distinct (table, slot) of the
        non-miss occurrences with their occurrence counts, ascending by
        (table, slot).  Returns (key index [U], table [U], slot [U], count [U])."""
        kidx, tab, slot = self.lookup(keys, offsets)
        hit = kidx[kidx >= 0]
        if hit.size == 0:
            z = np.zeros(0, dtype=np.int64)
            return z, z, z, z
        u, cnt = np.unique(hit, return_counts=True)
        order = np.lexsort((self.slot[u], self.tab[u]))
        u, cnt = u[order], cnt[order]
        return u, self.tab[u], self.slot[u], cnt

    def row_grads(self, keys: np.ndarray, offsets: np.ndarray, grad: np.ndarray,
                  only: Optional[np.ndarray] = None) -> Dict[int, np.ndarray]:
        """g_u = sum over the occurrences of row u of the upstream gradient slice
        of the occurrence's bag (float64; fp16 gradients widen exactly).  A key
        repeated inside one bag contributes once per occurrence.  Returns
        {key index: g}; with ``only`` just those key indices."""
        offsets = np.asarray(offsets, dtype=np.int64)
        kidx, _, _ = self.lookup(keys, offsets)
        bag = bag_of_occurrence(offsets)
        G = np.asarray(grad)
        sel = np.nonzero(kidx >= 0)[0]
        if only is not None:
            sel = sel[np.isin(kidx[sel], np.asarray(only))]
        out: Dict[int, np.ndarray] = {}
        # group occurrences by key, add their gradient slices
        order = np.argsort(kidx[sel], kind="stable")
        sel = sel[order]
        ks = kidx[sel]
        if ks.size == 0:
            return out
        starts = np.concatenate([[0], np.nonzero(np.diff(ks))[0] + 1, [ks.size]])
        for a, b in zip(starts[:-1], starts[1:]):
            u = int(ks[a])
            f = int(self.field[u])
            c0, D = int(self.col[f]), int(self.dims[f])
            occ = sel[a:b]
            rows_g = G[bag[occ] // self.F, c0:c0 + D].astype(np.float64)
            out[u] = rows_g.sum(axis=0)
        return out

    def adagrad_rows(self, g: Dict[int, np.ndarray], lr: float, eps: float) -> None:
        """Element-wise Adagrad on the given rows only:
        acc <- acc + g^2;  delta = lr * g / (sqrt(acc) + eps), with the new acc;
        fp32 rows:            w <- w - delta
        fp16 rows + master:   master <- master - delta;  row <- fp16(master)
        fp16 rows, no master: row <- fp16(row - delta)
        computed in float64 from the stored values and rounded once."""
        lr = float(np.float32(lr))
        eps = float(np.float32(eps))
        for u, gu in g.items():
            a, b = int(self.roff[u]), int(self.roff[u + 1])
            acc_new = self.acc[a:b].astype(np.float64) + gu * gu
            delta = lr * gu / (np.sqrt(acc_new) + eps)
            self.acc[a:b] = f32(acc_new)
            if self.row_dtype == "f32":
                self.rows[a:b] = f32(self.rows[a:b].astype(np.float64) - delta)
            elif self.has_master:
                m = f32(self.master[a:b].astype(np.float64) - delta)
                self.master[a:b] = m
                self.rows[a:b] = f16(m)
            else:
                self.rows[a:b] = f16(self.rows[a:b].astype(np.float64) - delta)

    def ftrl_rows(self, g: Dict[int, np.ndarray], alpha: float, beta: float, l1: float,
                  l2: float) -> None:
        """Per-coordinate FTRL-Proximal on the given rows only (McMahan et al. 2013,
        Algorithm 1), element by element, with w the stored weight (the fp32 master
        copy when the table keeps one, else the row):
            n' = n + g^2
            sigma = (sqrt(n') - sqrt(n)) / alpha
            z' = z + g - sigma * w
            w' = 0                                                 if |z'| <= l1
               = -(z' - sign(z') * l1) / ((beta + sqrt(n')) / alpha + l2)   otherwise
        n', z' and w' are computed in float64 from the stored values and rounded once
        to their stored types (w' like the Adagrad step: fp32 row, or fp32 master and
        fp16 row = fp16(master), or fp16 row)."""
        assert self.linear is not None, "table keeps no FTRL linear state"
        alpha, beta = float(np.float32(alpha)), float(np.float32(beta))
        l1, l2 = float(np.float32(l1)), float(np.float32(l2))
        for u, gu in g.items():
            a, b = int(self.roff[u]), int(self.roff[u + 1])
            n_old = self.acc[a:b].astype(np.float64)
            n_new = n_old + gu * gu
            w_src = self.master if self.has_master else self.rows
            w_old = w_src[a:b].astype(np.float64)
            sigma = (np.sqrt(n_new) - np.sqrt(n_old)) / alpha
            z_new = self.linear[a:b].astype(np.float64) + gu - sigma * w_old
            shrunk = z_new - np.sign(z_new) * l1
            w_new = np.where(np.abs(z_new) <= l1, 0.0,
                             -shrunk / ((beta + np.sqrt(n_new)) / alpha + l2))
            self.acc[a:b] = f32(n_new)
            self.linear[a:b] = f32(z_new)
            if self.row_dtype == "f32":
                self.rows[a:b] = f32(w_new)
            elif self.has_master:
                m = f32(w_new)
                self.master[a:b] = m
                self.rows[a:b] = f16(m)
            else:
                self.rows[a:b] = f16(w_new)

    def backward(self, keys: np.ndarray, offsets: np.ndarray, grad: np.ndarray,
                 lr: float, eps: float):
        """Dedup, reduce and apply Adagrad to the touched rows.  Returns the
        touched set as (key index, table, slot, count), ascending by (table, slot)."""
        t = self.touched(keys, offsets)
        g = self.row_grads(keys, offsets, grad)
        self.adagrad_rows(g, lr, eps)
        return t

    # ------------------------------------------------------------------ state access
    def state_of(self, i: int):
        a, b = int(self.roff[i]), int(self.roff[i + 1])
        return (self.rows[a:b].copy(), self.acc[a:b].copy(),
                None if self.master is None else self.master[a:b].copy())


# =========================================================================== CSR helpers
def bag_of_occurrence(offsets: np.ndarray) -> np.ndarray:
    """Bag index of every occurrence of a CSR batch (offsets[j] <= i < offsets[j+1])."""
    offsets = np.asarray(offsets, dtype=np.int64)
    lens = np.diff(offsets)
    return np.repeat(np.arange(lens.size, dtype=np.int64), lens)


def dedup_counts_plain(rowids: Sequence[int]) -> List[Tuple[int, int]]:
    """Distinct ids with their occurrence counts, ascending (Counter based)."""
    c = Counter(int(r) for r in rowids)
    return sorted(c.items())


def pool_plain(rows_by_key: Dict[int, np.ndarray], keys: Sequence[int], offsets: Sequence[int]):
    """Sum pooling written as loops: one float64 vector per bag (missing keys add nothing)."""
    out = []
    for j in range(len(offsets) - 1):
        acc = None
        for i in range(offsets[j], offsets[j + 1]):
            r = rows_by_key.get(int(keys[i]))
            if r is None:
                continue
            acc = r.astype(np.float64) if acc is None else acc + r
        out.append(acc)
    return out
