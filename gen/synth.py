"""Seeded synthetic inputs for the embedding training step.

This module only draws data: resident feature keys, initial rows, CSR batches
of multi-hot bags and upstream gradients.  It holds none of the method's
arithmetic (no hashing, probing, pooling, deduplication or optimizer step), so
both the CPU oracle and the GPU path can consume the same inputs without
sharing any computation.

Every draw comes from ``numpy.random.SeedSequence([1234, workload.seed_id,
stream, index])`` so each stream is reproducible on its own.

Input shapes follow the pages:
* keys are int64 with the field id in the high 16 bits and the raw id in the
  low 48 bits (Tencent PCG talk, unified hash table paragraph);
* a batch is CSR: flat keys plus int32 bag offsets, one bag per
  (sample, field), sample-major (Tencent talk, preprocessing: features are
  turned into CSR samples that form CSR batches);
* popularity is Zipf-like per field, or for the long-tail workload 90 % of the
  distinct ids of a batch occur once or twice (MetaApp/DeepRec article, 3.1).
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

from .workloads import DIM_CHOICES, Workload

ROOT_SEED = 1234
# stream ids
S_KEYS, S_ROWS, S_STATE, S_DIMS, S_BAGLEN, S_BATCHKEYS, S_GRADS = range(7)

RAW_MASK = (1 << 48) - 1


def rng_for(w: Workload, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [ROOT_SEED, w.seed_id, stream, index])))


# --------------------------------------------------------------------------- fields
def field_dims(w: Workload) -> np.ndarray:
    """Row width per field (int32 [F])."""
    if w.dim is not None:
        return np.full(w.n_fields, w.dim, dtype=np.int32)
    r = rng_for(w, S_DIMS)
    return np.asarray(DIM_CHOICES, dtype=np.int32)[r.integers(0, len(DIM_CHOICES), w.n_fields)]


def field_key_counts(w: Workload) -> np.ndarray:
    """Resident keys per field: an even split, the first ``N mod F`` fields get one more."""
    base, extra = divmod(w.n_keys, w.n_fields)
    c = np.full(w.n_fields, base, dtype=np.int64)
    c[:extra] += 1
    return c


def compose(field: np.ndarray, raw: np.ndarray) -> np.ndarray:
    """Pack a field id into the high 16 bits above a 48-bit raw id (uint64).

    This is the key encoding the caller hands to the library, not part of the
    lookup itself."""
    return (np.asarray(field, dtype=np.uint64) << np.uint64(48)) | (
        np.asarray(raw, dtype=np.uint64) & np.uint64(RAW_MASK))


def _distinct_raw(r: np.random.Generator, n: int, bits: int) -> np.ndarray:
    """n distinct uniform raw ids, kept in generation order."""
    out = np.empty(0, dtype=np.uint64)
    need = n
    while need > 0:
        draw = r.integers(0, 1 << bits, size=need + need // 64 + 16, dtype=np.uint64)
        cat = np.concatenate([out, draw])
        _, first = np.unique(cat, return_index=True)
        first.sort()
        out = cat[first][:n]
        need = n - out.size
    return out


def field_keys(w: Workload, f: int) -> np.ndarray:
    """The resident keys of field f (uint64), in generation order."""
    n_f = int(field_key_counts(w)[f])
    r = rng_for(w, S_KEYS, f)
    raw = _distinct_raw(r, n_f, w.raw_bits)
    fid = 0 if w.field0_only else f
    return compose(np.full(n_f, fid, dtype=np.uint64), raw)


def worker_count() -> int:
    """Threads for per-field generation (numpy releases the GIL inside bulk draws and sorts)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def per_field(w: Workload, fn):
    """[fn(f) for every field], fields drawn in parallel when the workload is large.  Every field
    has its own stream, so the result does not depend on the thread count."""
    if w.n_keys < (1 << 24) or worker_count() == 1:
        return [fn(f) for f in range(w.n_fields)]
    with ThreadPoolExecutor(worker_count()) as ex:
        return list(ex.map(fn, range(w.n_fields)))


@functools.lru_cache(maxsize=4)
def _resident_keys_cached(w: Workload) -> np.ndarray:
    parts = per_field(w, lambda f: field_keys(w, f))
    out = np.empty(w.n_keys, dtype=np.uint64)
    o = 0
    for p in parts:
        out[o:o + p.size] = p
        o += p.size
    return out


def resident_keys(w: Workload) -> np.ndarray:
    """All resident keys (uint64 [N]), field 0's first, each field in generation order."""
    k = _resident_keys_cached(w)
    k.flags.writeable = False
    return k


def field_key_offsets(w: Workload) -> np.ndarray:
    c = field_key_counts(w)
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int64)


# --------------------------------------------------------------------------- rows / state
def field_state(w: Workload, f: int):
    """Initial rows of field f's keys (packed in key order, D_f elements each) and their fp32
    master copy when the workload keeps one.

    Rows are N(0, row_std) drawn in fp32 from the field's own stream.  fp16 rows are the
    round-to-nearest fp16 of that draw, and the draw itself is the master copy.
    Returns (rows_f, master_f_or_None)."""
    n = int(field_key_counts(w)[f]) * int(field_dims(w)[f])
    draw = rng_for(w, S_ROWS, f).standard_normal(n, dtype=np.float32) * np.float32(w.row_std)
    if w.row_dtype == "f32":
        return draw, None
    return draw.astype(np.float16), (draw if w.has_master else None)


def initial_state(w: Workload):
    """Initial rows of every resident key (packed in key order, width D of the key's field) and
    the fp32 master copy when the workload keeps one: the fields' ``field_state`` in field order.
    The Adagrad accumulator starts at ``w.acc_init`` and is not materialised here."""
    parts = [field_state(w, f) for f in range(w.n_fields)]
    rows = np.concatenate([p[0] for p in parts])
    master = np.concatenate([p[1] for p in parts]) if w.has_master else None
    return rows, master


def row_offsets(w: Workload) -> np.ndarray:
    """Element offset of each resident key's row inside the packed rows array (int64 [N+1])."""
    dims = field_dims(w)
    per_key = np.repeat(dims.astype(np.int64), field_key_counts(w))
    return np.concatenate([[0], np.cumsum(per_key)])


# --------------------------------------------------------------------------- batches
def bag_lengths(w: Workload, b: int) -> np.ndarray:
    """Bag length per (sample, field): int64 [B, F]."""
    if w.bag_kind == "fixed":
        return np.full((w.batch, w.n_fields), int(w.bag_mean), dtype=np.int64)
    r = rng_for(w, S_BAGLEN, b)
    L = r.poisson(w.bag_mean, size=(w.batch, w.n_fields)).astype(np.int64)
    if w.bag_min > 0:
        np.maximum(L, w.bag_min, out=L)
    return L


@functools.lru_cache(maxsize=8)
def _zipf_cdf(n: int, alpha: float) -> np.ndarray:
    p = np.arange(1, n + 1, dtype=np.float64) ** (-alpha)
    c = np.cumsum(p)
    c /= c[-1]
    return c


def zipf_ranks(r: np.random.Generator, n_draw: int, n_items: int, alpha: float) -> np.ndarray:
    """Zipf(alpha) ranks in [1, n_items], truncated at n_items (inverse CDF of the
    truncated law, equivalent to rejecting draws above n_items)."""
    cdf = _zipf_cdf(int(n_items), float(alpha))
    u = r.random(n_draw)
    # search in ascending order of u (each search starts where the previous one ended), then put
    # the results back in draw order
    order = np.argsort(u, kind="stable")
    idx = np.empty(n_draw, dtype=np.int64)
    idx[order] = np.searchsorted(cdf, u[order], side="right")
    return np.minimum(idx, n_items - 1) + 1


def _longtail_occurrences(r: np.random.Generator, n_f: int, n_items: int, alpha: float):
    """Occurrence list (indices into the field's keys) for one (batch, field):
    90 % of the distinct ids occur once or twice, the remaining 10 % are a
    head whose multiplicities follow a Zipf(alpha)-shaped profile.

    With U_h head ids, the tail has 9*U_h ids of multiplicity 1 or 2 (fair
    coin), and head rank k has multiplicity max(3, round(3*(U_h/k)**alpha)).
    U_h is the smallest value whose expected total reaches n_f; the difference
    between the drawn total and n_f is put on head rank 1."""
    if n_f == 0:
        return np.empty(0, dtype=np.int64)

    def head_mult(uh):
        k = np.arange(1, uh + 1, dtype=np.float64)
        return np.maximum(3, np.rint(3.0 * (uh / k) ** alpha)).astype(np.int64)

    def expected(uh):
        return 13.5 * uh + int(head_mult(uh).sum())

    lo, hi = 1, max(1, n_f)
    while lo < hi:
        mid = (lo + hi) // 2
        if expected(mid) >= n_f:
            hi = mid
        else:
            lo = mid + 1
    uh = lo
    ut = 9 * uh
    if 10 * uh > n_items:
        raise ValueError("long-tail batch needs more distinct keys than the field holds")
    tail = 1 + r.integers(0, 2, size=ut).astype(np.int64)
    head = head_mult(uh)
    resid = n_f - int(tail.sum() + head.sum())
    if resid >= 0:
        head[0] += resid
    else:
        # take the excess back from the largest head multiplicities, keeping >= 3
        need = -resid
        for i in range(uh):
            give = min(need, int(head[i]) - 3)
            head[i] -= give
            need -= give
            if need == 0:
                break
        if need:  # very small batches only: drop tail duplicates, then tail ids
            twos = np.nonzero(tail == 2)[0]
            k = min(need, twos.size)
            tail[twos[:k]] = 1
            need -= k
        if need:
            raise ValueError("batch too small for the long-tail construction")
    ids = r.choice(n_items, size=uh + ut, replace=False)
    mult = np.concatenate([head, tail])
    occ = np.repeat(ids, mult)
    return r.permutation(occ)


def batch(w: Workload, b: int, *, with_grad: bool = True) -> Dict[str, np.ndarray]:
    """One CSR batch: ``keys`` int64 [nnz], ``offsets`` int32 [B*F+1] with bag
    j = sample*F + field, ``grad`` [B, sum(D)] (fp32 or fp16) when requested,
    ``lengths`` int64 [B, F]."""
    F, B = w.n_fields, w.batch
    L = bag_lengths(w, b)
    flatL = L.reshape(-1)
    offsets64 = np.concatenate([[0], np.cumsum(flatL)])
    nnz = int(offsets64[-1])
    if nnz >= (1 << 31):
        raise ValueError("nnz exceeds int32 offsets")
    offsets = offsets64.astype(np.int32)
    keys = np.empty(nnz, dtype=np.uint64)
    counts = field_key_counts(w)
    foffs = field_key_offsets(w)
    allkeys = resident_keys(w)
    r = rng_for(w, S_BATCHKEYS, b)
    if w.key_kind == "uniform":
        idx = r.integers(0, w.n_keys, size=nnz)
        keys[:] = allkeys[idx]
    else:
        for f in range(F):
            Lf = L[:, f]
            n_f = int(Lf.sum())
            if n_f == 0:
                continue
            starts = offsets64[np.arange(B) * F + f]
            within = np.arange(n_f) - np.repeat(np.cumsum(Lf) - Lf, Lf)
            pos = np.repeat(starts, Lf) + within
            if w.key_kind == "zipf":
                ranks = zipf_ranks(r, n_f, int(counts[f]), w.zipf_alpha)
                sel = ranks - 1
            elif w.key_kind == "longtail":
                sel = _longtail_occurrences(r, n_f, int(counts[f]), w.zipf_alpha)
            else:
                raise ValueError(w.key_kind)
            keys[pos] = allkeys[foffs[f] + sel]
    out = {"keys": keys.view(np.int64), "offsets": offsets, "lengths": L}
    if with_grad:
        out["grad"] = upstream_grad(w, b)
    return out


def upstream_grad(w: Workload, b: int) -> np.ndarray:
    """Upstream gradient of the pooled output, N(0,1) drawn in fp32 ([B, sum(D)])."""
    width = int(field_dims(w).sum())
    r = rng_for(w, S_GRADS, b)
    dt = np.float16 if w.grad_dtype == "f16" else np.float32
    g = np.empty((w.batch, width), dtype=dt)
    step = max(1, (1 << 24) // max(width, 1))
    for s in range(0, w.batch, step):
        e = min(w.batch, s + step)
        g[s:e] = r.standard_normal((e - s, width), dtype=np.float32).astype(dt)
    return g


def dyadic_grad(w: Workload, b: int) -> np.ndarray:
    """An upstream gradient of the pooled output whose every element is a multiple of 2^-7 in
    [-1, 1] (uniform over the 257 values), in the workload's gradient dtype, where such values are
    exact.  A sum of up to 2^17 of them needs at most 24 significant bits, so every fp32 partial
    sum of a row's gradient is exact in any order: the summed gradient of even the hottest row is
    the same on every side."""
    width = int(field_dims(w).sum())
    r = rng_for(w, S_GRADS, 1_000_000 + b)
    dt = np.float16 if w.grad_dtype == "f16" else np.float32
    g = np.empty((w.batch, width), dtype=dt)
    step = max(1, (1 << 24) // max(width, 1))
    for s in range(0, w.batch, step):
        e = min(w.batch, s + step)
        g[s:e] = (r.integers(-128, 129, size=(e - s, width)).astype(np.float32) /
                  np.float32(128.0)).astype(dt)
    return g
