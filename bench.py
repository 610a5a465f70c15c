"""Benchmark of one training step of the GPU-resident embedding layer (forward probe + sum pool,
backward dedup + segmented gradient reduction + sparse Adagrad) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload f64|f26|tiny|f100|f40]

The default workload is the PASS-scale one: 800M resident keys in one unified table (dim 32, fp16
rows, fp32 accumulators, ~167 GB of HBM), 64 fields, batch 131,072, the PASS's 50 batches cycled.

Prints one JSON line: rows looked up + updated per second over K timed steps (inputs resident in
HBM, a ring of distinct synthetic batches cycled in order so each step sees the previous step's
update), the roofline of the dominant kernel (algorithmic bytes per launch / its event-timed
duration, against 8 TB/s), and the CPU oracle's rate on a stated sub-batch as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
from concurrent.futures import ThreadPoolExecutor
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "embedding rows looked up+updated/sec (fwd+bwd) and achieved HBM GB/s vs peak"
# FTRL-Proximal hyperparameters besides alpha (the workload's learning rate)
FTRL_BETA, FTRL_L1, FTRL_L2 = 1.0, 0.01, 0.1
# the oracle's CPU baseline runs on every n-th sample of batch 0 (all fields of each such
# sample): about 0.3-0.8M lookups, a few seconds of single-threaded oracle work per step
CPU_SUBSAMPLE = {"tiny_f1_k10k_d16_fp32": 1, "f26_k4m_d16_fp32_zipf1.05": 1,
                 "f100_k50m_d64_fp16_zipf1.1": 64, "f40_k20m_vardim_fp16_2tables_longtail": 8,
                 "f64_k800m_d32_fp16_pass": 64}
SORT_KERNELS = ("sort_hist", "sort_scan", "sort_scatter")
KERNEL_SRC = os.path.join(ROOT, "ad_recommendation_amd", "csrc", "emb_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_src_hash() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


# --------------------------------------------------------------------------- byte model
def piece_plan(nnz, max_dim, row_f16, classed=False):
    """Piece length and count of the library's update kernels."""
    epl = 8 if row_f16 else 4
    lanes, gsl = (max_dim + epl - 1) // epl, 0
    while (1 << gsl) < lanes:
        gsl += 1
    ipr = 64 >> gsl
    br = 2 if row_f16 else 4
    r = (nnz + ipr * 131072 - 1) // (ipr * 131072)
    r = max(r, (192 + ipr - 1) // ipr)   # pieces of at least 192 occurrences
    r = min(max(r, br), 256 // ipr)
    rounds = (r + br - 1) // br * br
    if classed:   # mixed widths sorted by width class: full pieces
        rounds = 256 // ipr
    return rounds * ipr, (nnz + rounds * ipr - 1) // (rounds * ipr)


def batch_stats(w, bt, dims, rowref, classed=False):
    """Per-batch counts the byte model needs, from the batch and the rows its keys resolve to."""
    off = bt["offsets"]
    F = w.n_fields
    bag = np.repeat(np.arange(off.size - 1, dtype=np.int64), np.diff(off.astype(np.int64)))
    width = dims[bag % F].astype(np.int64)           # row width of each occurrence
    rr = rowref.astype(np.int64)
    if classed:                                      # the backward sorts by (width class, rowref)
        epl = 8 if w.row_dtype == "f16" else 4
        cls = np.ceil(np.log2(-(-dims.astype(np.int64) // epl))).astype(np.int64)
        key = (cls[bag % F] << 40) | rr
        order = np.argsort(key, kind="stable")
        srr = key[order]
        sw = width[order]
    elif np.all(dims == dims[0]):                    # one width: no permutation needed
        srr = np.sort(rr)
        sw = width
    else:
        order = np.argsort(rr, kind="stable")
        srr = rr[order]
        sw = width[order]
    heads = np.concatenate([[True], srr[1:] != srr[:-1]])
    starts = np.nonzero(heads)[0]
    ends = np.concatenate([starts[1:], [srr.size]]) - 1
    pw, n_pieces = piece_plan(srr.size, int(dims.max()), w.row_dtype == "f16", classed)
    cross = (starts // pw) != (ends // pw)          # finished by the fixup kernel
    uw = sw[starts]
    return {
        "nnz": int(rr.size), "U": int(starts.size), "bags": int(off.size - 1),
        "occ_elems": int(width.sum()),                      # sum of D over occurrences
        "bag_elems": int(dims.sum()) * (off.size - 1) // F,  # sum of D over bags
        "u_elems_inside": int(uw[~cross].sum()), "u_elems_cross": int(uw[cross].sum()),
        "u_cross": int(cross.sum()), "n_pieces": int(n_pieces), "pdim": int(dims.max()),
        "classed": bool(classed),
    }


def sort_plan(nnz, rowref_space, classed=False):
    """Items per thread, tiles and digit bits of the library's radix sort for a batch (mixed-width
    tables carry a 3-bit width class above the rowref bits)."""
    keybits = 0
    while keybits < 32 and rowref_space > 1 and ((rowref_space - 1) >> keybits) != 0:
        keybits += 1
    if classed:
        keybits += 3
    maxbits = 9 if nnz >= (4 << 20) else 8
    passes = 1 if keybits <= maxbits else (keybits + maxbits - 1) // maxbits
    bits = (keybits + passes - 1) // passes
    ipt = 8 if nnz >= (1 << 20) else 4
    return ipt, (nnz + 256 * ipt - 1) // (256 * ipt), bits


def kernel_bytes(name, st, w, rowref_space, ftrl=False):
    """Algorithmic bytes one launch of `name` moves for a batch with stats `st`: every datum the
    kernel must read or write once (no cache reuse), as in the design's byte model."""
    sr = 2 if w.row_dtype == "f16" else 4
    so = 2 if w.out_dtype == "f16" else 4
    sg = 2 if w.grad_dtype == "f16" else 4
    m = 1 if w.has_master else 0
    state = 2 * sr + 8 + 8 * m + (8 if ftrl else 0)    # per element: row, acc, master, z r/w
    n = st["nnz"]
    if name == "lookup_pool":
        # key in, slot hit (key compare + row prefix), row gather, rowref out; offsets, pooled out
        return n * (8 + 12 + 4) + st["occ_elems"] * sr + st["bags"] * 4 + st["bag_elems"] * so
    if name == "lookup_probe":                          # the probe alone: key in, hit, rowref out
        return n * (8 + 12 + 4) + st["bags"] * 4
    if name == "pool":                                  # the pooling alone: rowref in, row gather
        return n * 4 + st["occ_elems"] * sr + st["bags"] * 4 + st["bag_elems"] * so
    if name in ("sort_hist", "sort_scan", "sort_scatter"):
        ipt, tiles, bits = sort_plan(n, rowref_space, st.get("classed", False))
        bins = (1 << bits) + 1                          # digits plus the miss bin
        tile_group = 16 if tiles >= 512 * 16 else tiles // 512 if tiles >= 512 else 1
        groups = (tiles + tile_group - 1) // tile_group
        if name == "sort_hist":                         # keys in; per-tile and per-group counts out
            return n * 4 + (tiles + groups) * bins * 4
        if name == "sort_scan":                         # group totals scanned in place
            return groups * bins * 8
        return n * 16 + (tiles + groups) * bins * 4     # pairs in and out; counts in
    if name == "update_pieces":
        # every occurrence's sorted pair and gradient slice; rows finished inside a piece;
        # head/tail partials of pieces whose segments cross
        return (n * 8 + st["occ_elems"] * sg + st["u_elems_inside"] * state
                + st["u_cross"] * 2 * st["pdim"] * 4 + st["n_pieces"] * 12)
    if name == "mark_touched":                          # sorted keys; per row its bag and bitmap word
        return n * 4 + st["U"] * 12
    if name == "update_fixup":
        return st["n_pieces"] * 4 + st["u_cross"] * (8 + 2 * st["pdim"] * 4) + \
            st["u_elems_cross"] * state
    return 0


def b_min_bytes(st, w, ftrl=False):
    """Compulsory bytes of one step: every datum once -- keys in, rowrefs out and back, one bucket
    hit (key + prefix word) and one row read per distinct row, offsets, pooled output, upstream
    gradient, and each distinct row's state read and written."""
    sr = 2 if w.row_dtype == "f16" else 4
    so = 2 if w.out_dtype == "f16" else 4
    sg = 2 if w.grad_dtype == "f16" else 4
    m = 1 if w.has_master else 0
    ue = st["u_elems_inside"] + st["u_elems_cross"]
    fwd = st["nnz"] * 12 + st["U"] * 12 + ue * sr + st["bags"] * 4 + st["bag_elems"] * so
    bwd = (st["bags"] * 4 + st["bag_elems"] * sg + st["nnz"] * 4 +
           ue * (2 * sr + 8 + 8 * m + (8 if ftrl else 0)))
    return fwd + bwd


def b_alg_bytes(st, w, ftrl=False):
    """Algorithmic bytes of one step: what the method moves per occurrence with no cache reuse.
    Forward, per occurrence: key in, probe hit (key compare + rank word), row, rowref out; per bag:
    offset and pooled slice out.  Backward, per occurrence: rowref and gradient slice; per bag: its
    offset; per updated row: its state read and written, plus its rowref and count.  Sort passes
    are not algorithmic: they are reported as amplification."""
    sr = 2 if w.row_dtype == "f16" else 4
    so = 2 if w.out_dtype == "f16" else 4
    sg = 2 if w.grad_dtype == "f16" else 4
    m = 1 if w.has_master else 0
    ue = st["u_elems_inside"] + st["u_elems_cross"]
    fwd = st["nnz"] * (8 + 12 + 4) + st["occ_elems"] * sr + st["bags"] * 4 + st["bag_elems"] * so
    bwd = (st["nnz"] * 4 + st["occ_elems"] * sg + st["bags"] * 4 +
           ue * (2 * sr + 8 + 8 * m + (8 if ftrl else 0)) + 12 * st["U"])
    return fwd + bwd


def load_traffic(workload, kernel):
    """HBM bytes per launch from rocprofv3 counters, if measured on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
        e = t[workload][kernel]
        if e.get("src_hash") != kernel_src_hash():
            return None
        return float(e["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# --------------------------------------------------------------------------- table + ring
def build_table(w, pinned=True, extra_flags=0):
    """The workload's prebuilt table with its initial state in the host image.  Tables of 64M+
    keys have their layout built on the GPU (table_create_on_device), start without state and are
    filled field by field on a thread pool, so the state is never held twice on the host; their
    images exceed what the box can pin, so they stay pageable.  Returns (Table, keys, pinned)."""
    import torch
    from ad_recommendation_amd import emb
    from gen import synth
    dims = synth.field_dims(w)
    rdt = emb.EMB_F16 if w.row_dtype == "f16" else emb.EMB_F32
    t0 = time.perf_counter()
    keys = synth.resident_keys(w)
    big = w.n_keys >= (1 << 26)
    if big:
        log(f"[bench] {keys.size} resident keys drawn in {time.perf_counter() - t0:.0f}s")
    t0 = time.perf_counter()

    def make(flags):
        if not big:
            rows, master = synth.initial_state(w)
            return emb.Table(dims, rdt, w.has_master, w.n_tables, w.load_factor, w.acc_init,
                             keys, rows, None, master, flags=flags | extra_flags)
        ws = torch.empty(emb.table_build_workspace_bytes(dims, w.n_tables, w.load_factor,
                                                         keys.size), dtype=torch.uint8,
                         device="cuda")
        t = emb.Table(dims, rdt, w.has_master, w.n_tables, w.load_factor, w.acc_init, keys,
                      flags=flags | extra_flags, device_ws=ws)
        del ws
        torch.cuda.empty_cache()
        return t
    T = None
    if big:
        pinned = False
    if pinned:
        try:  # pinned host image: the PASS flash is one DMA from page-locked memory
            T = make(emb.FLAG_PINNED_STAGING)
        except emb.EmbError as e:
            log(f"[bench] pinned host image unavailable ({e}); using pageable memory")
    if T is None:
        T, pinned = make(0), False
    if big:
        log(f"[bench] table created in {time.perf_counter() - t0:.1f}s (layout built on the GPU); "
            f"filling state by field")
        foff = synth.field_key_offsets(w)

        def fill(f):
            r_f, m_f = synth.field_state(w, f)
            T.fill_state(int(foff[f]), int(foff[f + 1] - foff[f]), r_f, None, m_f)
        with ThreadPoolExecutor(max(1, min(8, synth.worker_count()))) as ex:
            list(ex.map(fill, range(w.n_fields)))
    return T, keys, pinned


def host_batch(w, T, dims, b):
    """Batch b with the byte-model statistics of its occurrences (host side)."""
    from ad_recommendation_amd import emb
    from gen import synth
    bt = synth.batch(w, b)
    rr, _ = emb.table_key_rowref(T.h, bt["keys"])
    bt["st"] = batch_stats(w, bt, dims, rr, bool(T.info["unique_by_width"]))
    return bt


def stage_ring(w, T, dims, R, dev):
    """R batches generated on the host (in parallel waves for large batches) and copied to HBM."""
    import torch
    from gen import synth
    ring = []
    workers = min(8, synth.worker_count()) if w.batch * w.n_fields >= (1 << 22) else 1
    for a in range(0, R, max(1, workers)):
        idx = list(range(a, min(R, a + max(1, workers))))
        if workers > 1:
            with ThreadPoolExecutor(workers) as ex:
                got = list(ex.map(lambda b: host_batch(w, T, dims, b), idx))
        else:
            got = [host_batch(w, T, dims, b) for b in idx]
        for bt in got:
            ring.append({
                "keys": torch.from_numpy(bt["keys"]).to(dev),
                "offsets": torch.from_numpy(bt["offsets"]).to(dev),
                "grad": torch.from_numpy(bt["grad"]).to(dev),
                "n_bags": bt["offsets"].size - 1, "nnz": bt["st"]["nnz"], "st": bt["st"],
            })
        del got
        if workers > 1:
            log(f"[bench] {len(ring)}/{R} batches staged")
    return ring


# --------------------------------------------------------------------------- CPU baseline
def cpu_sample(w, T, dims, sub):
    """The CPU baseline's input: every `sub`-th sample of batch 0 with all of its bags, the
    upstream-gradient rows of those samples, and the distinct keys they name with their state as
    the table was built (read from the host image before any write-back)."""
    from gen import synth
    bt = synth.batch(w, 0)
    F = w.n_fields
    off = bt["offsets"].astype(np.int64)
    lens = np.diff(off)
    samp = np.arange(0, w.batch, sub)
    bag_ids = (samp[:, None] * F + np.arange(F)[None, :]).reshape(-1)
    sl = lens[bag_ids]
    sub_off = np.concatenate([[0], np.cumsum(sl)])
    sub_idx = np.repeat(off[bag_ids], sl) + (np.arange(sub_off[-1]) - np.repeat(sub_off[:-1], sl))
    keys = bt["keys"][sub_idx]
    tkeys = np.unique(keys.view(np.uint64))
    rows, acc, master = T.export(tkeys)
    return {"keys": keys, "offsets": sub_off.astype(np.int32), "grad": bt["grad"][samp],
            "tkeys": tkeys.view(np.int64), "rows": rows, "acc": acc,
            "master": master if master is not None else np.zeros(0, np.float32),
            "dims": dims, "full_nnz": np.int64(bt["keys"].size),
            "full_U": np.int64(np.unique(bt["keys"]).size), "sub": np.int64(sub)}


def cpu_baseline_child(name: str, path: str, min_seconds: float, optimizer: str = "adagrad"):
    """Time the oracle's forward + backward (one thread) on the sub-batch saved at `path`, with
    the oracle table built over just the sub-batch's keys: at least 3 steps, more until
    min_seconds of oracle work; reports the median step."""
    from gen import workloads as W
    from oracle import emb_oracle as O
    w = W.get(name)
    d = np.load(path)
    ftrl = optimizer == "ftrl"
    t0 = time.perf_counter()
    ot = O.Table(d["tkeys"], d["dims"], w.row_dtype, w.has_master, w.n_tables, w.load_factor,
                 w.acc_init, d["rows"], acc=d["acc"],
                 master=d["master"] if w.has_master else None, ftrl=ftrl)
    build_s = time.perf_counter() - t0
    log(f"[cpu-baseline] oracle table over the sub-batch's {d['tkeys'].size} keys built in "
        f"{build_s:.1f}s; timing its steps")
    keys, offsets, grad = d["keys"], d["offsets"], d["grad"]
    times, t_fwd, n_u = [], [], 0
    while len(times) < 3 or (sum(times) < min_seconds and len(times) < 50):
        t0 = time.perf_counter()
        ot.forward(keys, offsets, w.out_dtype)
        t1 = time.perf_counter()
        if ftrl:
            u, _, _, _ = ot.touched(keys, offsets)
            ot.ftrl_rows(ot.row_grads(keys, offsets, grad), w.lr, FTRL_BETA, FTRL_L1, FTRL_L2)
        else:
            u, _, _, _ = ot.backward(keys, offsets, grad, w.lr, w.eps)
        times.append(time.perf_counter() - t0)
        t_fwd.append(t1 - t0)
        n_u = int(u.size)
        log(f"[cpu-baseline] step {len(times)}: {times[-1]:.2f}s")
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    print(json.dumps({"median_s": float(np.median(times)), "fwd_median_s": float(np.median(t_fwd)),
                      "steps": len(times), "build_seconds": build_s, "nnz": int(keys.size),
                      "U": n_u, "cpu": cpu, "nproc": os.cpu_count(),
                      "full_nnz": int(d["full_nnz"]), "full_U": int(d["full_U"]),
                      "sub": int(d["sub"]), "samples": int(grad.shape[0])}))


def run_cpu_baseline(name: str, sample: dict, optimizer: str = "adagrad"):
    import tempfile
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "cpu_sample.npz")
        np.savez(path, **sample)
        code = ("import os,sys; os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]}); "
                f"sys.path.insert(0, {ROOT!r}); import bench; "
                f"bench.cpu_baseline_child({name!r}, {path!r}, 10.0, {optimizer!r})")
        # the child's progress lines go straight to this process's stderr
        r = subprocess.run([sys.executable, "-c", code], env=env, stdout=subprocess.PIPE,
                           stderr=None, text=True, timeout=900)
    if r.returncode != 0:
        log(f"[cpu-baseline] the oracle run failed with status {r.returncode}")
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: four passes over the ring, at least 200)")
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed steps first (-1: one pass over the ring, at least 20)")
    ap.add_argument("--workload", default="f64")
    ap.add_argument("--ring", type=int, default=0, help="distinct batches cycled (0 = workload's)")
    ap.add_argument("--keys", type=int, default=0,
                    help="resident keys (0 = the workload's; other values give a scaled copy)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", action="store_true",
                    help="run each step as the split calls (lookup_probe, then pool_fwd on the "
                         "main stream while sparse_bwd_dedup runs on a second one, then "
                         "sparse_*_apply) instead of the two fused calls")
    ap.add_argument("--probe", choices=("auto", "lane", "coop"), default="auto",
                    help="bucket probe form: chosen by the bucket array's size, or forced")
    ap.add_argument("--optimizer", choices=("adagrad", "ftrl"), default="adagrad",
                    help="sparse update: Adagrad, or FTRL-Proximal (alpha = the workload's lr, "
                         f"beta {FTRL_BETA}, l1 {FTRL_L1}, l2 {FTRL_L2})")
    ap.add_argument("--flush-mall", action="store_true",
                    help="also time every kernel with a 512 MB scratch write between steps, so "
                         "that no step finds the previous one's data in the 256 MB Infinity Cache")
    ap.add_argument("--lifecycle", action="store_true",
                    help="track touched rows (adds the marking kernel to each step) and time the "
                         "end-of-PASS write-backs: touched rows only, then the whole state")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES, five times (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        sys.exit("bench.py measures one GPU: this build has no multi-GPU path (the sharded design "
                 "is described, not built); run with --gpus 1")

    import torch
    from ad_recommendation_amd import emb
    from gen import synth, workloads as W

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # a plain device copy: the counter scaling of the profiles, and the read + write rate the
        # memory system gives a streaming kernel (the practical ceiling under the 8 TB/s peak)
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        best = float("inf")
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.copy_(src)
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        moved = 2 * src.numel() * 4
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "best_ms": best,
                          "read_write_GB_per_s": moved / best / 1e6}), flush=True)
        return
    w = W.get(args.workload)
    if args.keys and args.keys != w.n_keys:
        w = W.scaled(w, n_keys=args.keys, name_suffix=f"_keys{args.keys}")
    R = args.ring or w.ring
    if args.steps <= 0:
        args.steps = max(200, 4 * R)
    if args.warmup < 0:
        args.warmup = max(20, R)
    dims = synth.field_dims(w)
    t0 = time.perf_counter()
    ftrl = args.optimizer == "ftrl"
    probe_flag = {"auto": 0, "lane": emb.FLAG_PROBE_LANE, "coop": emb.FLAG_PROBE_COOP}[args.probe]
    T, keys, pinned = build_table(w, extra_flags=(emb.FLAG_TRACK_TOUCHED if args.lifecycle else 0) |
                                  (emb.FLAG_FTRL if ftrl else 0) | probe_flag)
    log(f"[bench] {w.name}: {keys.size} keys, table built in {time.perf_counter() - t0:.1f}s; "
        f"arena {T.info['arena_bytes'] / 2**30:.2f} GiB")
    T.arena = torch.empty(emb.table_device_bytes(T.h), dtype=torch.uint8, device=dev)
    flash_ms = []
    for _ in range(2):  # the PASS flash (host image -> HBM), timed on its own
        torch.cuda.synchronize()
        f0 = time.perf_counter()
        T.flash(dev)
        torch.cuda.synchronize()
        flash_ms.append((time.perf_counter() - f0) * 1e3)
    flash = {"bytes": int(T.info["arena_bytes"]), "ms": min(flash_ms), "pinned": pinned,
             "GB_per_s": T.info["arena_bytes"] / (min(flash_ms) / 1e3) / 1e9}
    log(f"[bench] pass_flash: {flash['bytes'] / 1e9:.2f} GB in {flash['ms']:.1f} ms "
        f"({flash['GB_per_s']:.1f} GB/s, pinned={pinned})")
    cpu_in = None
    if not args.no_cpu_baseline:
        # the baseline's sub-batch and the state of its keys, read before any write-back
        t0 = time.perf_counter()
        cpu_in = cpu_sample(w, T, dims, CPU_SUBSAMPLE.get(w.name, 64))
        log(f"[cpu-baseline] sub-batch of {cpu_in['keys'].size} lookups over "
            f"{cpu_in['tkeys'].size} keys prepared in {time.perf_counter() - t0:.1f}s")

    odt = torch.float16 if w.out_dtype == "f16" else torch.float32
    out_code = emb.EMB_F16 if w.out_dtype == "f16" else emb.EMB_F32
    g_code = emb.EMB_F16 if w.grad_dtype == "f16" else emb.EMB_F32
    t0 = time.perf_counter()
    ring = stage_ring(w, T, dims, R, dev)
    max_nnz = max(r["nnz"] for r in ring)
    ws_bytes = max(emb.bwd_workspace_bytes(T.h, r["n_bags"], r["nnz"]) for r in ring)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(w.batch, int(dims.sum()), dtype=odt, device=dev)   # shared by the ring
    rowref = torch.empty(max(1, max_nnz), dtype=torch.int32, device=dev)
    n_unique = torch.zeros(R, dtype=torch.int64, device=dev)
    rowref_space = T.info["rowref_space"]
    log(f"[bench] ring of {R} batches staged in {time.perf_counter() - t0:.1f}s; mean nnz "
        f"{np.mean([r['nnz'] for r in ring]):.0f}, mean unique "
        f"{np.mean([r['st']['U'] for r in ring]):.0f}")

    main_stream = torch.cuda.current_stream()
    side_stream = torch.cuda.Stream()

    def step(i):
        r = ring[i % R]
        if args.split:
            # the dedup needs only the probe's rowrefs: it runs on a second stream while the
            # pooling runs on the main one; the update joins both
            emb.lookup_probe(T.h, r["keys"], r["offsets"], r["n_bags"], r["nnz"], rowref,
                             stream=main_stream)
            probed = torch.cuda.Event()
            probed.record(main_stream)
            side_stream.wait_event(probed)
            emb.sparse_bwd_dedup(T.h, rowref, r["offsets"], r["n_bags"], r["nnz"], ws,
                                 stream=side_stream)
            deduped = torch.cuda.Event()
            deduped.record(side_stream)
            emb.pool_fwd(T.h, rowref, r["offsets"], r["n_bags"], r["nnz"], out, out_code,
                         stream=main_stream)
            main_stream.wait_event(deduped)
            if ftrl:
                emb.sparse_ftrl_apply(T.h, r["n_bags"], r["nnz"], r["grad"], g_code, w.lr,
                                      FTRL_BETA, FTRL_L1, FTRL_L2, ws,
                                      n_unique=n_unique[i % R:i % R + 1], stream=main_stream)
            else:
                emb.sparse_adagrad_apply(T.h, r["n_bags"], r["nnz"], r["grad"], g_code, w.lr,
                                         w.eps, ws, n_unique=n_unique[i % R:i % R + 1],
                                         stream=main_stream)
            return
        fwd(i)
        bwd(i)

    def fwd(i):
        r = ring[i % R]
        emb.lookup_pool_fwd(T.h, r["keys"], r["offsets"], r["n_bags"], r["nnz"], out,
                            out_code, rowref)

    def bwd(i):
        r = ring[i % R]
        if ftrl:
            emb.sparse_ftrl_bwd(T.h, rowref, r["offsets"], r["n_bags"], r["nnz"], r["grad"],
                                g_code, w.lr, FTRL_BETA, FTRL_L1, FTRL_L2, ws,
                                n_unique=n_unique[i % R:i % R + 1])
        else:
            emb.sparse_adagrad_bwd(T.h, rowref, r["offsets"], r["n_bags"], r["nnz"], r["grad"],
                                   g_code, w.lr, w.eps, ws, n_unique=n_unique[i % R:i % R + 1])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # calibration.  One pass over the ring with every kernel timed names the kernels and counts
    # their launches; bracketing every launch with events adds gaps that inflate short kernels,
    # so each kernel is then timed in a pass of its own with only its launches bracketed.
    calib_steps = 0
    emb.emb_timing_enable(T.h, True)
    for i in range(R):
        step(i)
    torch.cuda.synchronize()
    calib_steps += R
    names = emb.emb_timing_read(T.h)
    calib = {}
    for k in names:
        emb.emb_timing_enable(T.h, True, k)
        for i in range(R):
            step(i)
        torch.cuda.synchronize()
        calib_steps += R
        calib[k] = emb.emb_timing_read(T.h)[k]
    emb.emb_timing_enable(T.h, False)
    per_step = {k: v[1] / R for k, v in calib.items()}
    kernels = {}
    for k, (cnt, kms) in calib.items():
        b = np.mean([kernel_bytes(k, r["st"], w, rowref_space, ftrl) for r in ring]) * cnt / R
        kernels[k] = {"launches_per_step": cnt / R, "ms_per_step": kms / R,
                      "avg_launch_ms": kms / max(cnt, 1),
                      "alg_bytes_per_step": float(b), "GB_per_s": float(b / (kms / R) / 1e6),
                      "frac": float(b / (kms / R) / 1e6 / HBM_PEAK_GBS)}
    # the dominant kernel: the longest per launch (each radix pass is its own launch)
    dominant = max(calib, key=lambda k: calib[k][1] / max(calib[k][0], 1))
    alg_step = float(np.mean([b_alg_bytes(r["st"], w, ftrl) for r in ring]))
    sort_step = sum(v["alg_bytes_per_step"] for k, v in kernels.items() if k in SORT_KERNELS)
    bmin_step = float(np.mean([b_min_bytes(r["st"], w, ftrl) for r in ring]))
    fwd_k = ("lookup_pool", "lookup_probe", "pool")
    ms_fwd = sum(v["ms_per_step"] for k, v in kernels.items() if k in fwd_k)
    ms_bwd = sum(v["ms_per_step"] for k, v in kernels.items() if k not in fwd_k)
    log("[bench] per-step kernel time (ms): " +
        ", ".join(f"{k} {v:.4f}" for k, v in sorted(per_step.items(), key=lambda x: -x[1])))
    got_u = n_unique.cpu().numpy()
    want_u = np.array([r["st"]["U"] for r in ring])
    if not np.array_equal(got_u, want_u):
        sys.exit(f"unique-row counts differ from the batches' distinct keys: {got_u} vs {want_u}")

    # probe statistics of one pass over the ring (collision monitoring), outside the timed region
    pstats = torch.zeros(4, dtype=torch.int64, device=dev)
    emb.table_probe_stats(T.h, pstats)
    for r in ring:
        emb.lookup_probe(T.h, r["keys"], r["offsets"], r["n_bags"], r["nnz"], rowref)
    emb.table_probe_stats(T.h, None)
    torch.cuda.synchronize()
    ps = pstats.cpu().numpy().tolist()
    probe_stats = {"batches": R, "scans": ps[0], "scans_past_home_bucket": ps[1],
                   "frac_past_home_bucket": ps[1] / max(ps[0], 1),
                   "buckets_per_scan": ps[2] / max(ps[0], 1), "max_buckets_one_scan": ps[3],
                   "mean_displacement_slots": T.info["mean_displacement"],
                   "max_displacement_slots": T.info["max_displacement"]}
    log(f"[bench] probe: {probe_stats['frac_past_home_bucket']:.4f} of scans read past the home "
        f"bucket, {probe_stats['buckets_per_scan']:.4f} buckets per scan, at most {ps[3]}")

    # per-step times over one pass of the ring, outside the timed region: events on the step's
    # stream around each step and, for the fused calls, between its forward and its backward
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(R)]
    for i in range(R):
        evs[i][0].record()
        if args.split:
            step(i)
        else:
            fwd(i)
            evs[i][1].record()
            bwd(i)
        evs[i][2].record()
    torch.cuda.synchronize()
    calib_steps += R
    per_step_ms = {"t_step": [e[0].elapsed_time(e[2]) for e in evs]}
    if not args.split:
        per_step_ms["t_fwd"] = [e[0].elapsed_time(e[1]) for e in evs]
        per_step_ms["t_bwd"] = [e[1].elapsed_time(e[2]) for e in evs]
    medians = {k + "_median_ms": float(np.median(v)) for k, v in per_step_ms.items()}
    log("[bench] per-step medians over the ring (ms): " +
        ", ".join(f"{k} {v:.4f}" for k, v in medians.items()))

    cold = None
    if args.flush_mall:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        emb.emb_timing_enable(T.h, True)
        for i in range(R):
            scratch.fill_(i & 0xFF)
            step(i)
        torch.cuda.synchronize()
        cc = emb.emb_timing_read(T.h)
        cold = {"kernels_ms_per_step": {k: v[1] / R for k, v in cc.items()},
                "ms_per_step": sum(v[1] for v in cc.values()) / R}
        del scratch
        log(f"[bench] with the Infinity Cache flushed between steps: {cold['ms_per_step']:.4f} ms "
            f"of kernels per step")

    # timed region: K steps, only the dominant kernel bracketed by events
    emb.emb_timing_enable(T.h, True, dominant)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    dom = emb.emb_timing_read(T.h)[dominant]
    emb.emb_timing_enable(T.h, False)

    rows_done = sum(ring[i % R]["nnz"] + ring[i % R]["st"]["U"] for i in range(args.steps))
    value = rows_done / (ms / 1e3)
    # algorithmic bytes of the dominant kernel over its timed launches
    per_step_launches = dom[0] / args.steps
    dom_bytes = sum(kernel_bytes(dominant, ring[i % R]["st"], w, rowref_space, ftrl)
                    for i in range(args.steps))
    dom_bytes *= per_step_launches
    achieved = dom_bytes / (dom[1] / 1e3) / 1e9
    # counter traffic was measured on the fused Adagrad step without tracking: other forms run
    # other kernel instantiations
    profiled = not (ftrl or args.lifecycle or args.split) and not args.keys and args.probe == "auto"
    traffic = load_traffic(w.name, dominant) if profiled else None
    # the whole step's counter traffic, when every kernel of the step has been measured
    counter_step = None
    if profiled:
        per = {k: load_traffic(w.name, k) for k in kernels}
        if all(v is not None for v in per.values()):
            counter_step = sum(per[k] * kernels[k]["launches_per_step"] for k in kernels)

    writeback = None
    if args.lifecycle:
        # end of the PASS: the rows updated by every step since the flash come back to the host
        # image, through the backward workspace (free once the steps are done)
        wb_ws = ws if ws.numel() >= emb.writeback_workspace_bytes(T.h) else torch.empty(
            emb.writeback_workspace_bytes(T.h), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        t_a = time.perf_counter()
        n_units = emb.pass_writeback_touched(T.h, wb_ws)
        t_b = time.perf_counter()
        emb.pass_writeback(T.h)
        t_c = time.perf_counter()
        g = int(T.info["granule"])
        unit_bytes = g * (2 if w.row_dtype == "f16" else 4) + 4 * g * (
            1 + (1 if w.has_master else 0) + (1 if ftrl else 0))
        moved = n_units * unit_bytes
        full = int(T.info["state_bytes"])
        writeback = {"touched_units": int(n_units), "rowref_units": int(T.info["rowref_space"]),
                     "touched_bytes": moved, "touched_ms": (t_b - t_a) * 1e3,
                     "touched_GB_per_s": moved / (t_b - t_a) / 1e9,
                     "full_bytes": full, "full_ms": (t_c - t_b) * 1e3,
                     "full_GB_per_s": full / (t_c - t_b) / 1e9,
                     "steps_since_flash": args.warmup + calib_steps + args.steps}
        log(f"[bench] write-back: touched {moved / 1e9:.2f} GB in {writeback['touched_ms']:.0f} ms"
            f" ({writeback['touched_GB_per_s']:.1f} GB/s), full {full / 1e9:.2f} GB in "
            f"{writeback['full_ms']:.0f} ms ({writeback['full_GB_per_s']:.1f} GB/s)")

    cpu = None
    if cpu_in is not None:
        c = run_cpu_baseline(w.name, cpu_in, args.optimizer)
        if c:
            sub_rate = (c["nnz"] + c["U"]) / c["median_s"]
            full_s = c["median_s"] * c["full_nnz"] / c["nnz"]
            cpu = {"value": sub_rate, "unit": "rows/s", "cores": 1, "kind": "oracle",
                   "sample": f"{'every sample' if c['sub'] == 1 else 'every %dth sample' % c['sub']} "
                             f"of batch 0 of {w.name} ({c['samples']} "
                             f"samples x {w.n_fields} fields: {c['nnz']} lookups, {c['U']} row "
                             f"updates); oracle table built over just those keys (build "
                             f"{c['build_seconds']:.1f}s excluded); forward+backward median of "
                             f"{c['steps']} steps {c['median_s']:.2f}s, 1 thread on {c['cpu']} "
                             f"({c['nproc']} cpus visible)",
                   "median_step_s": c["median_s"],
                   "full_batch_s_est": full_s,
                   "full_batch_note": f"median x {c['full_nnz']}/{c['nnz']} lookups "
                                      "(linear in occurrences)"}
    res = {
        "metric": METRIC, "value": value, "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if w.row_dtype == "f32" else "f16 rows/f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "fields": w.n_fields, "resident_keys": w.n_keys,
                   "dim": w.dim if w.dim else "per-field", "row_dtype": w.row_dtype,
                   "master": w.has_master, "tables": w.n_tables, "batch": w.batch,
                   "optimizer": args.optimizer,
                   "ring": R, "mean_lookups_per_step": float(np.mean([r["nnz"] for r in ring])),
                   "mean_rows_updated_per_step": float(np.mean([r["st"]["U"] for r in ring])),
                   "calls": "split, dedup on a second stream" if args.split else "fused",
                   "probe": args.probe,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "avg_launch_ms": dom[1] / max(dom[0], 1),
                     "alg_bytes_per_launch": dom_bytes / max(dom[0], 1)},
        "cpu_baseline": cpu,
        "probe_stats": probe_stats,
        "pass_flash": flash,
        "pass_writeback": writeback,
        "cold_cache": cold,
        "step_hbm": {"alg_bytes_per_step": alg_step,
                     "GB_per_s": alg_step / (ms / args.steps) / 1e6,
                     "frac": alg_step / (ms / args.steps) / 1e6 / HBM_PEAK_GBS,
                     "sort_bytes_per_step": sort_step,
                     "amplification_sort": (alg_step + sort_step) / alg_step,
                     "counter_bytes_per_step": counter_step,
                     "counter_GB_per_s": (counter_step / (ms / args.steps) / 1e6
                                          if counter_step else None),
                     "counter_frac": (counter_step / (ms / args.steps) / 1e6 / HBM_PEAK_GBS
                                      if counter_step else None),
                     "amplification_counters_vs_b_min": (counter_step / bmin_step
                                                         if counter_step else None),
                     "b_min_per_step": bmin_step,
                     "sol_frac": bmin_step / (ms / args.steps) / 1e6 / HBM_PEAK_GBS,
                     "ms_fwd": ms_fwd, "ms_bwd": ms_bwd, **medians},
        "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
