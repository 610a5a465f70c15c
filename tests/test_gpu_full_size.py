"""Parity at full size for the 100-field workload (50M resident keys, d64 fp16 rows with fp32
accumulator and master copy, batch 65,536 x 100 fields, ~32.8M lookups) and the 40-field
mixed-width workload (20M keys in two tables by key parity, widths 8-128, batch 32,768, ~5.2M
lookups), in the launch configuration the benchmark times: the table built by the benchmark's own
builder, flashed from pinned memory, one forward + backward step through the C ABI.

The whole-table oracle would need minutes here, so the checks are the sampled ones of the PASS-scale
test (tests/test_gpu_pass_scale.py): 20,000 occurrences' slots and rowrefs bit-exact (per-home
counting form of the layout, per table; on the mixed-width table each rowref is shown to name its
occurrence's key), the pooled output of 1 sample in 64, the unique count exactly, 1 % of
the touched rows' counts exactly and their rows, accumulators and master copies within the derived
budgets, and sampled untouched rows bit-identical.
"""
import sys
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ad_recommendation_amd import emb  # noqa: E402
from gen import synth, workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[full-size]", *a, flush=True)
    sys.stdout.flush()


def test_f100_full_size_sampled_parity():
    import bench
    from tests.test_gpu_parity import gpu_step
    from tests.test_gpu_pass_scale import check_sampled
    w = W.F100
    t0 = time.perf_counter()
    T, keys, pinned = bench.build_table(w)
    say(f"table of {keys.size} keys built in {time.perf_counter() - t0:.0f}s (pinned={pinned})")
    T.flash()
    torch.cuda.synchronize()
    bt = synth.batch(w, 0)
    say(f"batch 0: {bt['keys'].size} lookups")
    res = gpu_step(T, bt["keys"], bt["offsets"], bt["grad"], w.out_dtype, w.grad_dtype, w.lr,
                   w.eps)
    say(f"GPU step done: {res['n_unique']} unique rows")
    emb.pass_writeback(T.h)
    check_sampled(w, keys, bt, res, T.export)
    T.close()


def test_f40_mixed_width_two_tables_full_size_sampled_parity():
    import bench
    from tests.test_gpu_parity import gpu_step
    from tests.test_gpu_pass_scale import check_sampled
    w = W.F40_VARDIM
    t0 = time.perf_counter()
    T, keys, pinned = bench.build_table(w)
    say(f"table of {keys.size} keys built in {time.perf_counter() - t0:.0f}s (pinned={pinned})")
    T.flash()
    torch.cuda.synchronize()
    bt = synth.batch(w, 0)
    say(f"batch 0: {bt['keys'].size} lookups")
    res = gpu_step(T, bt["keys"], bt["offsets"], bt["grad"], w.out_dtype, w.grad_dtype, w.lr,
                   w.eps)
    say(f"GPU step done: {res['n_unique']} unique rows")
    emb.pass_writeback(T.h)
    check_sampled(w, keys, bt, res, T.export, rowref_keys=lambda rr: emb.table_rowref_keys(T.h, rr),
                  unique_by_width=bool(T.info["unique_by_width"]))
    T.close()


def test_f100_full_size_ftrl_sampled_parity():
    """The same workload and checks with the FTRL update (alpha = lr, beta 1, l1 0.01, l2 0.1):
    the table keeps the linear state, and the sampled rows, accumulators, masters and linear
    states are checked against the oracle's FTRL step."""
    import bench
    from tests.test_gpu_parity import gpu_step
    from tests.test_gpu_pass_scale import check_sampled
    w = W.F100
    prm = (w.lr, bench.FTRL_BETA, bench.FTRL_L1, bench.FTRL_L2)
    t0 = time.perf_counter()
    T, keys, pinned = bench.build_table(w, extra_flags=emb.FLAG_FTRL)
    say(f"FTRL table of {keys.size} keys built in {time.perf_counter() - t0:.0f}s (pinned={pinned})")
    T.flash()
    torch.cuda.synchronize()
    bt = synth.batch(w, 0)
    res = gpu_step(T, bt["keys"], bt["offsets"], bt["grad"], w.out_dtype, w.grad_dtype, 0.0, 0.0,
                   ftrl=prm)
    say(f"GPU FTRL step done: {res['n_unique']} unique rows")
    emb.pass_writeback(T.h)
    check_sampled(w, keys, bt, res, T.export, ftrl=prm, export_linear=T.export_linear)
    T.close()
