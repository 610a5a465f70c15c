"""Rows whose occurrences span many update pieces, against the whole-table oracle.

The backward cuts the sorted occurrences into pieces of PW (192 here); a row whose segment starts
in piece t and ends in piece e > t leaves a tail partial in t and head partials in t+1 .. e, and the
fixup joins them, reading the following pieces' flags 64 at a time.  A segment with e - t = 64
ends on the last flag of the first round, e - t = 65 on the first flag of the second, and longer
ones take several rounds.  These batches place segments of 64*PW - 1 .. 64*PW + 2 occurrences at
chosen offsets inside their first piece (so that e - t is 63, 64 and 65 exactly), one of ~40,000
occurrences and one of 130*PW + 3, each between short neighbouring rows, and check every row,
accumulator and master against the oracle over two steps: fp32 rows (one field, width 16) and fp16
rows with an fp32 master (100 fields, width 64).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gen import synth, workloads as W  # noqa: E402
from oracle import emb_oracle as O  # noqa: E402
from tests.sampled_parity import piece_width  # noqa: E402
from tests.test_gpu_parity import run_parity  # noqa: E402

pytestmark = pytest.mark.gpu


def long_segment_batch(w, seed):
    """A CSR batch of field-0 keys taken consecutively in rowref order, with the segment lengths
    and in-piece start offsets described above.  Returns (batch, spans) where spans lists e - t
    of every segment that crosses a piece boundary."""
    keys = synth.resident_keys(w)
    rows, master = synth.initial_state(w)
    dims = synth.field_dims(w)
    ot = O.Table(keys, dims, w.row_dtype, w.has_master, w.n_tables, w.load_factor, w.acc_init,
                 rows, master=master)
    f0 = np.nonzero(ot.field == 0)[0]
    by_slot = ot.keys[f0[np.argsort(ot.slot[f0])]]          # rowref order within field 0
    PW = 192
    plan = [(64 * PW - 1, 0), (64 * PW - 1, PW - 1), (64 * PW + 1, PW - 1), (64 * PW + 2, PW - 1),
            (64 * PW, 0), (40_000, 17), (130 * PW + 3, 5), (3, None)]
    segs = []
    pos = 0
    for c, start in plan:
        if start is not None:
            segs.append(1)                      # a one-occurrence neighbour just before it
            pos += 1
            gap = (start - pos) % PW            # short rows up to the wanted in-piece offset
            while gap > 0:
                n = min(gap, 3)
                segs.append(n)
                pos += n
                gap -= n
        segs.append(c)
        pos += c
    nnz = pos
    assert piece_width(w, nnz, False) == PW
    assert len(segs) <= by_slot.size
    seg_keys = by_slot[:len(segs)]
    counts = np.array(segs, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    ends = starts + counts - 1
    spans = [int(e // PW - s // PW) for s, e in zip(starts, ends) if e // PW > s // PW]
    # deal the occurrences over the field-0 bags in a seeded random order
    r = np.random.default_rng(seed)
    occ = np.repeat(seg_keys, counts)
    occ = occ[r.permutation(occ.size)]
    B = 4096
    F = w.n_fields
    bag_len = np.zeros(B * F, dtype=np.int64)
    b0 = np.sort(r.integers(0, B, size=occ.size))         # sample of each occurrence, ascending
    np.add.at(bag_len, b0 * F, 1)
    off = np.concatenate([[0], np.cumsum(bag_len)]).astype(np.int32)
    width = int(dims.sum())
    gdt = np.float16 if w.grad_dtype == "f16" else np.float32
    grad = r.standard_normal((B, width)).astype(gdt)
    return {"keys": occ.view(np.int64), "offsets": off, "grad": grad}, spans


@pytest.mark.parametrize("w", [
    W.scaled(W.TINY, n_keys=100_000, batch=4096, name_suffix="_long_fp32"),
    W.scaled(W.F100, n_keys=400_000, batch=4096, name_suffix="_long_fp16m")],
    ids=["fp32_d16", "fp16_master_d64"])
def test_segments_spanning_many_pieces(w):
    b1, spans = long_segment_batch(w, 1)
    b2, _ = long_segment_batch(w, 2)
    assert {63, 64, 65} <= set(spans) and max(spans) > 129
    run_parity(w, steps=2, batches=[b1, b2], check_all_keys=False)
