"""Workload descriptions for the embedding training step.

Each workload is a plain record of sizes and distributions: the number of
feature fields, resident keys, row widths and storage types, the batch shape,
bag-length and key-popularity distributions, and the sparse-Adagrad
hyper-parameters.  Nothing here computes any part of the method; the records
only parameterise the seeded generators in ``gen.synth``.

Shapes follow the pages' description of large-scale sparse training: CSR
multi-hot bags per sample and field (Tencent PCG GPU training framework talk,
section on preprocessing), a long-tailed key popularity where most ids occur
once or twice per batch (MetaApp/DeepRec article, section 3.1), feature ids
packed with a 16-bit field id above a 48-bit raw id (Tencent talk, unified
hash table paragraph) and fp16 rows with fp32 optimizer state (JD article,
section 3.2.3).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

DIM_CHOICES = (8, 16, 32, 64, 128)


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int                   # enters every SeedSequence of this workload
    n_fields: int
    n_keys: int                    # resident keys over all fields
    dim: Optional[int]             # row width; None = drawn per field from DIM_CHOICES
    row_dtype: str                 # "f32" | "f16"
    has_master: bool               # fp32 master copy beside fp16 rows
    n_tables: int                  # 1 = unified, 2 = split by key parity
    load_factor: float
    batch: int                     # samples per batch; bags = batch * n_fields
    bag_kind: str                  # "fixed" | "poisson"
    bag_mean: float
    bag_min: int                   # lower clamp on drawn bag lengths
    key_kind: str                  # "uniform" | "zipf" | "longtail"
    zipf_alpha: float
    grad_dtype: str                # "f32" | "f16"
    out_dtype: str                 # pooled output dtype
    lr: float = 0.05
    eps: float = 1e-8
    acc_init: float = 0.1
    ring: int = 16                 # distinct batches cycled by the benchmark
    row_std: float = 0.01
    raw_bits: int = 48
    field0_only: bool = False      # every key carries field id 0

    @property
    def n_bags(self) -> int:
        return self.batch * self.n_fields


def _w(**kw) -> Workload:
    return Workload(**kw)


# The five synthetic workloads.  Names state what each one is.
TINY = _w(name="tiny_f1_k10k_d16_fp32", seed_id=0, n_fields=1, n_keys=10_000, dim=16,
          row_dtype="f32", has_master=False, n_tables=1, load_factor=0.5, batch=256,
          bag_kind="fixed", bag_mean=4, bag_min=4, key_kind="uniform", zipf_alpha=0.0,
          grad_dtype="f32", out_dtype="f32", field0_only=True)

F26 = _w(name="f26_k4m_d16_fp32_zipf1.05", seed_id=1, n_fields=26, n_keys=1 << 22, dim=16,
         row_dtype="f32", has_master=False, n_tables=1, load_factor=0.5, batch=4096,
         bag_kind="poisson", bag_mean=3.0, bag_min=1, key_kind="zipf", zipf_alpha=1.05,
         grad_dtype="f32", out_dtype="f32")

F100 = _w(name="f100_k50m_d64_fp16_zipf1.1", seed_id=2, n_fields=100, n_keys=50_000_000, dim=64,
          row_dtype="f16", has_master=True, n_tables=1, load_factor=0.6, batch=65_536,
          bag_kind="poisson", bag_mean=5.0, bag_min=0, key_kind="zipf", zipf_alpha=1.1,
          grad_dtype="f16", out_dtype="f16")

F40_VARDIM = _w(name="f40_k20m_vardim_fp16_2tables_longtail", seed_id=3, n_fields=40,
                n_keys=20_000_000, dim=None, row_dtype="f16", has_master=True, n_tables=2,
                load_factor=0.5, batch=32_768, bag_kind="poisson", bag_mean=4.0, bag_min=0,
                key_kind="longtail", zipf_alpha=1.2, grad_dtype="f16", out_dtype="f16")

F64_PASS = _w(name="f64_k800m_d32_fp16_pass", seed_id=4, n_fields=64, n_keys=800_000_000, dim=32,
              row_dtype="f16", has_master=False, n_tables=1, load_factor=0.5, batch=131_072,
              bag_kind="poisson", bag_mean=6.0, bag_min=0, key_kind="zipf", zipf_alpha=1.05,
              grad_dtype="f16", out_dtype="f16", ring=50)

ALL = (TINY, F26, F100, F40_VARDIM, F64_PASS)
BY_NAME = {w.name: w for w in ALL}
# short aliases used on command lines
ALIASES = {"tiny": TINY, "f26": F26, "f100": F100, "f40": F40_VARDIM, "f64": F64_PASS}


def get(name: str) -> Workload:
    if name in ALIASES:
        return ALIASES[name]
    return BY_NAME[name]


def scaled(w: Workload, *, n_keys: Optional[int] = None, batch: Optional[int] = None,
           name_suffix: str = "_scaled") -> Workload:
    """Same distributions, smaller sizes (parity tests the oracle can finish)."""
    from dataclasses import replace
    return replace(w, n_keys=n_keys if n_keys is not None else w.n_keys,
                   batch=batch if batch is not None else w.batch,
                   name=w.name + name_suffix)
