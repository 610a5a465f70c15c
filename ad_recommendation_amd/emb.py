"""Python binding of libmi355emb.so (ctypes).  Argument marshalling only: every step of the
embedding training step runs in the library's HIP kernels.  PyTorch supplies device memory and
the stream; numpy arrays carry host inputs.

The functions keep the C names and argument order of include/emb.h.  Device arguments are torch
CUDA tensors, host arguments numpy arrays.  Errors raise EmbError with the library's message.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

EMB_F32, EMB_F16 = 0, 1
ROWREF_MISS = 0xFFFFFFFF
FLAG_PINNED_STAGING = 1
FLAG_PROBE_COOP = 2   # force the wave-cooperative bucket probe
FLAG_PROBE_LANE = 4   # force the one-lane-per-key bucket probe
FLAG_TRACK_TOUCHED = 8  # keep the device bitmap of updated rows for pass_writeback_touched
FLAG_FTRL = 16          # keep the FTRL linear state for sparse_ftrl_bwd

_HERE = os.path.dirname(os.path.abspath(__file__))
# MI355EMB_LIB selects another build of the same library (the sanitized host build of the CPU
# tests); the default is the in-tree one
LIB_PATH = os.environ.get("MI355EMB_LIB") or os.path.join(_HERE, "libmi355emb.so")

_STATUS = {0: "EMB_OK", -1: "EMB_EINVAL", -2: "EMB_EDUPKEY", -3: "EMB_ESENTINEL", -4: "EMB_ERANGE",
           -5: "EMB_ENOSPACE", -6: "EMB_ESTATE", -7: "EMB_EHIP", -8: "EMB_ENOMEM"}


class EmbError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code
        self.name = _STATUS.get(code, str(code))


class EmbTableDesc(C.Structure):
    _fields_ = [("n_fields", C.c_int32), ("field_dim", C.POINTER(C.c_int32)),
                ("row_dtype", C.c_int32), ("has_master", C.c_int32), ("n_tables", C.c_int32),
                ("load_factor", C.c_double), ("acc_init", C.c_float), ("flags", C.c_int32)]


class EmbTableInfo(C.Structure):
    _fields_ = [("arena_bytes", C.c_uint64), ("key_bytes", C.c_uint64), ("state_bytes", C.c_uint64),
                ("n_keys", C.c_uint64), ("total_elems", C.c_uint64), ("rowref_space", C.c_uint32),
                ("granule", C.c_uint32), ("n_home", C.c_uint64 * 2), ("n_keys_t", C.c_uint64 * 2),
                ("n_buckets", C.c_uint64 * 2), ("mean_displacement", C.c_double),
                ("max_displacement", C.c_uint64), ("unique_by_width", C.c_uint32)]


_LIB = None
_VP, _I32, _I64, _U64 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64


def lib() -> C.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback path)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP extension {LIB_PATH} is not built; run "
                           "python -m ad_recommendation_amd.build")
    L = C.CDLL(LIB_PATH)
    sig = {
        "table_create_from_prebuilt": [C.POINTER(EmbTableDesc), _VP, _I64, _VP, _VP, _VP, C.POINTER(_VP)],
        "table_info": [_VP, C.POINTER(EmbTableInfo)],
        "table_device_bytes": [_VP, C.POINTER(C.c_size_t)],
        "pass_flash": [_VP, _VP, C.c_size_t, _VP],
        "lookup_pool_fwd": [_VP, _VP, _VP, _I64, _I64, _VP, _I32, _VP, _VP, _VP, _VP],
        "bwd_workspace_bytes": [_VP, _I64, _I64, C.POINTER(C.c_size_t)],
        "sparse_adagrad_bwd": [_VP, _VP, _VP, _I64, _I64, _VP, _I32, C.c_float, C.c_float, _VP,
                               C.c_size_t, _VP, _VP, _VP, _VP],
        "sparse_adagrad_bwd_noalloc": [_VP, _VP, _VP, _I64, _I64, _VP, _I32, C.c_float, C.c_float,
                                       _VP, _VP, _VP, _VP],
        "sparse_ftrl_bwd": [_VP, _VP, _VP, _I64, _I64, _VP, _I32, C.c_float, C.c_float, C.c_float,
                            C.c_float, _VP, C.c_size_t, _VP, _VP, _VP, _VP],
        "lookup_probe": [_VP, _VP, _VP, _I64, _I64, _VP, _VP, _VP, _VP],
        "pool_fwd": [_VP, _VP, _VP, _I64, _I64, _VP, _I32, _VP],
        "sparse_bwd_dedup": [_VP, _VP, _VP, _I64, _I64, _VP, C.c_size_t, _VP],
        "sparse_adagrad_apply": [_VP, _I64, _I64, _VP, _I32, C.c_float, C.c_float, _VP, C.c_size_t,
                                 _VP, _VP, _VP, _VP],
        "sparse_ftrl_apply": [_VP, _I64, _I64, _VP, _I32, C.c_float, C.c_float, C.c_float, C.c_float,
                              _VP, C.c_size_t, _VP, _VP, _VP, _VP],
        "table_fill_linear": [_VP, _I64, _I64, _VP],
        "table_export_linear": [_VP, _VP, _I64, _VP],
        "table_build_workspace_bytes": [C.POINTER(EmbTableDesc), _I64, C.POINTER(C.c_size_t)],
        "table_create_on_device": [C.POINTER(EmbTableDesc), _VP, _I64, _VP, C.c_size_t, _VP,
                                   C.POINTER(_VP)],
        "pass_writeback": [_VP, _VP],
        "writeback_workspace_bytes": [_VP, C.POINTER(C.c_size_t)],
        "pass_writeback_touched": [_VP, _VP, C.c_size_t, C.POINTER(_I64), _VP],
        "table_dirty_keys": [_VP, _VP, _I64, C.POINTER(_I64), _I32],
        "table_carry_state": [_VP, _VP, C.POINTER(_I64)],
        "table_export": [_VP, _VP, _I64, _VP, _VP, _VP],
        "table_fill_state": [_VP, _I64, _I64, _VP, _VP, _VP],
        "table_key_rowref": [_VP, _VP, _I64, _VP, _VP],
        "table_rowref_keys": [_VP, _VP, _I64, _VP],
        "table_probe_stats": [_VP, _VP],
        "emb_timing_enable": [_VP, C.c_int, C.c_char_p],
        "emb_timing_read": [_VP, C.c_char_p, C.c_size_t, _VP, _VP, _I32, C.POINTER(_I32)],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = C.c_int
    L.table_destroy.argtypes = [_VP]
    L.table_destroy.restype = None
    L.emb_last_error.argtypes = []
    L.emb_last_error.restype = C.c_char_p
    _LIB = L
    return L


def exported_symbols():
    """Names include/emb.h declares (used by the load test)."""
    return ["table_create_from_prebuilt", "table_info", "table_device_bytes", "pass_flash",
            "lookup_pool_fwd", "bwd_workspace_bytes", "sparse_adagrad_bwd", "pass_writeback",
            "writeback_workspace_bytes", "pass_writeback_touched", "table_dirty_keys",
            "table_carry_state", "sparse_ftrl_bwd", "table_fill_linear", "table_export_linear",
            "lookup_probe", "pool_fwd", "sparse_bwd_dedup", "sparse_adagrad_apply",
            "sparse_ftrl_apply",
            "table_build_workspace_bytes", "table_create_on_device",
            "table_export", "table_fill_state", "table_key_rowref", "table_rowref_keys",
            "table_probe_stats", "sparse_adagrad_bwd_noalloc", "emb_timing_enable",
            "emb_timing_read", "table_destroy", "emb_last_error"]


def _check(rc: int):
    if rc != 0:
        raise EmbError(rc, lib().emb_last_error().decode(errors="replace"))


def _host(a, dtype) -> Optional[np.ndarray]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _hp(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _dp(t, dtypes=None) -> Optional[int]:
    """Device pointer of a torch CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError("expected a CUDA tensor")
    if not t.is_contiguous():
        raise TypeError("expected a contiguous tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"unexpected tensor dtype {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ C entry points
def table_create_from_prebuilt(field_dim, row_dtype: int, has_master: bool, n_tables: int,
                               load_factor: float, acc_init: float, keys, rows=None, acc=None,
                               master=None, flags: int = 0):
    """Returns an opaque table handle.  keys: int64 [N]; rows/acc/master packed in key order."""
    dims = _host(np.asarray(field_dim, dtype=np.int32), np.int32)
    keys = _host(np.asarray(keys).view(np.int64) if np.asarray(keys).dtype == np.uint64 else keys,
                 np.int64)
    rows = _host(rows, np.float16 if row_dtype == EMB_F16 else np.float32)
    acc = _host(acc, np.float32)
    master = _host(master, np.float32)
    d = EmbTableDesc(int(dims.size), dims.ctypes.data_as(C.POINTER(C.c_int32)), int(row_dtype),
                     int(bool(has_master)), int(n_tables), float(load_factor), float(acc_init),
                     int(flags))
    h = _VP()
    _check(lib().table_create_from_prebuilt(C.byref(d), _hp(keys), int(keys.size), _hp(rows),
                                            _hp(acc), _hp(master), C.byref(h)))
    return h


def _desc(field_dim, row_dtype, has_master, n_tables, load_factor, acc_init, flags):
    dims = _host(np.asarray(field_dim, dtype=np.int32), np.int32)
    d = EmbTableDesc(int(dims.size), dims.ctypes.data_as(C.POINTER(C.c_int32)), int(row_dtype),
                     int(bool(has_master)), int(n_tables), float(load_factor), float(acc_init),
                     int(flags))
    return d, dims


def table_build_workspace_bytes(field_dim, n_tables: int, load_factor: float, n_keys: int) -> int:
    d, _keep = _desc(field_dim, EMB_F32, False, n_tables, load_factor, 0.0, 0)
    n = C.c_size_t()
    _check(lib().table_build_workspace_bytes(C.byref(d), int(n_keys), C.byref(n)))
    return n.value


def table_create_on_device(field_dim, row_dtype: int, has_master: bool, n_tables: int,
                           load_factor: float, acc_init: float, keys, ws, flags: int = 0,
                           stream=None):
    """The prebuilt table with its layout computed on the GPU (rows zero, acc = acc_init)."""
    d, _keep = _desc(field_dim, row_dtype, has_master, n_tables, load_factor, acc_init, flags)
    keys = _host(np.asarray(keys).view(np.int64) if np.asarray(keys).dtype == np.uint64 else keys,
                 np.int64)
    h = _VP()
    _check(lib().table_create_on_device(C.byref(d), _hp(keys), int(keys.size), _dp(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(),
                                        _stream(stream), C.byref(h)))
    return h


def table_info(h) -> dict:
    i = EmbTableInfo()
    _check(lib().table_info(h, C.byref(i)))
    out = {k: getattr(i, k) for k, _ in EmbTableInfo._fields_}
    for k in ("n_home", "n_keys_t", "n_buckets"):
        out[k] = list(out[k])
    return out


def table_device_bytes(h) -> int:
    n = C.c_size_t()
    _check(lib().table_device_bytes(h, C.byref(n)))
    return n.value


def pass_flash(h, arena, stream=None):
    _check(lib().pass_flash(h, _dp(arena), arena.numel() * arena.element_size(), _stream(stream)))


def lookup_pool_fwd(h, keys, offsets, n_bags: int, nnz: int, out, out_dtype: int, rowref,
                    slot=None, n_miss=None, stream=None):
    import torch
    _check(lib().lookup_pool_fwd(
        h, _dp(keys, (torch.int64,)), _dp(offsets, (torch.int32,)), int(n_bags), int(nnz),
        _dp(out, (torch.float32, torch.float16)), int(out_dtype), _dp(rowref, (torch.int32,)),
        _dp(slot, (torch.int64,)), _dp(n_miss, (torch.int64,)), _stream(stream)))


def table_probe_stats(h, stats=None):
    """Count probe statistics into `stats` (int64 CUDA tensor of 4: scans, scans past the home
    bucket, buckets read, most buckets of one scan) on every later forward; None stops."""
    import torch
    if stats is not None and stats.numel() < 4:
        raise ValueError("stats needs 4 int64 entries")
    _check(lib().table_probe_stats(h, _dp(stats, (torch.int64,))))


def bwd_workspace_bytes(h, n_bags: int, nnz: int) -> int:
    n = C.c_size_t()
    _check(lib().bwd_workspace_bytes(h, int(n_bags), int(nnz), C.byref(n)))
    return n.value


def sparse_adagrad_bwd(h, rowref, offsets, n_bags: int, nnz: int, grad, grad_dtype: int,
                       lr: float, eps: float, ws, unique=None, count=None, n_unique=None,
                       stream=None):
    import torch
    _check(lib().sparse_adagrad_bwd(
        h, _dp(rowref, (torch.int32,)), _dp(offsets, (torch.int32,)), int(n_bags), int(nnz),
        _dp(grad, (torch.float32, torch.float16)), int(grad_dtype), float(lr), float(eps),
        _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(), _dp(unique, (torch.int32,)),
        _dp(count, (torch.int32,)), _dp(n_unique, (torch.int64,)), _stream(stream)))


def sparse_adagrad_bwd_noalloc(h, rowref, offsets, n_bags: int, nnz: int, grad, grad_dtype: int,
                               lr: float, eps: float, unique=None, count=None, n_unique=None,
                               stream=None):
    """sparse_adagrad_bwd on the library's static scratch: no workspace, no allocation."""
    import torch
    _check(lib().sparse_adagrad_bwd_noalloc(
        h, _dp(rowref, (torch.int32,)), _dp(offsets, (torch.int32,)), int(n_bags), int(nnz),
        _dp(grad, (torch.float32, torch.float16)), int(grad_dtype), float(lr), float(eps),
        _dp(unique, (torch.int32,)), _dp(count, (torch.int32,)), _dp(n_unique, (torch.int64,)),
        _stream(stream)))


def sparse_ftrl_bwd(h, rowref, offsets, n_bags: int, nnz: int, grad, grad_dtype: int,
                    alpha: float, beta: float, l1: float, l2: float, ws, unique=None, count=None,
                    n_unique=None, stream=None):
    import torch
    _check(lib().sparse_ftrl_bwd(
        h, _dp(rowref, (torch.int32,)), _dp(offsets, (torch.int32,)), int(n_bags), int(nnz),
        _dp(grad, (torch.float32, torch.float16)), int(grad_dtype), float(alpha), float(beta),
        float(l1), float(l2), _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _dp(unique, (torch.int32,)), _dp(count, (torch.int32,)), _dp(n_unique, (torch.int64,)),
        _stream(stream)))


def lookup_probe(h, keys, offsets, n_bags: int, nnz: int, rowref, slot=None, n_miss=None,
                 stream=None):
    import torch
    _check(lib().lookup_probe(
        h, _dp(keys, (torch.int64,)), _dp(offsets, (torch.int32,)), int(n_bags), int(nnz),
        _dp(rowref, (torch.int32,)), _dp(slot, (torch.int64,)), _dp(n_miss, (torch.int64,)),
        _stream(stream)))


def pool_fwd(h, rowref, offsets, n_bags: int, nnz: int, out, out_dtype: int, stream=None):
    import torch
    _check(lib().pool_fwd(
        h, _dp(rowref, (torch.int32,)), _dp(offsets, (torch.int32,)), int(n_bags), int(nnz),
        _dp(out, (torch.float32, torch.float16)), int(out_dtype), _stream(stream)))


def sparse_bwd_dedup(h, rowref, offsets, n_bags: int, nnz: int, ws, stream=None):
    import torch
    _check(lib().sparse_bwd_dedup(
        h, _dp(rowref, (torch.int32,)), _dp(offsets, (torch.int32,)), int(n_bags), int(nnz),
        _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def sparse_adagrad_apply(h, n_bags: int, nnz: int, grad, grad_dtype: int, lr: float, eps: float,
                         ws, unique=None, count=None, n_unique=None, stream=None):
    import torch
    _check(lib().sparse_adagrad_apply(
        h, int(n_bags), int(nnz), _dp(grad, (torch.float32, torch.float16)), int(grad_dtype),
        float(lr), float(eps), _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _dp(unique, (torch.int32,)), _dp(count, (torch.int32,)), _dp(n_unique, (torch.int64,)),
        _stream(stream)))


def sparse_ftrl_apply(h, n_bags: int, nnz: int, grad, grad_dtype: int, alpha: float, beta: float,
                      l1: float, l2: float, ws, unique=None, count=None, n_unique=None,
                      stream=None):
    import torch
    _check(lib().sparse_ftrl_apply(
        h, int(n_bags), int(nnz), _dp(grad, (torch.float32, torch.float16)), int(grad_dtype),
        float(alpha), float(beta), float(l1), float(l2), _dp(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _dp(unique, (torch.int32,)),
        _dp(count, (torch.int32,)), _dp(n_unique, (torch.int64,)), _stream(stream)))


def table_fill_linear(h, first: int, n: int, z):
    z = _host(np.asarray(z), np.float32)
    _check(lib().table_fill_linear(h, int(first), int(n), _hp(z)))


def table_export_linear(h, keys, width: int) -> np.ndarray:
    keys = _host(np.asarray(keys).view(np.int64), np.int64)
    z = np.empty(width, dtype=np.float32)
    _check(lib().table_export_linear(h, _hp(keys), int(keys.size), _hp(z)))
    return z


def pass_writeback(h, stream=None):
    _check(lib().pass_writeback(h, _stream(stream)))


def writeback_workspace_bytes(h) -> int:
    n = C.c_size_t()
    _check(lib().writeback_workspace_bytes(h, C.byref(n)))
    return n.value


def pass_writeback_touched(h, ws, stream=None) -> int:
    """Copies back the rows updated since the flash (or the last call); returns the units moved."""
    n = _I64()
    _check(lib().pass_writeback_touched(h, _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                        C.byref(n), _stream(stream)))
    return n.value


def table_dirty_keys(h, clear: bool = False) -> np.ndarray:
    """Keys written back by pass_writeback_touched since the last clear, in rowref order."""
    n = _I64()
    _check(lib().table_dirty_keys(h, None, 0, C.byref(n), 0))
    out = np.empty(n.value, dtype=np.int64)
    _check(lib().table_dirty_keys(h, _hp(out), int(out.size), C.byref(n), int(bool(clear))))
    return out


def table_carry_state(dst, src) -> int:
    """Copies the state of the keys dst shares with src from src's host image; returns their count."""
    n = _I64()
    _check(lib().table_carry_state(dst, src, C.byref(n)))
    return n.value


def table_export(h, keys, width: int, row_dtype: int, want_master: bool):
    """Rows, accumulators (and masters) of `keys` from the host image; `width` = total elements."""
    keys = _host(np.asarray(keys).view(np.int64), np.int64)
    rows = np.empty(width, dtype=np.float16 if row_dtype == EMB_F16 else np.float32)
    acc = np.empty(width, dtype=np.float32)
    master = np.empty(width, dtype=np.float32) if want_master else None
    _check(lib().table_export(h, _hp(keys), int(keys.size), _hp(rows), _hp(acc), _hp(master)))
    return rows, acc, master


def table_fill_state(h, first: int, n: int, row_dtype: int, rows=None, acc=None, master=None):
    """Write rows / acc / master of keys [first, first+n) of the create-time key list into the
    host image (packed in that list's order); takes effect at the next flash."""
    rdt = np.float16 if row_dtype == EMB_F16 else np.float32
    rows = None if rows is None else _host(np.asarray(rows), rdt)
    acc = None if acc is None else _host(np.asarray(acc), np.float32)
    master = None if master is None else _host(np.asarray(master), np.float32)
    _check(lib().table_fill_state(h, int(first), int(n), _hp(rows), _hp(acc), _hp(master)))


def table_key_rowref(h, keys):
    keys = _host(np.asarray(keys).view(np.int64), np.int64)
    rr = np.empty(keys.size, dtype=np.uint32)
    sl = np.empty(keys.size, dtype=np.int64)
    _check(lib().table_key_rowref(h, _hp(keys), int(keys.size), _hp(rr), _hp(sl)))
    return rr, sl


def table_rowref_keys(h, rowrefs):
    rr = _host(np.asarray(rowrefs, dtype=np.uint32), np.uint32)
    out = np.empty(rr.size, dtype=np.int64)
    _check(lib().table_rowref_keys(h, _hp(rr), int(rr.size), _hp(out)))
    return out


def emb_timing_enable(h, enable: bool, only: Optional[str] = None):
    _check(lib().emb_timing_enable(h, int(bool(enable)), None if only is None else only.encode()))


def emb_timing_read(h) -> dict:
    """{kernel name: (launches, total ms)} since the last read."""
    cap = 64
    names = C.create_string_buffer(4096)
    counts = np.zeros(cap, dtype=np.int64)
    ms = np.zeros(cap, dtype=np.float64)
    n = C.c_int32()
    _check(lib().emb_timing_read(h, names, 4096, _hp(counts), _hp(ms), cap, C.byref(n)))
    nm = [s for s in names.value.decode().split("\n") if s]
    return {nm[i]: (int(counts[i]), float(ms[i])) for i in range(min(n.value, cap))}


def table_destroy(h):
    if h:
        lib().table_destroy(h)


# ------------------------------------------------------------------ owning wrapper
class Table:
    """Owns a table handle, its field dims and (after flash) its device arena tensor."""

    def __init__(self, field_dim, row_dtype: int, has_master: bool, n_tables: int,
                 load_factor: float, acc_init: float, keys, rows=None, acc=None, master=None,
                 flags: int = 0, device_ws=None):
        """device_ws: a device tensor of table_build_workspace_bytes() bytes or more to build
        the layout on the GPU (rows, acc and master must then be None; fill them afterwards)."""
        self.field_dim = np.asarray(field_dim, dtype=np.int32)
        self.row_dtype = row_dtype
        self.has_master = bool(has_master)
        if device_ws is not None:
            if rows is not None or acc is not None or master is not None:
                raise ValueError("the device build takes no state; use fill_state")
            self.h = table_create_on_device(self.field_dim, row_dtype, has_master, n_tables,
                                            load_factor, acc_init, keys, device_ws, flags)
        else:
            self.h = table_create_from_prebuilt(self.field_dim, row_dtype, has_master, n_tables,
                                                load_factor, acc_init, keys, rows, acc, master,
                                                flags)
        self.arena = None
        self.info = table_info(self.h)

    @property
    def n_fields(self) -> int:
        return int(self.field_dim.size)

    @property
    def out_width(self) -> int:
        return int(self.field_dim.sum())

    def flash(self, device="cuda", stream=None):
        import torch
        if self.arena is None:
            self.arena = torch.empty(table_device_bytes(self.h), dtype=torch.uint8, device=device)
        pass_flash(self.h, self.arena, stream)

    def fill_linear(self, first: int, n: int, z):
        table_fill_linear(self.h, first, n, z)

    def writeback_touched(self, ws=None, stream=None) -> int:
        import torch
        if ws is None:
            ws = torch.empty(writeback_workspace_bytes(self.h), dtype=torch.uint8,
                             device=self.arena.device)
        return pass_writeback_touched(self.h, ws, stream)

    def carry_from(self, src: "Table") -> int:
        return table_carry_state(self.h, src.h)

    def fill_state(self, first: int, n: int, rows=None, acc=None, master=None):
        table_fill_state(self.h, first, n, self.row_dtype, rows, acc, master)

    def export(self, keys):
        k = np.asarray(keys).view(np.uint64)
        width = int(self.field_dim[(k >> np.uint64(48)).astype(np.int64)].sum())
        return table_export(self.h, k, width, self.row_dtype, self.has_master)

    def export_linear(self, keys):
        k = np.asarray(keys).view(np.uint64)
        width = int(self.field_dim[(k >> np.uint64(48)).astype(np.int64)].sum())
        return table_export_linear(self.h, k, width)

    def close(self):
        table_destroy(self.h)
        self.h = None
        self.arena = None

    def __del__(self):
        try:
            if getattr(self, "h", None):
                table_destroy(self.h)
        except Exception:
            pass
