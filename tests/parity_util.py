"""GPU-vs-oracle step runner shared by the parity tests and the benchmark's sampled check.

Tolerances (fp32 1e-5, fp16-stored 2e-3, relative) are taken against scales derived from the
arithmetic, so that cancellation in a sum cannot turn a tiny rounding difference into a large
"relative" error:
  pooled element      : sum over the bag of |row element|             (fp32 sum of n terms)
  gradient element    : S_g = sum over occurrences of |G element|
  accumulator         : acc' + 2 |g| S_g                               (error of g^2)
  row / master element: |w_prev| + lr * S_g / (sqrt(acc') + eps)        (error of delta via g)
Per-step budgets add up over steps, because an error in w_k carries one-for-one into w_{k+1}.
fp16-stored rows add one fp16 subnormal step (2^-24) per update for the final rounding.

FTRL-Proximal (n' = n + g^2, sigma = (sqrt n' - sqrt n)/alpha, z' = z + g - sigma w,
w' = -(z' - sign(z') l1) / q with q = (beta + sqrt n')/alpha + l2, or 0 when |z'| <= l1), each
error propagated one-for-one and each operation adding TOL_F32 times the magnitude of its operands:
  sqrt(n)             : TOL sqrt(n) + err_n / (2 sqrt n)   (sqrt(err_n) where n is 0)
  sigma               : (err_sqrt n' + err_sqrt n) / alpha + TOL |sigma|
  z'                  : err_z + err_g + err_sigma |w| + |sigma| err_w + TOL (|z| + |g| + |sigma w| + |z'|)
  q                   : err_sqrt n' / alpha + TOL q
  w'                  : (err_z' + TOL (|z'| + l1)) / q + |w'| err_q / q + TOL |w'|
The soft threshold is continuous in z', so a decision |z'| <= l1 taken differently on the two sides
moves w' by at most err_z' / q, which the w' budget covers.
"""
from __future__ import annotations

import numpy as np

from oracle import emb_oracle as O

TOL_F32 = 1e-5
TOL_F16 = 2e-3
F16_TINY = 2.0 ** -24


def take(flat, roff, idx):
    """The packed rows of entries `idx` (in that order) of a packed array with offsets `roff`."""
    if flat is None:
        return None
    idx = np.asarray(idx, dtype=np.int64)
    lens = roff[idx + 1] - roff[idx]
    starts = np.repeat(roff[idx], lens)
    within = np.arange(int(lens.sum())) - np.repeat(np.cumsum(lens) - lens, lens)
    return flat[starts + within]


def oracle_table(w, keys, rows, master, dims):
    return O.Table(keys, dims, w.row_dtype, w.has_master, w.n_tables, w.load_factor, w.acc_init,
                   rows, master=master)


def pooled_scale(ot: O.Table, keys, offsets, bud=None):
    """Per pooled element: the sum over the bag of |row element| (float64, [B, width]); with a
    Budget, plus the sum of the rows' accumulated error budgets (rows updated by earlier steps
    already differ within those budgets)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    kidx, _, _ = ot.lookup(keys, offsets)
    bag = O.bag_of_occurrence(offsets)
    B = (offsets.size - 1) // ot.F
    tol = TOL_F32 if ot.row_dtype == "f32" else TOL_F16
    S = np.zeros((B, int(ot.col[-1])), dtype=np.float64)
    for f in range(ot.F):
        D = int(ot.dims[f])
        sel = np.nonzero((bag % ot.F == f) & (kidx >= 0))[0]
        if sel.size == 0:
            continue
        ro = ot.roff[kidx[sel]]
        el = ro[:, None] + np.arange(D)[None, :]
        g = np.abs(ot.rows[el].astype(np.float64))
        if bud is not None:
            g = g + bud.row[el] / tol
        np.add.at(S, (bag[sel] // ot.F, slice(int(ot.col[f]), int(ot.col[f]) + D)), g)
    return S


class Budget:
    """Per-element error budgets of the oracle state (same packing as ot.rows)."""

    def __init__(self, ot: O.Table):
        n = ot.rows.size
        self.acc = np.zeros(n)
        self.row = np.zeros(n)
        self.master = np.zeros(n)
        self.lin = np.zeros(n)
        self.touched = np.zeros(ot.keys.size, dtype=bool)

    def oracle_step(self, ot: O.Table, keys, offsets, grad, lr, eps):
        """Run the oracle's backward and grow the budgets of the rows it touched."""
        g = ot.row_grads(keys, offsets, grad)
        Sg = ot.row_grads(keys, offsets, np.abs(np.asarray(grad, dtype=np.float64)))
        w_prev = {}
        for u in g:
            a, b = int(ot.roff[u]), int(ot.roff[u + 1])
            src = ot.master if ot.master is not None else ot.rows
            w_prev[u] = np.abs(src[a:b].astype(np.float64))
        t = ot.touched(keys, offsets)
        ot.adagrad_rows(g, lr, eps)
        lr32 = float(np.float32(lr))
        for u, gu in g.items():
            a, b = int(ot.roff[u]), int(ot.roff[u + 1])
            accn = ot.acc[a:b].astype(np.float64)
            self.acc[a:b] += TOL_F32 * (accn + 2 * np.abs(gu) * Sg[u])
            dscale = lr32 * Sg[u] / (np.sqrt(accn) + eps)
            self.master[a:b] += TOL_F32 * (w_prev[u] + dscale)
            if ot.row_dtype == "f32":
                self.row[a:b] += TOL_F32 * (w_prev[u] + dscale)
            else:
                self.row[a:b] += TOL_F16 * (w_prev[u] + dscale) + F16_TINY
            self.touched[u] = True
        return t


    def oracle_step_ftrl(self, ot: O.Table, keys, offsets, grad, alpha, beta, l1, l2):
        """Run the oracle's FTRL backward and grow the budgets of the rows it touched."""
        g = ot.row_grads(keys, offsets, grad)
        Sg = ot.row_grads(keys, offsets, np.abs(np.asarray(grad, dtype=np.float64)))
        prev = {}
        for u in g:
            a, b = int(ot.roff[u]), int(ot.roff[u + 1])
            src = ot.master if ot.master is not None else ot.rows
            prev[u] = (ot.acc[a:b].astype(np.float64), src[a:b].astype(np.float64),
                       ot.linear[a:b].astype(np.float64))
        t = ot.touched(keys, offsets)
        ot.ftrl_rows(g, alpha, beta, l1, l2)
        alpha, beta = float(np.float32(alpha)), float(np.float32(beta))
        l1, l2 = float(np.float32(l1)), float(np.float32(l2))

        def sqrt_err(n, en):
            r = np.sqrt(n)
            return TOL_F32 * r + np.where(n > 0, en / (2 * np.maximum(r, 1e-300)), np.sqrt(en))
        for u, gu in g.items():
            a, b = int(ot.roff[u]), int(ot.roff[u + 1])
            n0, w0, z0 = prev[u]
            en0 = self.acc[a:b].copy()
            ew0 = self.master[a:b] if ot.master is not None else self.row[a:b]
            ez0 = self.lin[a:b].copy()
            eg = TOL_F32 * Sg[u]
            n1 = n0 + gu * gu
            en1 = en0 + TOL_F32 * (n1 + 2 * np.abs(gu) * Sg[u])
            es0, es1 = sqrt_err(n0, en0), sqrt_err(n1, en1)
            sig = (np.sqrt(n1) - np.sqrt(n0)) / alpha
            esig = (es0 + es1) / alpha + TOL_F32 * np.abs(sig)
            z1 = z0 + gu - sig * w0
            ez1 = (ez0 + eg + esig * np.abs(w0) + np.abs(sig) * ew0 +
                   TOL_F32 * (np.abs(z0) + np.abs(gu) + np.abs(sig * w0) + np.abs(z1)))
            q = (beta + np.sqrt(n1)) / alpha + l2
            eq = es1 / alpha + TOL_F32 * q
            w1 = np.where(np.abs(z1) <= l1, 0.0, -(z1 - np.sign(z1) * l1) / q)
            ew1 = (ez1 + TOL_F32 * (np.abs(z1) + l1)) / q + np.abs(w1) * eq / q + TOL_F32 * np.abs(w1)
            self.acc[a:b] = en1
            self.lin[a:b] = ez1
            self.master[a:b] = ew1
            if ot.row_dtype == "f32":
                self.row[a:b] = ew1
            else:
                self.row[a:b] = ew1 + TOL_F16 * np.abs(w1) + F16_TINY
            self.touched[u] = True
        return t


def check_pooled(out_gpu, out_oracle, scale, out_dtype):
    tol = TOL_F32 if out_dtype == "f32" else TOL_F16
    absl = 0.0 if out_dtype == "f32" else F16_TINY
    d = np.abs(np.asarray(out_gpu, dtype=np.float64) - np.asarray(out_oracle, dtype=np.float64))
    lim = tol * scale + absl
    bad = d > lim
    assert not bad.any(), (f"pooled mismatch at {np.argwhere(bad)[:5].tolist()}: "
                           f"max excess {(d - lim).max():.3g}")


def check_state(ot: O.Table, bud: Budget, keys_sel, rows_gpu, acc_gpu, master_gpu, lin_gpu=None):
    """Compare exported GPU state of keys_sel with the oracle's, within the budgets."""
    idx = ot.key_index(keys_sel)
    assert np.all(idx >= 0)
    seg = np.concatenate([np.arange(ot.roff[i], ot.roff[i + 1]) for i in idx]) if idx.size else \
        np.zeros(0, dtype=np.int64)
    ro = ot.rows[seg].astype(np.float64)
    d = np.abs(rows_gpu.astype(np.float64) - ro)
    assert np.all(d <= bud.row[seg]), f"rows off by up to {(d - bud.row[seg]).max():.3g}"
    d = np.abs(acc_gpu.astype(np.float64) - ot.acc[seg])
    assert np.all(d <= bud.acc[seg]), f"acc off by up to {(d - bud.acc[seg]).max():.3g}"
    if lin_gpu is not None:
        d = np.abs(lin_gpu.astype(np.float64) - ot.linear[seg])
        assert np.all(d <= bud.lin[seg]), f"linear state off by up to {(d - bud.lin[seg]).max():.3g}"
    if master_gpu is not None:
        d = np.abs(master_gpu.astype(np.float64) - ot.master[seg])
        assert np.all(d <= bud.master[seg]), f"master off by up to {(d - bud.master[seg]).max():.3g}"
        # the stored fp16 row is the rounding of the GPU's own master copy
        assert rows_gpu.tobytes() == master_gpu.astype(np.float16).tobytes()
    # untouched rows and state: bit-identical to the oracle (which never changed them)
    untouched = ~bud.touched[idx]
    if untouched.any():
        oo = np.concatenate([[0], np.cumsum(ot.width[idx])])
        pos = np.concatenate([np.arange(oo[j], oo[j + 1]) for j in np.nonzero(untouched)[0]])
        useg = seg[pos]
        assert rows_gpu[pos].tobytes() == ot.rows[useg].tobytes()
        assert acc_gpu[pos].tobytes() == ot.acc[useg].tobytes()
        if lin_gpu is not None:
            assert lin_gpu[pos].tobytes() == ot.linear[useg].tobytes()
