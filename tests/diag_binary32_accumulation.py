"""How far binary32 accumulation alone moves the bf16-storage Newton-Schulz
result away from the oracle's bf16-storage emulation (which sums in float64).

    python tests/diag_binary32_accumulation.py [matrix index ...]

A diagnostic, not a test and not the oracle: it derives the tolerance of the
d24 parity gate.  The bf16 path stores U, A, B and every iterate in bfloat16
and accumulates each product in binary32.  The method leaves the order of a
product's sum open, so the oracle's emulation (oracle.orthogonalise_bf16_storage)
sums in float64.  This script evaluates the same storage points with one
binary32 rounding per 16-term slab of every sum, slabs in increasing k (the
order in which the GPU's 32x32x16 bf16 matrix instructions accumulate), and
the additive terms a X and (b/c) A added as a bf16 hi + lo pair after the slab
that holds the output row, then reports its distance from the emulation after
1..5 steps on the d24 gradients (rank 16 plus noise).

The rank-16-plus-noise gradients put most singular values at the bf16
quantisation floor, where the quintic amplifies any difference by up to
3.4445 per step; a binary32 sum that rounds a stored value the other way
than the float64 sum is such a difference.  Measured on two d24 matrices
(1536 x 1536 and 1536 x 6144; host generator): 4.7e-6, 4.3e-4, 3.3e-3,
8.2e-3 and 3.0e-2 after 1..5 steps, and 2.6e-2 after 5 steps on the
rectangular one.  The GPU path is at the same distance at every step
(recorded with the parity gate in the design notes).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as orc  # noqa: E402
from muon_newton_schulz_02_amd import workloads as wlm  # noqa: E402

SLAB = 16


def _bf16(x):
    return orc.to_bf16(np.asarray(x, dtype=np.float32))


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _hi_lo(alpha):
    """alpha (binary32) as hi + lo, both bfloat16."""
    a = np.float32(alpha)
    hi = np.float32(_bf16(a))
    lo = np.float32(_bf16(np.float32(a - hi)))
    return hi, lo


def slab_product(p, q, ident=None):
    """acc[i][j] = sum_k p[i][k] q[j][k], rounded to binary32 after every
    SLAB consecutive k (each slab summed exactly).  ident = (hi, lo, d): after
    the slab holding k = i, add lo*d[i][j] and then hi*d[i][j], each rounded."""
    m, n = p.shape[0], q.shape[0]
    k_all = p.shape[1]
    acc = np.zeros((m, n), np.float32)
    p64 = p.astype(np.float64)
    q64 = q.astype(np.float64)
    for k0 in range(0, k_all, SLAB):
        acc = _f32(acc.astype(np.float64) + p64[:, k0:k0 + SLAB] @ q64[:, k0:k0 + SLAB].T)
        if ident is not None and k0 < m:
            hi, lo, d = ident
            rows = slice(k0, min(k0 + SLAB, m))
            d64 = d[rows].astype(np.float64)
            acc[rows] = _f32(acc[rows].astype(np.float64) + np.float64(lo) * d64)
            acc[rows] = _f32(acc[rows].astype(np.float64) + np.float64(hi) * d64)
    return acc


def binary32_storage_ns(u, coeffs, steps, norm=None):
    """The iterates X_1 .. X_steps (oriented back) of the bf16-storage
    schedule with binary32 slab accumulation.  `norm` is ||U||_F as binary32
    (default: a binary32 sum of squares)."""
    u = _f32(u)
    tr = u.shape[0] > u.shape[1]
    xw = u.T if tr else u
    if norm is None:
        norm = np.float32(np.sqrt(np.sum(u * u, dtype=np.float32)))
    inv = np.float32(np.float32(1.0) / np.float32(np.float32(norm) + np.float32(orc.EPS)))
    inv2 = np.float32(inv * inv)
    x = _bf16(xw)
    outs = []
    for k in range(steps):
        a, b, c = (np.float32(v) for v in coeffs)
        m = x.shape[0]
        first = k == 0
        gram = slab_product(x, x)
        if c != 0:
            a_st = _bf16(_f32((inv2 if first else np.float32(1)) * gram))
            hi, lo = _hi_lo(np.float32(b / c))
            b_st = _bf16(_f32(c * slab_product(a_st, a_st, ident=(hi, lo, a_st))))
        else:
            b_st = _bf16(_f32(np.float32((inv2 if first else np.float32(1)) * b) * gram))
        hi, lo = _hi_lo(a)
        comb = slab_product(b_st, np.ascontiguousarray(x.T), ident=(hi, lo, x))
        xn = _f32((inv if first else np.float32(1)) * comb)
        if k < steps - 1:
            x = _bf16(xn)
        outs.append(xn.T if tr else xn)
    return outs


def main(argv):
    wl = wlm.workload("d24_bf16", layers=1)
    idxs = [int(a) for a in argv] or [0, 4]
    for idx in idxs:
        g = wlm.gradient(wl, idx, 0).float().numpy()
        _, u = orc.momentum(np.zeros_like(g), g, wl.beta, wl.nesterov)
        t = time.time()
        model = binary32_storage_ns(u, wl.coeffs, wl.ns_steps)
        print(f"d24[{idx}] {g.shape[0]}x{g.shape[1]}: binary32 evaluation {time.time() - t:.1f} s", flush=True)
        for k in range(1, wl.ns_steps + 1):
            emu = orc.orthogonalise_bf16_storage(u, wl.coeffs, k)
            ref = orc.orthogonalise(u, wl.coeffs, k)
            print(f"  k={k}: binary32 vs emulation {orc.rel_frobenius(model[k - 1], emu):.3e}, "
                  f"binary32 vs float64 {orc.rel_frobenius(model[k - 1], ref):.3e}, "
                  f"emulation vs float64 {orc.rel_frobenius(emu, ref):.3e}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
