"""Parity of the HIP path with the CPU oracle on the large workloads, at their
full sizes, in the launch configuration bench.py times (one grouped call over
every matrix of the stack).  The oracle runs on a sample of the matrices (it
needs minutes per large matrix); every matrix is checked for bit-exact
momentum where that is cheap, and the rest through properties.

Gates (relative Frobenius error of the update O):
  * bf16 path on Gaussian gradients (3.8B-like): <= 2e-2 against float64.
  * bf16 path on the d24 gradients (rank 16 + noise, so most singular values
    sit near the bf16 quantisation floor, where the quintic amplifies storage
    noise to O(1), and the float64 error of any bf16 evaluation is ~0.2-0.3):
    no less accurate against float64 than the oracle's own bf16-storage
    emulation (at most 1.1 x its error + 2e-3); <= 2e-2 on the dominant
    rank-16 block against float64; the dominant singular values inside the
    quintic's band; and within 5e-2 of the emulation (two bf16 evaluations
    that differ only in accumulation order already differ by 1e-2 to 3e-2
    in this regime, so the emulation cannot be matched more closely).
  * split-bf16 path on the stress stack: <= 2e-2 against float64 (and the
    band); plain bf16 on the same inputs is printed, not gated.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle as orc
from muon_newton_schulz_02_amd import binding as mb
from muon_newton_schulz_02_amd import workloads as wlm

from gpu_helpers import TOL_BF16, bits, f32, to_np

pytestmark = pytest.mark.gpu

MUON_BAND_K5 = (0.6818, 1.1344)     # p^5 over singular values in [1e-2, 1], Muon triple
MUON_MAX = 1.2024                    # max of p over [0, 1]


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _run_stack(wl, dev="cuda", precision=None):
    n = len(wl.specs)
    st = [wlm.initial_state(wl, i, device=dev) for i in range(n)]
    w = [s[0] for s in st]
    m = [s[1] for s in st]
    g = [wlm.gradient(wl, i, 0, device=dev) for i in range(n)]
    return w, g, m


def _top_subspace(g64, k=16):
    from scipy.sparse.linalg import svds
    u, s, vt = svds(g64, k=k)
    return u, vt.T


def test_d24_full_stack():
    _announce("d24 full stack (144 matrices), bf16")
    wl = wlm.workload("d24_bf16")
    n = len(wl.specs)
    w, g, m = _run_stack(wl)
    sample = [0, 4, 5, 76, 142, 143]      # Q, up, down of layer 0; layer 12 Q-proj; last up, down
    host = {i: (to_np(w[i]), to_np(g[i]), to_np(m[i])) for i in sample}
    upd = [torch.empty((s.rows, s.cols), device="cuda") if i in sample else None for i, s in enumerate(wl.specs)]
    lr = f32(wl.lr)
    t0 = time.time()
    mb.muon_step_batched(w, g, m, lr=lr, beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs,
                         ns_steps=wl.ns_steps, precision=mb.NS_BF16, updates_out=upd)
    torch.cuda.synchronize()
    print(f"gpu step {time.time() - t0:.3f} s")
    # every matrix: momentum started at 0, so M' = G bit for bit
    for i in range(n):
        assert torch.equal(m[i], g[i].float()), f"matrix {i}: momentum"
        assert torch.isfinite(w[i]).all()
    for i in sample:
        w0, g0, m0 = host[i]
        o = to_np(upd[i])
        ref64 = orc.muon_step(w0, g0, m0, lr=lr, beta=wl.beta, nesterov=wl.nesterov, coeffs=wl.coeffs,
                              steps=wl.ns_steps, param_bf16=True)
        emu = orc.orthogonalise_bf16_storage(ref64.u, wl.coeffs, wl.ns_steps)
        assert np.array_equal(bits(to_np(m[i])), bits(ref64.m))
        w_exp = orc.write_back(w0, o, lr, 1.0, True)
        assert np.array_equal(bits(to_np(w[i])), bits(w_exp)), f"matrix {i}: write-back"
        e_emu = orc.rel_frobenius(o, emu)
        e_64 = orc.rel_frobenius(o, ref64.o)
        e_emu64 = orc.rel_frobenius(emu, ref64.o)
        u16, v16 = _top_subspace(g0.astype(np.float64))
        blk_gpu = u16.T @ o @ v16
        blk_64 = u16.T @ ref64.o @ v16
        e_top = orc.rel_frobenius(blk_gpu, blk_64)
        sv_top = np.linalg.svd(blk_gpu, compute_uv=False)
        print(f"d24[{i}] {wl.specs[i].rows}x{wl.specs[i].cols}: rel-F vs float64 {e_64:.3e} "
              f"(emulation vs float64 {e_emu64:.3e}), vs emulation {e_emu:.2e}, top-16 block vs float64 "
              f"{e_top:.2e}, top sv [{sv_top.min():.4f}, {sv_top.max():.4f}]")
        assert e_64 <= 1.1 * e_emu64 + 2e-3
        assert e_emu <= 5e-2
        assert e_top <= TOL_BF16
        assert MUON_BAND_K5[0] - 0.02 <= sv_top.min() and sv_top.max() <= MUON_BAND_K5[1] + 0.02
        assert np.linalg.norm(o, 2) <= MUON_MAX * 1.02


def test_lm38_full_stack():
    _announce("3.8B-like full stack (192 matrices), bf16, resident in HBM")
    wl = wlm.workload("lm3p8b_bf16")
    n = len(wl.specs)
    w, g, m = _run_stack(wl)
    sample = [1, 2, 0]                    # K, V (3072x1024, tall) and Q (3072^2) of layer 0
    host = {i: (to_np(w[i]), to_np(g[i]), to_np(m[i])) for i in sample}
    upd = [torch.empty((s.rows, s.cols), device="cuda") if i in sample else None for i, s in enumerate(wl.specs)]
    lr = f32(wl.lr)
    mb.muon_step_batched(w, g, m, lr=lr, beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs,
                         ns_steps=wl.ns_steps, precision=mb.NS_BF16, updates_out=upd)
    torch.cuda.synchronize()
    for i in range(n):
        assert torch.equal(m[i], g[i].float()), f"matrix {i}: momentum"
    for i in sample:
        w0, g0, m0 = host[i]
        o = to_np(upd[i])
        ref = orc.muon_step(w0, g0, m0, lr=lr, beta=wl.beta, nesterov=wl.nesterov, coeffs=wl.coeffs,
                            steps=wl.ns_steps, param_bf16=True)
        err = orc.rel_frobenius(o, ref.o)
        print(f"lm38[{i}] {wl.specs[i].rows}x{wl.specs[i].cols}: rel-F vs float64 {err:.2e}")
        assert err <= TOL_BF16
        assert np.array_equal(bits(to_np(w[i])), bits(orc.write_back(w0, o, lr, 1.0, True)))
    # release this test's tensors before the next large test
    del w, g, m, upd
    mb.muon_release_workspace()
    torch.cuda.empty_cache()


def test_stress_stack_bf16x3():
    _announce("stress stack (64 mixed matrices), split-bf16, 10 steps")
    wl = wlm.workload("stress_mixed_bf16")
    w, g, m = _run_stack(wl)
    small = [i for i, s in enumerate(wl.specs) if s.rows * s.cols <= 1024 * 2048][:6]
    host = {i: (to_np(w[i]), to_np(g[i]), to_np(m[i])) for i in small}
    upd = [torch.empty((s.rows, s.cols), device="cuda") if i in small else None for i, s in enumerate(wl.specs)]
    lr = f32(wl.lr)
    # the same inputs through the plain bf16 path, for the report
    w_b = [x.clone() for x in w]
    m_b = [x.clone() for x in m]
    upd_b = [torch.empty((s.rows, s.cols), device="cuda") if i in small else None for i, s in enumerate(wl.specs)]
    mb.muon_step_batched(w, g, m, lr=lr, beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs,
                         ns_steps=wl.ns_steps, precision=mb.NS_BF16X3, updates_out=upd)
    mb.muon_step_batched(w_b, g, m_b, lr=lr, beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs,
                         ns_steps=wl.ns_steps, precision=mb.NS_BF16, updates_out=upd_b)
    torch.cuda.synchronize()
    for i, s in enumerate(wl.specs):
        assert torch.equal(m[i], g[i].float()) and torch.isfinite(w[i]).all()
    for i in small:
        w0, g0, m0 = host[i]
        ref = orc.muon_step(w0, g0, m0, lr=lr, beta=wl.beta, nesterov=wl.nesterov, coeffs=wl.coeffs,
                            steps=wl.ns_steps, param_bf16=True)
        o = to_np(upd[i])
        err = orc.rel_frobenius(o, ref.o)
        err_b = orc.rel_frobenius(to_np(upd_b[i]), ref.o)
        sv = np.linalg.svd(o, compute_uv=False)
        print(f"stress[{i}] {wl.specs[i].rows}x{wl.specs[i].cols}: split-bf16 rel-F {err:.2e}, "
              f"plain bf16 {err_b:.2e}, sv max {sv.max():.4f}")
        assert err <= TOL_BF16
        assert sv.max() <= MUON_MAX * 1.001
        assert np.array_equal(bits(to_np(w[i])), bits(orc.write_back(w0, o, lr, 1.0, True)))
    del w, g, m, w_b, m_b
    mb.muon_release_workspace()
    torch.cuda.empty_cache()
