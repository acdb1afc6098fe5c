"""Parity of the HIP path with the CPU oracle on the large workloads, at their
full sizes, in the launch configuration bench.py times (one grouped call over
every matrix of the stack).  The oracle runs on a sample of the matrices (it
needs minutes per large matrix); every matrix is checked for bit-exact
momentum where that is cheap, and the rest through properties.

Gates (relative Frobenius error of the update O):
  * bf16 path on Gaussian gradients (3.8B-like): <= 2e-2 against float64.
  * bf16 path on the d24 gradients (rank 16 + noise, so most singular values
    sit near the bf16 quantisation floor, where the quintic amplifies any
    difference by up to 3.4445 per step, and the float64 error of any bf16
    evaluation is ~0.2-0.3 after 5 steps): against the oracle's bf16-storage
    emulation (float64 sums) within D24_EMU_GATE after 1, 2 and 5 steps of the
    same grouped launch.  Binary32 accumulation alone, in the order the
    matrix instructions sum, sits 4.7-5.0e-6, 4.3-4.5e-4 and 2.7-3.0e-2 from
    the emulation after 1, 2 and 5 steps (tests/diag_binary32_accumulation.py);
    leaving one storage point out (A unrounded) moves the result 2.8e-5 and
    1.0e-3 after 1 and 2 steps, so the short runs pin the storage points.
    After 5 steps also: no less accurate against float64 than the emulation
    (at most 1.1 x its error + 2e-3); <= 2e-2 on the dominant rank-16 block
    against float64; the dominant singular values inside the quintic's band.
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
# d24 bf16 path against the bf16-storage emulation, per number of steps: about
# 2.5 x (1 step), 1.6 x (2) and 1.5 x (5) the distance binary32 accumulation
# alone produces, and below the 2.8e-5 and 1.0e-3 of a misplaced storage point
D24_EMU_GATE = {1: 1.2e-5, 2: 7e-4, 5: 4.5e-2}
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
    kw = dict(lr=lr, beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs, precision=mb.NS_BF16)
    u_host = {i: orc.momentum(host[i][2], host[i][1], wl.beta, wl.nesterov)[1] for i in sample}
    # 1 and 2 steps of the same grouped launch, on copies of W and M: the
    # storage points, before the quintic's amplification takes over
    for k in (1, 2):
        wk = [x.clone() for x in w]
        mk = [x.clone() for x in m]
        upd_k = [torch.empty((s.rows, s.cols), device="cuda") if i in sample[:3] else None
                 for i, s in enumerate(wl.specs)]
        mb.muon_step_batched(wk, g, mk, ns_steps=k, updates_out=upd_k, **kw)
        torch.cuda.synchronize()
        for i in sample[:3]:
            emu = orc.orthogonalise_bf16_storage(u_host[i], wl.coeffs, k)
            e = orc.rel_frobenius(to_np(upd_k[i]), emu)
            print(f"d24[{i}] {k} step(s): rel-F vs bf16-storage emulation {e:.3e} (gate {D24_EMU_GATE[k]:.1e})")
            assert e <= D24_EMU_GATE[k]
        del wk, mk, upd_k
    t0 = time.time()
    mb.muon_step_batched(w, g, m, ns_steps=wl.ns_steps, updates_out=upd, **kw)
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
        assert e_emu <= D24_EMU_GATE[wl.ns_steps]
        assert e_top <= TOL_BF16
        assert MUON_BAND_K5[0] - 0.02 <= sv_top.min() and sv_top.max() <= MUON_BAND_K5[1] + 0.02
        assert np.linalg.norm(o, 2) <= MUON_MAX * 1.02


def test_lm38_full_stack():
    _announce("3.8B-like full stack (192 matrices), bf16, resident in HBM")
    wl = wlm.workload("lm3p8b_bf16")
    n = len(wl.specs)
    w, g, m = _run_stack(wl)
    sample = [1, 2, 0, 4, 5]              # K, V (3072x1024, tall), Q (3072^2), up (3072x12288), down of layer 0
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


def scalar_map(coeffs, k, sigma):
    """p^k on singular values, p(s) = a s + b s^3 + c s^5."""
    a, b, c = coeffs
    s = np.asarray(sigma, dtype=np.float64)
    for _ in range(k):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def _spectral_norm(o, iters=30, seed=0):
    """Largest singular value of o by power iteration on o^T o (float64)."""
    o = np.asarray(o, dtype=np.float64)
    v = np.random.default_rng(seed).standard_normal(o.shape[1])
    for _ in range(iters):
        v = o.T @ (o @ v)
        v /= np.linalg.norm(v)
    return float(np.linalg.norm(o @ v))


def test_stress_stack_bf16x3():
    _announce("stress stack (64 mixed matrices), split-bf16, 10 steps")
    wl = wlm.workload("stress_mixed_bf16")
    w, g, m = _run_stack(wl)
    # small matrices, and every aspect the 8192 matrices of the stack take
    # whose float64 oracle stays cheap (Gram side <= 1024): 8192 x 1024 (tall),
    # 1024 x 8192 and 512 x 8192 (16:1)
    small = [i for i, s in enumerate(wl.specs) if s.rows * s.cols <= 1024 * 2048][:6]
    wide = {(8192, 1024): None, (1024, 8192): None, (512, 8192): None}
    for i, s in enumerate(wl.specs):
        if (s.rows, s.cols) in wide and wide[(s.rows, s.cols)] is None:
            wide[(s.rows, s.cols)] = i
    small += [i for i in wide.values() if i is not None]
    squares = [i for i, s in enumerate(wl.specs) if (s.rows, s.cols) == (8192, 8192)]
    host = {i: (to_np(w[i]), to_np(g[i]), to_np(m[i])) for i in small}
    host8192 = {i: (None, to_np(g[i]), to_np(m[i])) for i in squares[:1]}
    upd = [torch.empty((s.rows, s.cols), device="cuda") if i in small + squares else None
           for i, s in enumerate(wl.specs)]
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
    # the 8192 x 8192 matrices: finite, and their largest singular value
    # within the quintic's bound; the first against the float64 oracle
    for k, i in enumerate(squares):
        o = to_np(upd[i])
        assert np.isfinite(o).all()
        top = _spectral_norm(o)
        msg = f"stress[{i}] 8192x8192: largest singular value {top:.4f}"
        if k == 0:
            t0 = time.time()
            ref = orc.orthogonalise(orc.momentum(host8192[i][2], host8192[i][1], wl.beta, wl.nesterov)[1],
                                    wl.coeffs, wl.ns_steps)
            err = orc.rel_frobenius(o, ref)
            msg += f", split-bf16 rel-F vs float64 {err:.2e} (oracle {time.time() - t0:.0f} s)"
            assert err <= TOL_BF16
        print(msg)
        assert top <= MUON_MAX * 1.001
    del w, g, m, w_b, m_b
    mb.muon_release_workspace()
    torch.cuda.empty_cache()


# With a binary32 gradient the i^-2 tail reaches singular values of 1e-6
# (8192 x 1024) to 1e-8 (8192 x 8192), where p^10 is linear with gain
# 3.4445^10 = 2.4e5.  Split-bf16 operands carry about 16 bits: a storage error
# of 2^-17 |x|, about 4.4e-6 in Frobenius norm per stored matrix, amplified
# there, is a few per cent of ||O|| (measured 3.3e-2 and 4.1e-2); it gets
# this bound, and the binary32 path the 2e-2 contract.  (With the stack's
# bf16 gradients the bf16 noise floor, near 2e-5, lifts the tail out of the
# linear range: split-bf16 is within 4.3e-3 of float64 there.)
TOL_BF16X3_DEEP_TAIL = 5e-2
@pytest.mark.parametrize("rows,cols,prec,gate", [
    (8192, 8192, mb.NS_F32, TOL_BF16),
    (8192, 1024, mb.NS_F32, TOL_BF16),
    (8192, 8192, mb.NS_BF16X3, TOL_BF16X3_DEEP_TAIL),
    (8192, 1024, mb.NS_BF16X3, TOL_BF16X3_DEEP_TAIL),
])
def test_stress_shapes_against_the_closed_form(rows, cols, prec, gate):
    """The stress construction at its largest shapes, with the gradient kept
    in binary32 so that it carries the i^-2 spectrum: O must equal
    Q_u diag(p^10(s/||s||)) Q_v^T (float64, no iteration) within `gate`.  A
    bf16 gradient would move the spectrum below the bf16 floor by O(1) and
    void the closed form.  The factors are drawn in float64 on the GPU (input
    generation only); the expected value is formed on the host.  Split-bf16
    is held to its own, derived bound (TOL_BF16X3_DEEP_TAIL)."""
    _announce(f"stress construction {rows}x{cols}, binary32 gradient, precision {prec}, 10 steps, closed form")
    wl = wlm.workload("stress_mixed_bf16")
    qu, s, qv = wlm.spectral_factors(rows, cols, wl.seed, 1000 + rows // 1024 + cols, device="cuda")
    g = ((qu * s) @ qv.t()).float().contiguous()
    w = (torch.randn(rows, cols, device="cuda") * 0.02).to(torch.bfloat16)
    m = torch.zeros(rows, cols, device="cuda")
    o = torch.empty(rows, cols, device="cuda")
    lr = f32(wl.lr)
    w0 = to_np(w)
    mb.muon_step_batched([w], [g], [m], lr=lr, beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs,
                         ns_steps=wl.ns_steps, precision=prec, updates_out=[o])
    torch.cuda.synchronize()
    assert torch.equal(m, g)
    qu_h, s_h, qv_h = (t.cpu().numpy() for t in (qu, s, qv))
    del qu, s, qv
    p = scalar_map(wl.coeffs, wl.ns_steps, s_h / np.linalg.norm(s_h))
    ref = (qu_h * p) @ qv_h.T
    oh = to_np(o)
    err = orc.rel_frobenius(oh, ref)
    top = _spectral_norm(oh)
    print(f"{rows}x{cols} precision {prec}: rel-F vs closed form {err:.2e} (gate {gate:.0e}); largest singular "
          f"value {top:.4f} (closed form {p.max():.4f})")
    assert err <= gate
    # Weyl: every singular value moves by at most ||O - ref||_2 <= ||O - ref||_F
    assert abs(top - p.max()) <= np.linalg.norm(oh - ref) + 1e-6
    assert top <= MUON_MAX * 1.001
    assert np.array_equal(bits(to_np(w)), bits(orc.write_back(w0, oh, lr, 1.0, True)))
    del w, g, m, o
    torch.cuda.empty_cache()
