"""Shared helpers of the GPU parity tests (not collected as tests)."""
import numpy as np
import torch

import oracle as orc
from muon_newton_schulz_02_amd import binding as mb

# Gates, relative Frobenius error of the update O against the float64 oracle:
# 1e-4 for the float32 path and 2e-2 for the bf16 path (the tolerances the
# library is specified to); the split-bf16 path is held to the bf16 gate and, on
# well-conditioned inputs, to TOL_BF16X3_TIGHT (about 16 significant bits per
# operand, five products per step: errors of order 1e-4 expected).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_BF16X3_TIGHT = 2e-3

MUON = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)
TEXTBOOK = (15 / 8, -5 / 4, 3 / 8)

PREC_TOL = {mb.NS_F32: TOL_F32, mb.NS_BF16X3: TOL_BF16X3_TIGHT, mb.NS_BF16: TOL_BF16}


def f32(x):
    return float(np.float32(x))


def to_np(t):
    return t.detach().float().cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def run_step(ws, gs, ms, *, lr, beta, nesterov, coeffs, steps, precision, scale_rule=0, dev="cuda"):
    """Copy host tensors to the GPU, run one step with the update exported,
    and return the new (W, M, O) lists as numpy arrays plus device tensors."""
    w_d = [w.to(dev) for w in ws]
    g_d = [g.to(dev) for g in gs]
    m_d = [m.to(dev) for m in ms]
    u_d = [torch.full(tuple(g.shape), float("nan"), dtype=torch.float32, device=dev) for g in gs]
    mb.muon_step_batched(w_d, g_d, m_d, lr=lr, beta=beta, nesterov=nesterov, ns_coeffs=coeffs,
                         ns_steps=steps, precision=precision, scale_rule=scale_rule, updates_out=u_d)
    torch.cuda.synchronize()
    return [to_np(w) for w in w_d], [to_np(m) for m in m_d], [to_np(u) for u in u_d]


def check_step(w0, g0, m0, w1, m1, o1, *, lr, beta, nesterov, coeffs, steps, tol, param_bf16,
               scale_rule=0, ref_storage="fp64"):
    """Momentum bit-exact, O within tol of the oracle, W bit-exact given O."""
    ref = orc.muon_step(w0, g0, m0, lr=lr, beta=beta, nesterov=nesterov, coeffs=coeffs, steps=steps,
                        scale_rule=scale_rule, param_bf16=param_bf16, storage=ref_storage)
    assert np.array_equal(bits(m1), bits(ref.m)), "momentum not bit-exact"
    err = orc.rel_frobenius(o1, ref.o)
    assert err <= tol, f"update rel-F error {err:.3e} > {tol:.1e}"
    s = orc.scale_factor(scale_rule, *np.asarray(w0).shape)
    w_exp = orc.write_back(w0, o1, lr, s, param_bf16)
    assert np.array_equal(bits(w1), bits(w_exp)), "write-back not bit-exact given O"
    return err, ref
