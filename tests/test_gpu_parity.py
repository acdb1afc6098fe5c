"""Parity of the HIP path (through the C ABI) with the CPU oracle, on small
and ragged shapes, every precision and dtype, and the small workloads.

Each case prints its name before running so a failing GPU run names it."""
import sys

import numpy as np
import pytest
import torch

import oracle as orc
from muon_newton_schulz_02_amd import binding as mb
from muon_newton_schulz_02_amd import workloads as wlm

from gpu_helpers import (CUBIC, MUON, PREC_TOL, TEXTBOOK, TOL_BF16, TOL_F32, bits, check_step, f32,
                         run_step, to_np)

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(shapes, seed, pdt, gdt, m_random=True):
    gen = torch.Generator().manual_seed(seed)
    ws = [(torch.randn(s, generator=gen) * 0.02).to(pdt) for s in shapes]
    gs = [torch.randn(s, generator=gen).to(gdt) for s in shapes]
    ms = [torch.randn(s, generator=gen) if m_random else torch.zeros(s) for s in shapes]
    return ws, gs, ms


SHAPES = [(1, 1), (1, 300), (300, 1), (130, 257), (257, 130), (64, 64), (520, 300), (256, 768), (4097, 5)]


@pytest.mark.parametrize("prec", [mb.NS_F32, mb.NS_BF16X3, mb.NS_BF16])
@pytest.mark.parametrize("steps,coeffs", [(5, MUON), (5, CUBIC), (1, TEXTBOOK), (0, MUON)])
def test_ragged_shapes(prec, steps, coeffs):
    _announce(f"ragged prec={prec} steps={steps} coeffs={coeffs}")
    pdt = torch.bfloat16 if prec == mb.NS_BF16 else torch.float32
    ws, gs, ms = _inputs(SHAPES, 11 + steps, pdt, torch.bfloat16)
    lr = f32(0.02)
    w1, m1, o1 = run_step(ws, gs, ms, lr=lr, beta=0.95, nesterov=True, coeffs=coeffs, steps=steps,
                          precision=prec)
    for i in range(len(SHAPES)):
        check_step(to_np(ws[i]), to_np(gs[i]), to_np(ms[i]), w1[i], m1[i], o1[i], lr=lr, beta=0.95,
                   nesterov=True, coeffs=coeffs, steps=steps, tol=PREC_TOL[prec],
                   param_bf16=pdt == torch.bfloat16)


MULTI_TILE = [(700, 1100), (1100, 700), (769, 769)]


@pytest.mark.parametrize("prec", [mb.NS_BF16X3, mb.NS_BF16])
def test_multi_tile_shapes(prec):
    """Three or more 256-row tiles per symmetric product: blocks below the diagonal
    are read through their mirror in several k-ranges, with ragged edges."""
    _announce(f"multi-tile prec={prec}")
    pdt = torch.bfloat16 if prec == mb.NS_BF16 else torch.float32
    ws, gs, ms = _inputs(MULTI_TILE, 29, pdt, torch.bfloat16)
    lr = f32(0.02)
    w1, m1, o1 = run_step(ws, gs, ms, lr=lr, beta=0.95, nesterov=True, coeffs=MUON, steps=5, precision=prec)
    for i in range(len(MULTI_TILE)):
        check_step(to_np(ws[i]), to_np(gs[i]), to_np(ms[i]), w1[i], m1[i], o1[i], lr=lr, beta=0.95,
                   nesterov=True, coeffs=MUON, steps=5, tol=PREC_TOL[prec], param_bf16=pdt == torch.bfloat16)


@pytest.mark.parametrize("nesterov", [0, 1])
@pytest.mark.parametrize("pdt,gdt", [(torch.float32, torch.float32), (torch.bfloat16, torch.float32),
                                     (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("rule", [mb.SCALE_NONE, mb.SCALE_SQRT_ASPECT, mb.SCALE_RMS_MATCH])
def test_dtypes_nesterov_scale(nesterov, pdt, gdt, rule):
    _announce(f"dtypes {pdt} {gdt} nesterov={nesterov} rule={rule}")
    shapes = [(200, 72), (72, 200), (128, 128)]
    ws, gs, ms = _inputs(shapes, 5, pdt, gdt)
    lr = f32(0.013)
    w1, m1, o1 = run_step(ws, gs, ms, lr=lr, beta=0.9, nesterov=nesterov, coeffs=MUON, steps=5,
                          precision=mb.NS_BF16X3, scale_rule=rule)
    for i in range(len(shapes)):
        check_step(to_np(ws[i]), to_np(gs[i]), to_np(ms[i]), w1[i], m1[i], o1[i], lr=lr, beta=0.9,
                   nesterov=nesterov, coeffs=MUON, steps=5, tol=PREC_TOL[mb.NS_BF16X3],
                   param_bf16=pdt == torch.bfloat16, scale_rule=rule)


@pytest.mark.parametrize("prec,gdt,nesterov", [(mb.NS_BF16X3, torch.bfloat16, 1), (mb.NS_BF16, torch.bfloat16, 1),
                                               (mb.NS_BF16, torch.float32, 0)])
def test_strided_rows(prec, gdt, nesterov):
    """Row strides beyond cols: the momentum pass takes its element path (no
    vector loads); (100, 90) and (300, 130) are tall, so U leaves through the
    LDS transpose (64 x 64 binary32 tiles for split-bf16, 64 x 128 bf16-staged
    tiles for bf16)."""
    _announce(f"strided rows prec={prec} gdt={gdt} nesterov={nesterov}")
    dev = "cuda"
    shapes = [(100, 90), (90, 333), (300, 130)]
    lr = f32(0.02)
    ws_full = [torch.randn(r, c + 24) * 0.02 for r, c in shapes]
    gs_full = [torch.randn(r, c + 8).to(gdt) for r, c in shapes]
    ms_full = [torch.randn(r, c + 4) for r, c in shapes]
    w_d = [w.to(dev) for w in ws_full]
    g_d = [g.to(dev) for g in gs_full]
    m_d = [m.to(dev) for m in ms_full]
    views = lambda ts: [t[:, :c] for t, (r, c) in zip(ts, shapes)]  # noqa: E731
    u_d = [torch.empty(s, device=dev) for s in shapes]
    mb.muon_step_batched(views(w_d), views(g_d), views(m_d), lr=lr, beta=0.95, nesterov=nesterov,
                         ns_coeffs=MUON, ns_steps=5, precision=prec, updates_out=u_d)
    torch.cuda.synchronize()
    for i, (r, c) in enumerate(shapes):
        check_step(ws_full[i][:, :c].numpy(), to_np(gs_full[i][:, :c]), ms_full[i][:, :c].numpy(),
                   to_np(w_d[i][:, :c]), to_np(m_d[i][:, :c]), to_np(u_d[i]), lr=lr, beta=0.95,
                   nesterov=nesterov, coeffs=MUON, steps=5, tol=PREC_TOL[prec], param_bf16=False)
        # the padding columns beyond cols are untouched
        assert torch.equal(w_d[i][:, c:].cpu(), ws_full[i][:, c:])
        assert torch.equal(m_d[i][:, c:].cpu(), ms_full[i][:, c:])


def test_single256_f32():
    """One 256x256 float32 matrix, W, G, M iid N(0,1) from seed 0, cubic, 5 steps."""
    _announce("workload single256_f32")
    wl = wlm.workload("single256_f32")
    w, m = wlm.initial_state(wl, 0)
    g = wlm.gradient(wl, 0)
    lr = f32(wl.lr)
    w1, m1, o1 = run_step([w], [g], [m], lr=lr, beta=wl.beta, nesterov=wl.nesterov, coeffs=wl.coeffs,
                          steps=wl.ns_steps, precision=mb.NS_F32)
    err, _ = check_step(w.numpy(), g.numpy(), m.numpy(), w1[0], m1[0], o1[0], lr=lr, beta=wl.beta,
                        nesterov=wl.nesterov, coeffs=wl.coeffs, steps=wl.ns_steps, tol=TOL_F32,
                        param_bf16=False)
    print(f"single256_f32 rel-F {err:.3e}")


def test_gpt2s_three_steps():
    """12 x 768^2 bf16, G ~ N(0, 1e-3^2), M0 = 0, three consecutive steps."""
    _announce("workload gpt2s_attn768_bf16")
    wl = wlm.workload("gpt2s_attn768_bf16")
    dev = "cuda"
    n = len(wl.specs)
    st = [wlm.initial_state(wl, i) for i in range(n)]
    w_d = [s[0].to(dev) for s in st]
    m_d = [s[1].to(dev) for s in st]
    u_d = [torch.empty((sp.rows, sp.cols), device=dev) for sp in wl.specs]
    lr = f32(wl.lr)
    for step in range(wl.n_steps):
        g_d = [wlm.gradient(wl, i, step).to(dev) for i in range(n)]
        w0 = [to_np(w) for w in w_d]
        m0 = [to_np(m) for m in m_d]
        mb.muon_step_batched(w_d, g_d, m_d, lr=lr, beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs,
                             ns_steps=wl.ns_steps, precision=mb.NS_BF16, updates_out=u_d)
        torch.cuda.synchronize()
        errs = []
        for i in range(n):
            err, _ = check_step(w0[i], to_np(g_d[i]), m0[i], to_np(w_d[i]), to_np(m_d[i]), to_np(u_d[i]),
                                lr=lr, beta=wl.beta, nesterov=wl.nesterov, coeffs=wl.coeffs,
                                steps=wl.ns_steps, tol=TOL_BF16, param_bf16=True)
            errs.append(err)
        print(f"gpt2s step {step}: max rel-F {max(errs):.3e}")


@pytest.mark.parametrize("prec", [mb.NS_F32, mb.NS_BF16X3, mb.NS_BF16])
def test_ns_only(prec):
    _announce(f"ns only prec={prec}")
    shapes = [(96, 96), (50, 300), (300, 50), (3, 7)]
    gen = torch.Generator().manual_seed(3)
    xs = [torch.randn(s, generator=gen) for s in shapes]
    xs = [x.to(torch.bfloat16) if i % 2 else x for i, x in enumerate(xs)]
    x_d = [x.cuda() for x in xs]
    y_d = [torch.empty(s, device="cuda") for s in shapes]
    mb.muon_ns_batched(x_d, y_d, ns_coeffs=MUON, ns_steps=5, precision=prec)
    torch.cuda.synchronize()
    for x, y in zip(xs, y_d):
        ref = orc.orthogonalise(to_np(x), MUON, 5)
        assert orc.rel_frobenius(to_np(y), ref) <= PREC_TOL[prec]


def test_polar_limit_on_gpu():
    """Many cubic steps on the float32 path reach the SVD polar factor."""
    _announce("polar limit f32")
    gen = torch.Generator().manual_seed(4)
    x = torch.randn(200, 120, generator=gen)
    y = torch.empty(200, 120, device="cuda")
    mb.muon_ns_batched([x.cuda()], [y], ns_coeffs=CUBIC, ns_steps=60, precision=mb.NS_F32)
    torch.cuda.synchronize()
    assert np.max(np.abs(to_np(y) - orc.polar_factor(x.numpy()))) < 1e-4


def test_frobenius_norms():
    _announce("norms")
    shapes = [(1, 1), (64, 64), (65, 130), (1000, 3), (700, 1500)]
    gen = torch.Generator().manual_seed(6)
    xs = [torch.randn(s, generator=gen) * (i + 1) for i, s in enumerate(shapes)]
    xs[1] = xs[1].to(torch.bfloat16)
    out = torch.empty(len(xs), device="cuda")
    mb.muon_frobenius_norms([x.cuda() for x in xs], out)
    torch.cuda.synchronize()
    for x, v in zip(xs, out.cpu().tolist()):
        ref = orc.frobenius_norm(to_np(x))
        assert abs(v - ref) <= 2e-6 * ref


def test_zero_gradient_and_zero_steps():
    _announce("zero gradient")
    shapes = [(40, 70), (70, 40)]
    ws = [torch.randn(s).to(torch.bfloat16) for s in shapes]
    gs = [torch.zeros(s, dtype=torch.bfloat16) for s in shapes]
    ms = [torch.zeros(s) for s in shapes]
    for steps in (0, 5):
        w1, m1, o1 = run_step(ws, gs, ms, lr=0.5, beta=0.95, nesterov=1, coeffs=MUON, steps=steps,
                              precision=mb.NS_BF16)
        for i in range(2):
            assert np.all(o1[i] == 0) and np.all(m1[i] == 0)
            assert np.array_equal(bits(w1[i]), bits(to_np(ws[i])))


def test_deterministic_and_order_independent():
    _announce("determinism")
    shapes = [(300, 200), (128, 640), (640, 128), (77, 77)]
    ws, gs, ms = _inputs(shapes, 21, torch.bfloat16, torch.bfloat16)
    kw = dict(lr=f32(0.02), beta=0.95, nesterov=1, coeffs=MUON, steps=5, precision=mb.NS_BF16)
    a = run_step(ws, gs, ms, **kw)
    b = run_step(ws, gs, ms, **kw)
    rev = run_step(ws[::-1], gs[::-1], ms[::-1], **kw)
    for k in range(3):
        for i in range(len(shapes)):
            assert np.array_equal(bits(a[k][i]), bits(b[k][i]))
            assert np.array_equal(bits(a[k][i]), bits(rev[k][len(shapes) - 1 - i]))


def test_errors_leave_state_untouched():
    _announce("error path on device")
    w = torch.randn(32, 48, device="cuda").to(torch.bfloat16)
    g = torch.randn(32, 48, device="cuda").to(torch.bfloat16)
    m = torch.randn(32, 48, device="cuda")
    w0, m0 = w.clone(), m.clone()
    with pytest.raises(mb.MuonError) as ei:
        mb.muon_step_batched([w], [g], [m], lr=0.02, beta=1.5, nesterov=1, ns_coeffs=MUON, ns_steps=5)
    assert ei.value.status == mb.MUON_ERR_INVALID_ARGUMENT
    with pytest.raises(mb.MuonError) as ei:
        mb.muon_step_batched([w], [w], [m], lr=0.02, beta=0.5, nesterov=1, ns_coeffs=MUON, ns_steps=5)
    assert ei.value.status == mb.MUON_ERR_ALIAS
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and torch.equal(m, m0)
