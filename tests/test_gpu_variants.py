"""The update variants of muon_step_batched_v2 on the GPU against the oracle:
Newton-Schulz schedules, EMA momentum, decoupled weight decay, per-matrix
learning rates and scales.  Momentum is compared bit for bit, O within the
precision's gate, and W bit for bit given the exported O."""
import sys

import numpy as np
import pytest
import torch

import oracle as orc
from muon_newton_schulz_02_amd import binding as mb

from gpu_helpers import MUON, PREC_TOL, bits, f32, to_np

pytestmark = pytest.mark.gpu

SHAPES = [(130, 257), (520, 300), (64, 64), (769, 300)]
SCHEDULE5 = [(4.0848, -6.8946, 2.9270), (3.9505, -6.3029, 2.6377), (3.7418, -5.5913, 2.3037),
             (2.8769, -3.1427, 1.2046), (1.5, -0.5, 0.0)]


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(seed, pdt):
    gen = torch.Generator().manual_seed(seed)
    ws = [(torch.randn(s, generator=gen) * 0.02).to(pdt) for s in SHAPES]
    gs = [torch.randn(s, generator=gen).to(torch.bfloat16) for s in SHAPES]
    ms = [torch.randn(s, generator=gen) for s in SHAPES]
    return ws, gs, ms


def _run_v2(ws, gs, ms, *, precision, steps, **kw):
    w_d = [w.cuda() for w in ws]
    g_d = [g.cuda() for g in gs]
    m_d = [m.cuda() for m in ms]
    u_d = [torch.full(tuple(g.shape), float("nan"), dtype=torch.float32, device="cuda") for g in gs]
    mb.muon_step_batched_v2(w_d, g_d, m_d, lr=kw.pop("lr"), beta=kw.pop("beta"), nesterov=kw.pop("nesterov"),
                            ns_coeffs=MUON, ns_steps=steps, precision=precision, updates_out=u_d, **kw)
    torch.cuda.synchronize()
    return [to_np(w) for w in w_d], [to_np(m) for m in m_d], [to_np(u) for u in u_d]


@pytest.mark.parametrize("prec", [mb.NS_F32, mb.NS_BF16])
@pytest.mark.parametrize("kind", [mb.MOMENTUM_HEAVY_BALL, mb.MOMENTUM_EMA])
@pytest.mark.parametrize("nesterov", [0, 1])
def test_schedule_and_momentum_kind(prec, kind, nesterov):
    _announce(f"schedule prec={prec} kind={kind} nesterov={nesterov}")
    pdt = torch.bfloat16 if prec == mb.NS_BF16 else torch.float32
    ws, gs, ms = _inputs(41 + 2 * kind + nesterov, pdt)
    lr = f32(0.02)
    w1, m1, o1 = _run_v2(ws, gs, ms, precision=prec, steps=len(SCHEDULE5), lr=lr, beta=0.95, nesterov=nesterov,
                         ns_schedule=SCHEDULE5, momentum_kind=kind)
    for i in range(len(SHAPES)):
        w0, g0, m0 = to_np(ws[i]), to_np(gs[i]), to_np(ms[i])
        ref = orc.muon_step(w0, g0, m0, lr=lr, beta=0.95, nesterov=bool(nesterov), coeffs=SCHEDULE5,
                            steps=len(SCHEDULE5), param_bf16=pdt == torch.bfloat16, momentum_kind=kind)
        assert np.array_equal(bits(m1[i]), bits(ref.m)), f"matrix {i}: momentum"
        err = orc.rel_frobenius(o1[i], ref.o)
        print(f"  {SHAPES[i]}: rel-F {err:.2e}")
        assert err <= PREC_TOL[prec]
        w_exp = orc.write_back(w0, o1[i], lr, 1.0, pdt == torch.bfloat16)
        assert np.array_equal(bits(w1[i]), bits(w_exp)), f"matrix {i}: write-back"


@pytest.mark.parametrize("pdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("steps", [5, 0])
def test_weight_decay_and_per_matrix_rates(pdt, steps):
    _announce(f"weight decay pdt={pdt} steps={steps}")
    ws, gs, ms = _inputs(53 + steps, pdt)
    lrs = [0.02, 0.0, 0.05, 0.013]
    scales = [1.0, 2.5, 0.2 * np.sqrt(520.0), 1.7]
    wd = 0.1
    w1, m1, o1 = _run_v2(ws, gs, ms, precision=mb.NS_BF16, steps=steps, lr=0.02, beta=0.9, nesterov=1,
                         weight_decay=wd, lr_per_matrix=lrs, scale_per_matrix=scales, scale_rule=mb.SCALE_SQRT_ASPECT)
    for i in range(len(SHAPES)):
        w0, g0, m0 = to_np(ws[i]), to_np(gs[i]), to_np(ms[i])
        ref = orc.muon_step(w0, g0, m0, lr=f32(lrs[i]), beta=0.9, nesterov=True, coeffs=MUON, steps=steps,
                            param_bf16=pdt == torch.bfloat16, weight_decay=f32(wd), scale=f32(scales[i]))
        assert np.array_equal(bits(m1[i]), bits(ref.m)), f"matrix {i}: momentum"
        assert orc.rel_frobenius(o1[i], ref.o) <= PREC_TOL[mb.NS_BF16]
        w_exp = orc.write_back(w0, o1[i], f32(lrs[i]), f32(scales[i]), pdt == torch.bfloat16, f32(wd))
        assert np.array_equal(bits(w1[i]), bits(w_exp)), f"matrix {i}: write-back"


@pytest.mark.parametrize("tile_mode", [mb.TILES_LARGE, mb.TILES_SMALL])
@pytest.mark.parametrize("steps", [0, 1])
def test_few_steps_on_both_bf16_tile_sizes(tile_mode, steps):
    # no Newton-Schulz step (the write-back reads U back from the workspace)
    # and one step, on the tile-major workspace of the 256 x 256 tiles and on
    # the row-major one of the 128 x 128 tiles
    _announce(f"bf16 steps={steps} tile_mode={tile_mode}")
    ws, gs, ms = _inputs(83 + steps + 2 * tile_mode, torch.bfloat16)
    lr = f32(0.02)
    w1, m1, o1 = _run_v2(ws, gs, ms, precision=mb.NS_BF16, steps=steps, lr=lr, beta=0.95, nesterov=1,
                         tile_mode=tile_mode)
    for i in range(len(SHAPES)):
        w0, g0, m0 = to_np(ws[i]), to_np(gs[i]), to_np(ms[i])
        ref = orc.muon_step(w0, g0, m0, lr=lr, beta=0.95, nesterov=True, coeffs=MUON, steps=steps, param_bf16=True)
        assert np.array_equal(bits(m1[i]), bits(ref.m)), f"matrix {i}: momentum"
        err = orc.rel_frobenius(o1[i], ref.o)
        print(f"  {SHAPES[i]}: rel-F {err:.2e}")
        assert err <= PREC_TOL[mb.NS_BF16]
        assert np.array_equal(bits(w1[i]), bits(orc.write_back(w0, o1[i], lr, 1.0, True))), f"matrix {i}: write-back"


def test_default_options_match_plain_step():
    _announce("v2 with default options equals the plain step")
    ws, gs, ms = _inputs(61, torch.bfloat16)
    a = _run_v2(ws, gs, ms, precision=mb.NS_BF16, steps=5, lr=0.02, beta=0.95, nesterov=1)
    w_d = [w.cuda() for w in ws]
    m_d = [m.cuda() for m in ms]
    mb.muon_step_batched(w_d, [g.cuda() for g in gs], m_d, lr=0.02, beta=0.95, nesterov=1, ns_coeffs=MUON,
                         ns_steps=5, precision=mb.NS_BF16)
    torch.cuda.synchronize()
    for i in range(len(SHAPES)):
        assert np.array_equal(bits(a[0][i]), bits(to_np(w_d[i])))
        assert np.array_equal(bits(a[1][i]), bits(to_np(m_d[i])))


@pytest.mark.parametrize("tile_mode", [mb.TILES_LARGE, mb.TILES_SMALL])
@pytest.mark.parametrize("launch_mode", [mb.LAUNCH_PHASE_GRIDS, mb.LAUNCH_CHAIN])
def test_f32_tile_sizes(tile_mode, launch_mode):
    # binary32 on 128 x 128 and 64 x 64 tiles, per-phase grids and the
    # persistent chain: O within the fp32 gate, W bit-exact given O
    _announce(f"fp32 tiles mode={tile_mode} launch={launch_mode}")
    ws, gs, ms = _inputs(71 + tile_mode, torch.float32)
    lr = f32(0.02)
    w1, m1, o1 = _run_v2(ws, gs, ms, precision=mb.NS_F32, steps=5, lr=lr, beta=0.95, nesterov=1,
                         tile_mode=tile_mode, launch_mode=launch_mode)
    for i in range(len(SHAPES)):
        w0, g0, m0 = to_np(ws[i]), to_np(gs[i]), to_np(ms[i])
        ref = orc.muon_step(w0, g0, m0, lr=lr, beta=0.95, nesterov=True, coeffs=MUON, steps=5, param_bf16=False)
        assert np.array_equal(bits(m1[i]), bits(ref.m))
        err = orc.rel_frobenius(o1[i], ref.o)
        print(f"  {SHAPES[i]}: rel-F {err:.2e}")
        assert err <= PREC_TOL[mb.NS_F32]
        assert np.array_equal(bits(w1[i]), bits(orc.write_back(w0, o1[i], lr, 1.0, False)))


@pytest.mark.parametrize("tile_mode", [mb.TILES_LARGE, mb.TILES_SMALL])
@pytest.mark.parametrize("launch_mode", [mb.LAUNCH_PHASE_GRIDS, mb.LAUNCH_CHAIN])
def test_split_bf16_tile_sizes(tile_mode, launch_mode):
    # split-bf16 on the pipelined 256 x 256 tiles (three bf16 products per
    # product) and on the one-stage 128 x 128 tiles, per-phase grids and the
    # persistent chain, with a schedule whose last step has c = 0 (GRAM then
    # stores B = b A and POLY is skipped): O within the split-bf16 gate, W
    # bit-exact given O
    _announce(f"split-bf16 tiles mode={tile_mode} launch={launch_mode}")
    ws, gs, ms = _inputs(91 + tile_mode, torch.float32)
    lr = f32(0.02)
    w1, m1, o1 = _run_v2(ws, gs, ms, precision=mb.NS_BF16X3, steps=len(SCHEDULE5), lr=lr, beta=0.95, nesterov=1,
                         ns_schedule=SCHEDULE5, tile_mode=tile_mode, launch_mode=launch_mode)
    for i in range(len(SHAPES)):
        w0, g0, m0 = to_np(ws[i]), to_np(gs[i]), to_np(ms[i])
        ref = orc.muon_step(w0, g0, m0, lr=lr, beta=0.95, nesterov=True, coeffs=SCHEDULE5, steps=len(SCHEDULE5),
                            param_bf16=False)
        assert np.array_equal(bits(m1[i]), bits(ref.m))
        err = orc.rel_frobenius(o1[i], ref.o)
        print(f"  {SHAPES[i]}: rel-F {err:.2e}")
        assert err <= PREC_TOL[mb.NS_BF16X3]
        assert np.array_equal(bits(w1[i]), bits(orc.write_back(w0, o1[i], lr, 1.0, False)))


@pytest.mark.parametrize("tile_mode", [mb.TILES_LARGE, mb.TILES_SMALL])
@pytest.mark.parametrize("launch_mode", [mb.LAUNCH_PHASE_GRIDS, mb.LAUNCH_CHAIN])
def test_bf16_tile_sizes(tile_mode, launch_mode):
    # 256 x 256 (pipelined) and 128 x 128 (one-stage) bf16 tiles, per-phase
    # grids and the persistent chain: O within the bf16 gate, W bit-exact given O
    _announce(f"bf16 tiles mode={tile_mode} launch={launch_mode}")
    ws, gs, ms = _inputs(67 + tile_mode, torch.bfloat16)
    lr = f32(0.02)
    w1, m1, o1 = _run_v2(ws, gs, ms, precision=mb.NS_BF16, steps=5, lr=lr, beta=0.95, nesterov=1,
                         tile_mode=tile_mode, launch_mode=launch_mode)
    for i in range(len(SHAPES)):
        w0, g0, m0 = to_np(ws[i]), to_np(gs[i]), to_np(ms[i])
        ref = orc.muon_step(w0, g0, m0, lr=lr, beta=0.95, nesterov=True, coeffs=MUON, steps=5, param_bf16=True)
        assert np.array_equal(bits(m1[i]), bits(ref.m))
        err = orc.rel_frobenius(o1[i], ref.o)
        print(f"  {SHAPES[i]}: rel-F {err:.2e}")
        assert err <= PREC_TOL[mb.NS_BF16]
        assert np.array_equal(bits(w1[i]), bits(orc.write_back(w0, o1[i], lr, 1.0, True)))
