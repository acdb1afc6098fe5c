"""The persistent Newton-Schulz chain (one launch for every phase of every
step, per-XCD work queues, per-(matrix, phase) completion counts) against the
per-phase grids: the same tiles in the same arithmetic, so W, M and the
exported update must agree bit for bit; and against the oracle directly."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle as orc
from muon_newton_schulz_02_amd import binding as mb
from muon_newton_schulz_02_amd import workloads as wlm

from gpu_helpers import CUBIC, MUON, PREC_TOL, bits, f32, to_np

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(shapes, seed, pdt=torch.bfloat16):
    gen = torch.Generator().manual_seed(seed)
    ws = [(torch.randn(s, generator=gen) * 0.02).to(pdt) for s in shapes]
    gs = [torch.randn(s, generator=gen).to(torch.bfloat16) for s in shapes]
    ms = [torch.randn(s, generator=gen) for s in shapes]
    return ws, gs, ms


def _run(ws, gs, ms, mode, *, precision, steps, schedule=None, coeffs=MUON, **kw):
    w_d = [w.cuda() for w in ws]
    g_d = [g.cuda() for g in gs]
    m_d = [m.cuda() for m in ms]
    u_d = [torch.full(tuple(g.shape), float("nan"), dtype=torch.float32, device="cuda") for g in gs]
    mb.muon_step_batched_v2(w_d, g_d, m_d, lr=f32(0.02), beta=0.95, nesterov=1, ns_coeffs=coeffs, ns_steps=steps,
                            precision=precision, updates_out=u_d, ns_schedule=schedule, launch_mode=mode, **kw)
    torch.cuda.synchronize()
    return [to_np(t) for t in w_d], [to_np(t) for t in m_d], [to_np(t) for t in u_d]


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(bits(x), bits(y)), f"{what} {i} differs between the chain and the per-phase grids"


MIXED = [(700, 1100), (1100, 700), (769, 769), (300, 520), (64, 64), (1, 300)]


@pytest.mark.parametrize("prec,steps,tiles", [(mb.NS_BF16, 5, mb.TILES_AUTO), (mb.NS_BF16, 1, mb.TILES_AUTO),
                                               (mb.NS_BF16X3, 3, mb.TILES_AUTO), (mb.NS_BF16X3, 3, mb.TILES_LARGE),
                                               (mb.NS_F32, 5, mb.TILES_AUTO)])
def test_chain_equals_phase_grids(prec, steps, tiles):
    _announce(f"chain vs grids prec={prec} steps={steps} tiles={tiles}")
    shapes = MIXED if prec == mb.NS_BF16 else MIXED[2:]
    pdt = torch.float32 if prec == mb.NS_F32 else torch.bfloat16
    ws, gs, ms = _inputs(shapes, 71 + steps, pdt)
    a = _run(ws, gs, ms, mb.LAUNCH_PHASE_GRIDS, precision=prec, steps=steps, tile_mode=tiles)
    b = _run(ws, gs, ms, mb.LAUNCH_CHAIN, precision=prec, steps=steps, tile_mode=tiles)
    _same(a[0], b[0], "W")
    _same(a[1], b[1], "M")
    _same(a[2], b[2], "O")


def test_chain_schedule_with_c_zero_steps_and_options():
    # cubic steps (c = 0: POLY skipped, GRAM stores B = b A) between quintic
    # ones; decay and per-matrix rates in the write-back
    _announce("chain schedule with c = 0 steps")
    shapes = MIXED
    ws, gs, ms = _inputs(shapes, 83)
    sched = [MUON, CUBIC, MUON, CUBIC]
    kw = dict(weight_decay=0.05, lr_per_matrix=[0.02, 0.01, 0.03, 0.0, 0.02, 0.05])
    a = _run(ws, gs, ms, mb.LAUNCH_PHASE_GRIDS, precision=mb.NS_BF16, steps=4, schedule=sched, **kw)
    b = _run(ws, gs, ms, mb.LAUNCH_CHAIN, precision=mb.NS_BF16, steps=4, schedule=sched, **kw)
    _same(a[0], b[0], "W")
    _same(a[2], b[2], "O")
    for i in range(len(shapes)):
        ref = orc.muon_step(to_np(ws[i]), to_np(gs[i]), to_np(ms[i]), lr=f32(0.02), beta=0.95, nesterov=True,
                            coeffs=sched, steps=4, param_bf16=True)
        assert orc.rel_frobenius(b[2][i], ref.o) <= PREC_TOL[mb.NS_BF16]


def test_chain_rebuilds_when_steps_change_and_reuses_plans():
    _announce("chain plan reuse")
    shapes = MIXED[:4]
    ws, gs, ms = _inputs(shapes, 89)
    w_d = [w.cuda() for w in ws]
    g_d = [g.cuda() for g in gs]
    m_d = [m.cuda() for m in ms]
    args = mb.StepArgs(w_d, g_d, m_d)
    for steps in (5, 3, 5, 2):
        mb.muon_step_batched_v2(args, lr=0.02, beta=0.95, nesterov=1, ns_coeffs=MUON, ns_steps=steps,
                                launch_mode=mb.LAUNCH_CHAIN)
    torch.cuda.synchronize()
    w_c = [to_np(w) for w in w_d]
    w_d = [w.cuda() for w in ws]
    m_d = [m.cuda() for m in ms]
    args = mb.StepArgs(w_d, g_d, m_d)
    for steps in (5, 3, 5, 2):
        mb.muon_step_batched_v2(args, lr=0.02, beta=0.95, nesterov=1, ns_coeffs=MUON, ns_steps=steps,
                                launch_mode=mb.LAUNCH_PHASE_GRIDS)
    torch.cuda.synchronize()
    _same([to_np(w) for w in w_d], w_c, "W after four steps")


def test_chain_and_auto_timing_classes():
    # the chain is one launch of its own class; AUTO keeps the per-phase grids
    _announce("launch classes")
    shapes = [(768, 768)] * 4
    ws, gs, ms = _inputs(shapes, 97)
    w_d = [w.cuda() for w in ws]
    g_d = [g.cuda() for g in gs]
    m_d = [m.cuda() for m in ms]
    mb.muon_timing_enable(True)
    mb.muon_timing_read()
    mb.muon_step_batched_v2(w_d, g_d, m_d, lr=0.02, beta=0.95, nesterov=1, ns_coeffs=MUON, ns_steps=5,
                            launch_mode=mb.LAUNCH_CHAIN)
    torch.cuda.synchronize()
    kern = mb.muon_timing_read()
    assert kern["chain"][1] == 1 and kern["gram"][1] == 0
    mb.muon_step_batched(w_d, g_d, m_d, lr=0.02, beta=0.95, nesterov=1, ns_coeffs=MUON, ns_steps=5)
    torch.cuda.synchronize()
    kern = mb.muon_timing_read()
    mb.muon_timing_enable(False)
    assert kern["chain"][1] == 0 and kern["gram"][1] == 5


def test_chain_d24_share_equals_phase_grids():
    # three d24 layers (one GPU's share of eight) at full size
    _announce("chain d24 share")
    wl = wlm.workload("d24_bf16", layers=3)
    ws, gs, ms = [], [], []
    for i in range(len(wl.specs)):
        w, m = wlm.initial_state(wl, i, device="cuda")
        ws.append(w)
        ms.append(m)
        gs.append(wlm.gradient(wl, i, 0, device="cuda"))
    outs = []
    for mode in (mb.LAUNCH_PHASE_GRIDS, mb.LAUNCH_CHAIN):
        w_d = [w.clone() for w in ws]
        m_d = [m.clone() for m in ms]
        mb.muon_step_batched_v2(w_d, gs, m_d, lr=wl.lr, beta=wl.beta, nesterov=1, ns_coeffs=wl.coeffs,
                                ns_steps=wl.ns_steps, launch_mode=mode)
        torch.cuda.synchronize()
        outs.append([w.view(torch.int16).cpu().numpy() for w in w_d])
    for i, (a, b) in enumerate(zip(*outs)):
        assert np.array_equal(a, b), f"{wl.specs[i].name}: W differs between the chain and the grids"


def test_chain_wait_give_up_is_reported_and_cleared():
    # the host sets the chain's wait limit to zero polls: items that find
    # their inputs incomplete give up and skip, every wait ends, the launch
    # finishes, and the next call on the device reports it once
    _announce("chain give-up path")
    shapes = [(1024, 1024)] * 4
    ws, gs, ms = _inputs(shapes, 101)
    os.environ["MUON_CHAIN_SPIN_LIMIT"] = "0"
    try:
        _run(ws, gs, ms, mb.LAUNCH_CHAIN, precision=mb.NS_BF16, steps=5)
    finally:
        del os.environ["MUON_CHAIN_SPIN_LIMIT"]
    with pytest.raises(mb.MuonError) as ei:
        _run(ws, gs, ms, mb.LAUNCH_CHAIN, precision=mb.NS_BF16, steps=5)
    assert ei.value.status == mb.MUON_ERR_HIP and "gave up" in ei.value.detail
    # the next call reports it with no synchronisation in between: it waits
    # for the earlier chain to end before reading the flag
    w_d, g_d, m_d = ([t.cuda() for t in x] for x in (ws, gs, ms))
    torch.cuda.synchronize()
    kw = dict(lr=f32(0.02), beta=0.95, nesterov=1, ns_coeffs=MUON, ns_steps=5, launch_mode=mb.LAUNCH_CHAIN)
    os.environ["MUON_CHAIN_SPIN_LIMIT"] = "0"
    try:
        mb.muon_step_batched_v2(w_d, g_d, m_d, **kw)
    finally:
        del os.environ["MUON_CHAIN_SPIN_LIMIT"]
    with pytest.raises(mb.MuonError) as ei:
        mb.muon_step_batched_v2(w_d, g_d, m_d, **kw)
    assert ei.value.status == mb.MUON_ERR_HIP and "gave up" in ei.value.detail
    torch.cuda.synchronize()
    # cleared: the next calls run and agree with the per-phase grids
    a = _run(ws, gs, ms, mb.LAUNCH_PHASE_GRIDS, precision=mb.NS_BF16, steps=5)
    b = _run(ws, gs, ms, mb.LAUNCH_CHAIN, precision=mb.NS_BF16, steps=5)
    _same(a[0], b[0], "W")
