"""The allocation-free entry point (muon_step_batched_noalloc) through the C
ABI against muon_step_batched_ex on the same inputs: W, M and the exported
O bit for bit, on calls in a row whose second input is smaller than the
first (the scratch array keeps the last call's contents), and a stack too
large for the scratch array refused with nothing changed."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from muon_newton_schulz_02_amd import binding as mb

from gpu_helpers import MUON, f32

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(shapes, seed):
    gen = torch.Generator().manual_seed(seed)
    ws, gs, ms, precs = [], [], [], []
    for rows, cols, prec in shapes:
        pdt = torch.float32 if prec == mb.NS_F32 else torch.bfloat16
        ws.append((torch.randn(rows, cols, generator=gen) * 0.02).to(pdt))
        gs.append(torch.randn(rows, cols, generator=gen).to(torch.bfloat16))
        ms.append(torch.randn(rows, cols, generator=gen))
        precs.append(prec)
    return ws, gs, ms, precs


def _call(entry, ws, gs, ms, us, precs, steps=5):
    """One call of `entry` (a C function taking muon_step_batched_ex's arguments)."""
    args = mb.StepArgs(ws, gs, ms, precs, us)
    fn = getattr(mb.lib(), entry)
    return fn(args.params, args.grads, args.momenta, args.descs, args.count, f32(0.02), 0.95, 1,
              mb.NsCoeffs(*MUON), steps, mb.SCALE_NONE, args.updates,
              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _compare(shapes, seed):
    ws, gs, ms, precs = _inputs(shapes, seed)
    dev = [[t.cuda() for t in x] for x in (ws, gs, ms)]
    ref = [[t.clone() for t in x] for x in dev]
    us_ref = [torch.full(g.shape, float("nan"), device="cuda") for g in gs]
    us = [torch.full(g.shape, float("nan"), device="cuda") for g in gs]
    assert _call("muon_step_batched_ex", ref[0], ref[1], ref[2], us_ref, precs) == mb.MUON_OK, mb.muon_last_error()
    assert _call("muon_step_batched_noalloc", dev[0], dev[1], dev[2], us, precs) == mb.MUON_OK, mb.muon_last_error()
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        for what, a, b in (("W", dev[0][i], ref[0][i]), ("M", dev[2][i], ref[2][i]), ("O", us[i], us_ref[i])):
            assert np.array_equal(_bits(a), _bits(b)), f"{shapes[i]}: {what} differs from muon_step_batched_ex"
    assert all(torch.isfinite(u).all() for u in us)


def test_noalloc_equals_step_batched_ex_on_calls_in_a_row():
    big = [(768, 768, mb.NS_BF16)] * 12                    # the largest stack here that fits the scratch array
    small = [(300, 520, mb.NS_BF16), (520, 300, mb.NS_BF16), (64, 64, mb.NS_F32), (1, 300, mb.NS_BF16),
             (257, 129, mb.NS_BF16X3)]
    _announce("no-allocation entry point: twelve 768 x 768 bf16")
    _compare(big, 1)
    _announce("no-allocation entry point: a smaller ragged, mixed-format stack next")
    _compare(small, 2)
    _announce("no-allocation entry point: the large stack again")
    _compare(big, 3)


def test_noalloc_refuses_a_stack_too_large_for_its_scratch():
    _announce("no-allocation entry point: one d24 layer is refused")
    shapes = [(1536, 1536, mb.NS_BF16)] * 4 + [(1536, 6144, mb.NS_BF16), (6144, 1536, mb.NS_BF16)]
    ws, gs, ms, precs = _inputs(shapes, 4)
    dev = [[t.cuda() for t in x] for x in (ws, gs, ms)]
    before = [_bits(t) for t in dev[0] + dev[2]]
    st = _call("muon_step_batched_noalloc", dev[0], dev[1], dev[2], None, precs)
    assert st == mb.MUON_ERR_UNSUPPORTED and "scratch" in mb.muon_last_error()
    torch.cuda.synchronize()
    assert all(np.array_equal(a, _bits(t)) for a, t in zip(before, dev[0] + dev[2]))
