"""Failure handling and checkpoint/resume on the GPU.

* The allocation fault hook (MUON_FAULT_ALLOC): a call that needs device
  memory fails with OUT_OF_MEMORY and changes nothing; the next call without
  the hook runs.
* Checkpoint/resume: the optimizer's state is the caller's weights and
  momenta.  Saving them after two steps and restoring them into new tensors,
  with the library's workspace and plans released in between, gives a third
  step bit-identical to the one taken without the interruption.
"""
import io
import os
import sys

import numpy as np
import pytest
import torch

from muon_newton_schulz_02_amd import binding as mb
from muon_newton_schulz_02_amd import workloads as wlm

from gpu_helpers import f32

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def test_allocation_fault_hook():
    _announce("allocation fault hook")
    gen = torch.Generator().manual_seed(21)
    shapes = [(333, 444), (444, 333), (96, 96)]
    w = [(torch.randn(s, generator=gen) * 0.02).to(torch.bfloat16).cuda() for s in shapes]
    g = [torch.randn(s, generator=gen).to(torch.bfloat16).cuda() for s in shapes]
    m = [torch.randn(s, generator=gen).cuda() for s in shapes]
    before = [_bits(t) for t in w + m]
    kw = dict(lr=f32(0.02), beta=0.95, nesterov=1, ns_coeffs=wlm.QUINTIC_MUON, ns_steps=5)
    os.environ["MUON_FAULT_ALLOC"] = "1"
    try:
        with pytest.raises(mb.MuonError) as ei:
            mb.muon_step_batched(w, g, m, **kw)       # new tensors: a new plan must be allocated
        assert ei.value.status == mb.MUON_ERR_OUT_OF_MEMORY
        with pytest.raises(mb.MuonError) as ei:
            mb.StreamPlan(w, g, m, [0, 0, 1], 2)
        assert ei.value.status == mb.MUON_ERR_OUT_OF_MEMORY
    finally:
        del os.environ["MUON_FAULT_ALLOC"]
    torch.cuda.synchronize()
    assert all(np.array_equal(a, _bits(t)) for a, t in zip(before, w + m)), "a failed call changed its inputs"
    mb.muon_step_batched(w, g, m, **kw)
    torch.cuda.synchronize()
    assert not np.array_equal(before[0], _bits(w[0]))


def test_checkpoint_resume_is_bit_identical():
    _announce("checkpoint after two steps, resume into new tensors after releasing the workspace")
    wl = wlm.workload("gpt2s_attn768_bf16")
    n = len(wl.specs)
    st = [wlm.initial_state(wl, i, device="cuda") for i in range(n)]
    w = [s[0] for s in st]
    m = [s[1] for s in st]
    grads = [[wlm.gradient(wl, i, k, device="cuda") for i in range(n)] for k in range(3)]
    kw = dict(lr=f32(wl.lr), beta=wl.beta, nesterov=wl.nesterov, ns_coeffs=wl.coeffs, ns_steps=wl.ns_steps,
              weight_decay=0.01)
    for k in range(2):
        mb.muon_step_batched_v2(w, grads[k], m, **kw)
    torch.cuda.synchronize()
    buf = io.BytesIO()
    torch.save({"w": [t.cpu() for t in w], "m": [t.cpu() for t in m]}, buf)
    mb.muon_step_batched_v2(w, grads[2], m, **kw)
    torch.cuda.synchronize()
    ref = [_bits(t) for t in w + m]
    # resume: a fresh workspace and plans, the state loaded into new tensors
    mb.muon_release_workspace()
    buf.seek(0)
    state = torch.load(buf, weights_only=True)
    w2 = [t.cuda() for t in state["w"]]
    m2 = [t.cuda() for t in state["m"]]
    mb.muon_step_batched_v2(w2, grads[2], m2, **kw)
    torch.cuda.synchronize()
    got = [_bits(t) for t in w2 + m2]
    assert all(np.array_equal(a, b) for a, b in zip(ref, got)), "the resumed step differs"
