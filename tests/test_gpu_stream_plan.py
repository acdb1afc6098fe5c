"""Streaming the Muon step into backward (a stream plan): each group's step is
submitted behind the event that marks its gradients complete.

A synthetic producer stream stands in for backward: it writes the gradients
layer by layer, last layer first, each layer after a spin kernel that keeps
the producer busy while leaving the compute units free, and records one
event per layer.  The optimizer stream submits each layer's step behind its
event.  The results must be bit-identical to one muon_step_batched_v2 call
over every matrix, and the streamed step must overlap the producer.
"""
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


def _spin_cycles_per_ms():
    """Cycles of torch.cuda._sleep per millisecond on this GPU."""
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / a.elapsed_time(b)


def _concurrent_pair(cyc):
    """A producer stream and an optimizer stream that run concurrently.  HIP
    maps streams onto a few hardware queues per process, and two streams that
    share one run in submission order; try candidates until a small kernel on
    one finishes while the other spins."""
    producer = torch.cuda.Stream()
    x = torch.ones(1024, device="cuda")
    for _ in range(8):
        cand = torch.cuda.Stream()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(producer)
        with torch.cuda.stream(producer):
            torch.cuda._sleep(int(20 * cyc))
        with torch.cuda.stream(cand):
            x.add_(1.0)
        t1.record(cand)
        torch.cuda.synchronize()
        if t0.elapsed_time(t1) < 10.0:
            return producer, cand
    return None, None


def _stack(layers, seed_offset=0):
    wl = wlm.workload("d24_bf16", layers=layers)
    n = len(wl.specs)
    st = [wlm.initial_state(wl, i, device="cuda") for i in range(n)]
    w = [s[0] for s in st]
    m = [s[1] for s in st]
    g_src = [wlm.gradient(wl, i, 0, device="cuda") for i in range(n)]
    return wl, w, m, g_src


def _produce(g, g_src, layer_of, order, events, stream, spin):
    """On `stream`: for each layer in `order`, spin, write its gradients, record its event."""
    with torch.cuda.stream(stream):
        for layer in order:
            if spin:
                torch.cuda._sleep(spin)
            for i, lay in enumerate(layer_of):
                if lay == layer:
                    g[i].copy_(g_src[i])
            events[layer].record(stream)


def test_stream_plan_equals_one_call():
    _announce("stream plan, 4 d24 layers, groups = layers, behind a producer stream")
    layers = 4
    wl, w, m, g_src = _stack(layers)
    n = len(wl.specs)
    layer_of = [i // 6 for i in range(n)]
    lr_pm = [f32(0.02 * (1 + (i % 3) / 4)) for i in range(n)]
    hp = dict(lr=f32(wl.lr), beta=wl.beta, nesterov=1, ns_coeffs=wl.coeffs, ns_steps=wl.ns_steps,
              weight_decay=0.01, lr_per_matrix=lr_pm)
    w0 = [t.clone() for t in w]
    m0 = [t.clone() for t in m]
    # reference: one call over every matrix
    g_ref = [t.clone() for t in g_src]
    o_ref = [torch.empty(t.shape, device="cuda") for t in g_src]
    mb.muon_step_batched_v2(w, g_ref, m, updates_out=o_ref, **hp)
    torch.cuda.synchronize()
    ref = ([_bits(t) for t in w], [_bits(t) for t in m], [_bits(t) for t in o_ref])
    # streamed: the optimizer reads gradients the producer is still writing
    for d, s in zip(w + m, w0 + m0):
        d.copy_(s)
    g = [torch.zeros_like(t) for t in g_src]
    o = [torch.full(t.shape, float("nan"), device="cuda") for t in g_src]
    plan = mb.StreamPlan(w, g, m, layer_of, layers, updates_out=o)
    cyc = _spin_cycles_per_ms()
    torch.cuda.synchronize()
    producer, opt = torch.cuda.Stream(), torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(layers)]
    order = list(reversed(range(layers)))
    _produce(g, g_src, layer_of, order, events, producer, int(2 * cyc))
    for layer in order:
        plan.submit(layer, events[layer], stream=opt, **hp)
    torch.cuda.synchronize()
    got = ([_bits(t) for t in w], [_bits(t) for t in m], [_bits(t) for t in o])
    for what, a, b in zip(("W", "M", "O"), ref, got):
        for i, (x, y) in enumerate(zip(a, b)):
            assert np.array_equal(x, y), f"{what} of matrix {i} differs from the one-call result"
    # a second step through the same plan, groups submitted in another order
    ref2_w = [t.clone() for t in w]
    ref2_m = [t.clone() for t in m]
    mb.muon_step_batched_v2(ref2_w, g_ref, ref2_m, **hp)
    for layer in range(layers):
        plan.submit(layer, None, stream=opt, **hp)
    torch.cuda.synchronize()
    for i in range(n):
        assert np.array_equal(_bits(w[i]), _bits(ref2_w[i])) and np.array_equal(_bits(m[i]), _bits(ref2_m[i]))
    plan.close()


def test_stream_plan_overlaps_the_producer():
    _announce("stream plan, d24 (24 layers, 6 groups of 4), overlap with a latency-bound producer")
    layers, per_group = 24, 4
    wl, w, m, g_src = _stack(layers)
    n = len(wl.specs)
    group_of = [(i // 6) // per_group for i in range(n)]
    ngroups = layers // per_group
    hp = dict(lr=f32(wl.lr), beta=wl.beta, nesterov=1, ns_coeffs=wl.coeffs, ns_steps=wl.ns_steps)
    g = [t.clone() for t in g_src]
    plan = mb.StreamPlan(w, g, m, group_of, ngroups)
    args = mb.StepArgs(w, g, m)
    cyc = _spin_cycles_per_ms()
    spin = int(3.0 * cyc)                  # 3 ms of producer time per group
    producer, opt = _concurrent_pair(cyc)
    if producer is None:
        pytest.skip("no two streams of this process run concurrently (they share a hardware queue)")
    order = list(reversed(range(ngroups)))

    def timed(streamed):
        events = [torch.cuda.Event() for _ in range(ngroups)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(producer)
        _produce(g, g_src, group_of, order, events, producer, spin)
        if streamed:
            for grp in order:
                plan.submit(grp, events[grp], stream=opt, **hp)
        else:
            opt.wait_event(events[order[-1]])
            mb.muon_step_batched(args, stream=opt, **hp)
        end.record(opt)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    def producer_only():
        events = [torch.cuda.Event() for _ in range(ngroups)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(producer)
        _produce(g, g_src, group_of, order, events, producer, spin)
        end.record(producer)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    for _ in range(2):                     # warm both paths
        timed(True)
        timed(False)
    t_prod = min(producer_only() for _ in range(3))
    t_seq = min(timed(False) for _ in range(3))
    t_stream = min(timed(True) for _ in range(3))
    print(f"producer {t_prod:.2f} ms; producer then one call {t_seq:.2f} ms; streamed {t_stream:.2f} ms "
          f"(optimizer hidden: {(t_seq - t_stream):.2f} ms)")
    assert t_stream < t_seq - 0.25 * t_prod, "the streamed step did not overlap the producer"
    plan.close()


def test_stream_plan_mixed_formats_and_ragged_shapes():
    """Groups that mix binary32, split-bf16 and bf16 matrices of ragged shapes,
    one group empty: every matrix keeps the working format the whole set
    gives it (a group alone would get smaller tiles), so the result is
    bit-identical to one call, whatever the order of the submits."""
    _announce("stream plan over mixed formats and ragged shapes")
    spec = [((700, 1100), mb.NS_BF16), ((1100, 700), mb.NS_BF16), ((769, 769), mb.NS_F32),
            ((300, 520), mb.NS_BF16X3), ((64, 64), mb.NS_BF16), ((1, 300), mb.NS_F32),
            ((2049, 257), mb.NS_BF16), ((257, 2049), mb.NS_BF16X3)]
    group_of = [0, 1, 0, 3, 1, 3, 0, 1]            # group 2 is empty
    gen = torch.Generator().manual_seed(31)
    w = [(torch.randn(s, generator=gen) * 0.02).to(torch.float32 if p == mb.NS_F32 else torch.bfloat16).cuda()
         for s, p in spec]
    g = [torch.randn(s, generator=gen).to(torch.bfloat16).cuda() for s, _ in spec]
    m = [torch.randn(s, generator=gen).cuda() for s, _ in spec]
    precs = [p for _, p in spec]
    w0 = [t.clone() for t in w]
    m0 = [t.clone() for t in m]
    hp = dict(lr=f32(0.02), beta=0.95, nesterov=1, ns_coeffs=(3.4445, -4.775, 2.0315), ns_steps=4,
              weight_decay=0.02, scale_per_matrix=[1.0, 1.5, 0.5, 2.0, 1.0, 0.25, 1.0, 3.0])
    o_ref = [torch.empty(s, device="cuda") for s, _ in spec]
    mb.muon_step_batched_v2(w, g, m, precision=precs, updates_out=o_ref, **hp)
    torch.cuda.synchronize()
    ref = [_bits(t) for t in w + m + o_ref]
    for d, s in zip(w + m, w0 + m0):
        d.copy_(s)
    o = [torch.full(s, float("nan"), device="cuda") for s, _ in spec]
    plan = mb.StreamPlan(w, g, m, group_of, 4, precision=precs, updates_out=o)
    for grp in (3, 2, 0, 1):
        plan.submit(grp, None, **hp)
    torch.cuda.synchronize()
    got = [_bits(t) for t in w + m + o]
    for i, (a, b) in enumerate(zip(ref, got)):
        assert np.array_equal(a, b), f"tensor {i} differs from the one-call result"
    plan.close()
