"""Pins of the AdamW oracle (oracle/adamw_oracle.py) against facts that do not
come from its code: exact first-step values, a float64 evaluation in another
arrangement within a derived rounding bound, torch.optim.AdamW in float64,
exact scale invariance, closed forms of the decay, and bfloat16 ties.

Which plausible mistake each pin catches:
* no bias correction, or t off by one        first-step sign descent, float64, torch
* eps inside the square root, or dropped     float64 (eps comparable to sqrt(v_hat)), torch
* coupled (L2) decay instead of decoupled    torch, decay closed form
* beta1 and beta2 swapped                    float64, torch
* |g| or g in place of g*g, missing sqrt     scale invariance, first step
* truncating instead of RNE to bfloat16      bfloat16 ties
"""
import math

import numpy as np
import pytest
import torch

import oracle as orc

U24 = 2.0 ** -24


def test_constants_closed_values():
    c1, c2, bc1, bc2 = orc.adamw_constants(0.5, 0.75, 3)
    assert (c1, c2) == (np.float32(0.5), np.float32(0.25))
    assert bc1 == np.float32(0.875) and bc2 == np.float32(1 - 0.75 ** 3)
    # at t = 1 the bias corrections equal 1 - beta
    c1, c2, bc1, bc2 = orc.adamw_constants(0.9, 0.95, 1)
    assert bc1 == c1 and bc2 == c2
    with pytest.raises(ValueError):
        orc.adamw_constants(0.9, 0.95, 0)


def test_first_step_is_sign_descent():
    # From m = v = 0 with eps = 0, the bias-corrected moments are g and g^2,
    # so u = g / |g| exactly.  beta1 = 1/2, beta2 = 15/16 keep every operation
    # exact for gradients of few significant bits; without bias correction u
    # would be 2 sign(g).
    g = np.array([3.0, -0.5, 1.25, -96.0, 0.0078125], np.float32)
    p = np.array([1.0, -2.0, 0.5, 4.0, -0.25], np.float32)
    z = np.zeros_like(g)
    p1, m1, v1 = orc.adamw(p, g, z, z, lr=0.25, beta1=0.5, beta2=0.9375, eps=0.0, weight_decay=0.0, step=1)
    assert np.array_equal(m1, g / 2)
    assert np.array_equal(v1, g * g / 16)
    assert np.array_equal(p1, p - np.float32(0.25) * np.sign(g))


def _float64_adamw(p, g, m, v, lr, beta1, beta2, eps, wd, step):
    """The same update from [KB]/[LH], arranged differently: step size
    lr / bc1 and denominator sqrt(v) / sqrt(bc2) + eps, all in float64."""
    p, g, m, v = (np.asarray(a, np.float64) for a in (p, g, m, v))
    b1, b2 = float(np.float32(beta1)), float(np.float32(beta2))
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    bc1, bc2 = 1 - b1 ** step, 1 - b2 ** step
    denom = np.sqrt(v) / math.sqrt(bc2) + float(np.float32(eps))
    lr = float(np.float32(lr))
    p = p * (1 - lr * float(np.float32(wd))) - (lr / bc1) * m / denom
    return p, m, v


@pytest.mark.parametrize("step", [1, 2, 7, 1000])
def test_matches_float64_within_rounding_bound(step):
    # m0 has the sign of g, so no sum cancels: every operation of the moments
    # and of u has relative error <= 2^-24, u has <= 8 of them (and the binary32
    # constants one each); the final subtraction may cancel, so its bound is
    # taken on |p d| + |lr u|.
    rng = np.random.default_rng(90 + step)
    n = 4096
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (np.abs(rng.standard_normal(n)) * 1e-3 * np.sign(g)).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-4, weight_decay=0.1, step=step)
    p1, m1, v1 = orc.adamw(p, g, m, v, **kw)
    p64, m64, v64 = _float64_adamw(p, g, m, v, kw["lr"], kw["beta1"], kw["beta2"], kw["eps"], kw["weight_decay"], step)
    assert np.all(np.abs(m1 - m64) <= 4 * U24 * np.abs(m64))
    assert np.all(np.abs(v1 - v64) <= 4 * U24 * np.abs(v64))
    lr_u = np.abs(p * (1 - 1e-4) - p64)      # |lr u| to first order
    bound = 16 * U24 * (np.abs(p64) + lr_u)
    assert np.all(np.abs(p1 - p64) <= bound)
    # the comparison sees eps: without it p moves by far more than the bound
    p_noeps, _, _ = _float64_adamw(p, g, m, v, kw["lr"], kw["beta1"], kw["beta2"], 0.0, kw["weight_decay"], step)
    assert np.median(np.abs(p_noeps - p64) / bound) > 100


def test_matches_torch_adamw_float64():
    # torch.optim.AdamW on float64 tensors, 8 steps, with decay; the oracle
    # iterates in binary32.  The accumulated change of p and the moments agree
    # to binary32 accuracy.
    rng = np.random.default_rng(91)
    shape = (33, 65)
    p0 = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal(shape) * 1e-2).astype(np.float32) for _ in range(8)]
    kw = dict(lr=3e-3, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.05)
    t = torch.nn.Parameter(torch.from_numpy(p0.astype(np.float64)))
    opt = torch.optim.AdamW([t], foreach=False, **kw)
    p, m, v = p0, np.zeros(shape, np.float32), np.zeros(shape, np.float32)
    for k, gk in enumerate(grads, start=1):
        t.grad = torch.from_numpy(gk.astype(np.float64))
        opt.step()
        p, m, v = orc.adamw(p, gk, m, v, lr=kw["lr"], beta1=kw["betas"][0], beta2=kw["betas"][1],
                            eps=kw["eps"], weight_decay=kw["weight_decay"], step=k)
    st = opt.state[t]
    d_ref = t.detach().numpy() - p0
    d_or = p.astype(np.float64) - p0
    assert np.linalg.norm(d_or - d_ref) <= 1e-5 * np.linalg.norm(d_ref)
    # the moments, in norm (single entries of m may cancel to near zero)
    for ours, ref in ((m, st["exp_avg"].numpy()), (v, st["exp_avg_sq"].numpy())):
        assert np.linalg.norm(ours - ref) <= 1e-6 * np.linalg.norm(ref)


def test_scale_invariance_exact():
    # eps = 0: multiplying g by 2^k multiplies m by 2^k and v by 4^k exactly,
    # and leaves u, hence p, unchanged bit for bit
    rng = np.random.default_rng(92)
    g = rng.standard_normal(1000).astype(np.float32)
    m = rng.standard_normal(1000).astype(np.float32)
    v = (rng.random(1000) + 0.1).astype(np.float32)
    p = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.99, eps=0.0, weight_decay=0.01, step=5)
    base = orc.adamw(p, g, m, v, **kw)
    for k in (-7, 3, 12):
        s = np.float32(2.0 ** k)
        r = orc.adamw(p, g * s, m * s, v * s * s, **kw)
        assert np.array_equal(r[0], base[0])
        assert np.array_equal(r[1], base[1] * s)
        assert np.array_equal(r[2], base[2] * s * s)


def test_decay_closed_form_and_zero_rate():
    # g = m = v = 0 and eps > 0: u = 0, so p <- p (1 - lr wd); lr = wd = 1/2
    # makes d = 3/4 and every product exact
    p = np.array([4.0, -8.0, 0.5, 1.0, -16.0], np.float32)
    z = np.zeros_like(p)
    for bf in (False, True):
        p1, m1, v1 = orc.adamw(p, z, z, z, lr=0.5, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.5,
                               step=3, param_bf16=bf)
        assert np.array_equal(p1, 0.75 * p)
        assert not m1.any() and not v1.any()
    # lr = 0 leaves p unchanged, decay or not, while the moments still move
    rng = np.random.default_rng(93)
    g = rng.standard_normal(64).astype(np.float32)
    p = (rng.standard_normal(64) * 0.02).astype(np.float32)
    p1, m1, _ = orc.adamw(p, g, np.zeros(64, np.float32), np.zeros(64, np.float32), lr=0.0, beta1=0.9,
                          beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    assert np.array_equal(p1, p)
    assert np.array_equal(m1, np.float32(1.0 - np.float32(0.9)) * g)


def test_bf16_parameter_ties_round_to_even():
    # first-step sign descent with lr = 2^-8 moves p by exactly 2^-8, half a
    # bfloat16 ulp at 1: 1 + 2^-8 rounds to 1 (even), 1 + 2^-7 + 2^-8 to 1 + 2^-6
    g = np.array([-1.0, -1.0, 1.0], np.float32)
    p = np.array([1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -7], np.float32)
    z = np.zeros_like(g)
    kw = dict(lr=2.0 ** -8, beta1=0.5, beta2=0.9375, eps=0.0, weight_decay=0.0, step=1)
    p32, _, _ = orc.adamw(p, g, z, z, **kw)
    assert np.array_equal(p32, np.array([1 + 2 ** -8, 1 + 2 ** -7 + 2 ** -8, 1 + 2 ** -8], np.float32))
    pbf, _, _ = orc.adamw(p, g, z, z, param_bf16=True, **kw)
    assert np.array_equal(pbf, np.array([1.0, 1.0 + 2 ** -6, 1.0], np.float32))


def test_d24_adamw_workload_matches_the_page_counts():
    # the page's total, transformer-matrix and head counts leave 13 tables of
    # vocab x width plus 48 scalars; the AdamW workload is those plus the head
    import json
    import os

    from muon_newton_schulz_02_amd import workloads as wlm
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "d24_shapes.json")))
    rest = g["total_params"] - g["transformer_matrices"] - g["lm_head"]
    table = g["vocab"] * g["width"]
    assert table == g["lm_head"]
    assert rest == 13 * table + 2 * g["layers"]
    wl = wlm.adamw_workload()
    assert wl.elements == rest + g["lm_head"]
    assert sum(s.numel == table for s in wl.specs) == 14
