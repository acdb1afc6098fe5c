"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import subprocess

import pytest
import torch

from muon_newton_schulz_02_amd import binding as mb
from muon_newton_schulz_02_amd import build as mbuild


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mb.LIB_PATH):
        mbuild.build(verbose=False)
    return mb.lib()


def test_exports_every_declared_symbol(L):
    names = mb.exported_names()
    assert len(names) == 18
    out = subprocess.run(["nm", "-D", "--defined-only", mb.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_version_and_strings(L):
    assert mb.muon_abi_version() == 4
    assert mb.muon_status_string(mb.MUON_OK) == "MUON_OK"
    assert mb.muon_status_string(mb.MUON_ERR_ALIAS) == "MUON_ERR_ALIAS"
    assert mb.muon_status_string(99) == "MUON_ERR_UNKNOWN"


def _desc(rows, cols, ld=None, pdt=mb.DTYPE_BF16, gdt=mb.DTYPE_BF16, mdt=mb.DTYPE_F32, prec=mb.NS_BF16):
    d = mb.MatrixDesc()
    d.rows, d.cols = rows, cols
    d.ld_param = d.ld_grad = d.ld_mom = cols if ld is None else ld
    d.param_dtype, d.grad_dtype, d.mom_dtype, d.precision = pdt, gdt, mdt, prec
    return d


def _call(L, descs, params, grads, moms, lr=0.02, beta=0.95, nesterov=1, coeffs=(3.4445, -4.775, 2.0315),
          steps=5, rule=0, updates=None):
    n = len(descs)
    D = (mb.MatrixDesc * max(n, 1))(*descs)
    P = mb._ptr_array(params)
    G = mb._ptr_array(grads)
    M = mb._ptr_array(moms)
    co = mb.NsCoeffs(*coeffs)
    if updates is None:
        return L.muon_step_batched(P, G, M, D, n, lr, beta, nesterov, co, steps, rule, None)
    return L.muon_step_batched_ex(P, G, M, D, n, lr, beta, nesterov, co, steps, rule,
                                  mb._ptr_array(updates), None)


# Fake device addresses: validation only compares them, nothing dereferences them.
BASE = 0x7F0000000000


def _ptrs(i, rows, cols):
    p = BASE + i * 0x10000000
    return p, p + 0x1000000, p + 0x2000000


def test_count_zero_is_noop(L):
    assert _call(L, [], [], [], []) == mb.MUON_OK


@pytest.mark.parametrize("field,value,status", [
    ("rows", 0, mb.MUON_ERR_INVALID_ARGUMENT),
    ("cols", -3, mb.MUON_ERR_INVALID_ARGUMENT),
    ("rows", 70000, mb.MUON_ERR_UNSUPPORTED),
    ("ld_grad", 10, mb.MUON_ERR_INVALID_ARGUMENT),
    ("ld_mom", 10, mb.MUON_ERR_INVALID_ARGUMENT),
    ("mom_dtype", mb.DTYPE_BF16, mb.MUON_ERR_UNSUPPORTED),
    ("param_dtype", 7, mb.MUON_ERR_UNSUPPORTED),
    ("grad_dtype", 7, mb.MUON_ERR_UNSUPPORTED),
    ("precision", 9, mb.MUON_ERR_INVALID_ARGUMENT),
])
def test_descriptor_errors(L, field, value, status):
    d = _desc(16, 32)
    setattr(d, field, value)
    p, g, m = _ptrs(0, 16, 32)
    assert _call(L, [d], [p], [g], [m]) == status
    assert mb.muon_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(lr=float("nan")), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(lr=float("inf")), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(beta=1.0), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(beta=-0.1), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(beta=float("nan")), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(nesterov=2), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(steps=-1), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(rule=5), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(coeffs=(float("nan"), 0.0, 0.0)), mb.MUON_ERR_INVALID_ARGUMENT),
])
def test_scalar_errors(L, kw, status):
    p, g, m = _ptrs(0, 16, 32)
    assert _call(L, [_desc(16, 32)], [p], [g], [m], **kw) == status


@pytest.mark.parametrize("coeffs", [
    (3.4445, -4.775, 1e-39),             # subnormal c: b/c is -inf in binary32
    (3.4445, -4.775, 1e-38),             # b/c = -4.8e38: finite binary32, but its bf16 part is not
    (3.4e38, -4.775, 2.0315),            # a too large for a finite bf16 hi part
])
def test_coefficients_that_cannot_be_split_are_rejected(L, coeffs):
    # the products run a X and (b/c) A as bfloat16 hi + lo pairs; a triple
    # whose a or fl32(b/c) has no finite bf16 hi part would turn B into NaN
    p, g, m = _ptrs(0, 16, 32)
    assert _call(L, [_desc(16, 32)], [p], [g], [m], coeffs=coeffs) == mb.MUON_ERR_UNSUPPORTED
    assert "split" in mb.muon_last_error()
    # the same triple in a schedule, at its step only
    sched = (mb.NsCoeffs * 2)(mb.NsCoeffs(3.4445, -4.775, 2.0315), mb.NsCoeffs(*coeffs))
    o = _opt(ns_schedule=ctypes.cast(sched, ctypes.POINTER(mb.NsCoeffs)))
    assert _call_v2(L, ctypes.byref(o), steps=2) == mb.MUON_ERR_UNSUPPORTED
    assert "ns_schedule[1]" in mb.muon_last_error()
    assert _call_v2(L, ctypes.byref(o), steps=1) != mb.MUON_ERR_UNSUPPORTED


def test_coefficients_at_the_split_limit_pass(L):
    # c = 0 never forms b/c; a large but splittable b/c passes validation
    p, g, m = _ptrs(0, 16, 32)
    for coeffs in [(1.5, -0.5, 0.0), (3.4445, -4.775, 1e-30), (3.3e38, 1.0, 0.0)]:
        st = _call(L, [_desc(16, 32)], [p], [g], [m], coeffs=coeffs)
        assert st not in (mb.MUON_ERR_UNSUPPORTED, mb.MUON_ERR_INVALID_ARGUMENT), (coeffs, mb.muon_last_error())
    # with no Newton-Schulz step the triple is not used
    assert _call(L, [_desc(16, 32)], [p], [g], [m], coeffs=(1.0, 1.0, 1e-39), steps=0) \
        not in (mb.MUON_ERR_UNSUPPORTED, mb.MUON_ERR_INVALID_ARGUMENT)


def _call_v2(L, opt, steps=5, n=1):
    descs = [_desc(16, 32) for _ in range(n)]
    ptrs = [_ptrs(i, 16, 32) for i in range(n)]
    D = (mb.MatrixDesc * n)(*descs)
    return L.muon_step_batched_v2(mb._ptr_array([p for p, _, _ in ptrs]), mb._ptr_array([g for _, g, _ in ptrs]),
                                  mb._ptr_array([m for _, _, m in ptrs]), D, n, 0.02, 0.95, 1,
                                  mb.NsCoeffs(3.4445, -4.775, 2.0315), steps, 0, opt, None, None)


def _opt(**kw):
    o = mb.StepOptions()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def _floats(*v):
    arr = (ctypes.c_float * len(v))(*v)
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)), arr


def test_tile_mode_errors(L):
    assert _call_v2(L, ctypes.byref(_opt(tile_mode=3))) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _call_v2(L, ctypes.byref(_opt(tile_mode=-1))) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _call_v2(L, ctypes.byref(_opt(tile_mode=mb.TILES_SMALL))) != mb.MUON_ERR_INVALID_ARGUMENT


def test_launch_mode_errors(L):
    assert _call_v2(L, ctypes.byref(_opt(launch_mode=3))) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _call_v2(L, ctypes.byref(_opt(launch_mode=-1))) == mb.MUON_ERR_INVALID_ARGUMENT
    # the chain takes at most 16 steps; the per-phase grids take any number
    assert _call_v2(L, ctypes.byref(_opt(launch_mode=mb.LAUNCH_CHAIN)), steps=17) == mb.MUON_ERR_UNSUPPORTED
    assert _call_v2(L, ctypes.byref(_opt(launch_mode=mb.LAUNCH_CHAIN)), steps=16) != mb.MUON_ERR_UNSUPPORTED
    assert _call_v2(L, ctypes.byref(_opt(launch_mode=mb.LAUNCH_PHASE_GRIDS)), steps=17) \
        not in (mb.MUON_ERR_UNSUPPORTED, mb.MUON_ERR_INVALID_ARGUMENT)


@pytest.mark.parametrize("case", ["kind", "wd_neg", "wd_nan", "schedule_nan", "lr_nan", "scale_inf"])
def test_option_errors(L, case):
    keep = []
    if case == "kind":
        o = _opt(momentum_kind=2)
    elif case == "wd_neg":
        o = _opt(weight_decay=-0.1)
    elif case == "wd_nan":
        o = _opt(weight_decay=float("nan"))
    elif case == "schedule_nan":
        sched = (mb.NsCoeffs * 5)(*([mb.NsCoeffs(3.4445, -4.775, 2.0315)] * 4 + [mb.NsCoeffs(float("nan"), 0, 0)]))
        keep.append(sched)
        o = _opt(ns_schedule=ctypes.cast(sched, ctypes.POINTER(mb.NsCoeffs)))
    elif case == "lr_nan":
        ptr, arr = _floats(0.02, float("nan"))
        keep.append(arr)
        o = _opt(lr_per_matrix=ptr)
    else:
        ptr, arr = _floats(1.0, float("inf"))
        keep.append(arr)
        o = _opt(scale_per_matrix=ptr)
    assert _call_v2(L, ctypes.byref(o), n=2) == mb.MUON_ERR_INVALID_ARGUMENT
    assert mb.muon_last_error() != ""


def test_option_schedule_only_read_for_its_steps(L):
    # a schedule of 2 valid triples with ns_steps = 2 passes validation (the
    # call then fails only for want of a GPU, or runs on one)
    sched = (mb.NsCoeffs * 2)(mb.NsCoeffs(3.4445, -4.775, 2.0315), mb.NsCoeffs(1.5, -0.5, 0.0))
    o = _opt(ns_schedule=ctypes.cast(sched, ctypes.POINTER(mb.NsCoeffs)), weight_decay=0.1, momentum_kind=1)
    assert _call_v2(L, ctypes.byref(o), steps=2) != mb.MUON_ERR_INVALID_ARGUMENT
    assert _call_v2(L, None) != mb.MUON_ERR_INVALID_ARGUMENT


def test_null_and_alignment(L):
    p, g, m = _ptrs(0, 16, 32)
    assert _call(L, [_desc(16, 32)], [0], [g], [m]) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _call(L, [_desc(16, 32)], [p], [0], [m]) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _call(L, [_desc(16, 32)], [p + 1], [g], [m]) == mb.MUON_ERR_UNSUPPORTED
    assert _call(L, [_desc(16, 32)], [p], [g], [m + 2]) == mb.MUON_ERR_UNSUPPORTED
    D = (mb.MatrixDesc * 1)(_desc(16, 32))
    assert L.muon_step_batched(None, mb._ptr_array([g]), mb._ptr_array([m]), D, 1, 0.02, 0.9, 0,
                               mb.NsCoeffs(1.5, -0.5, 0.0), 5, 0, None) == mb.MUON_ERR_INVALID_ARGUMENT


def test_alias_detection(L):
    p, g, m = _ptrs(0, 16, 32)
    # param overlapping its own gradient
    assert _call(L, [_desc(16, 32)], [p], [p + 64], [m]) == mb.MUON_ERR_ALIAS
    # momentum of matrix 1 overlapping the param of matrix 0
    p1, g1, _ = _ptrs(1, 16, 32)
    assert _call(L, [_desc(16, 32), _desc(16, 32)], [p, p1], [g, g1], [m, p + 16 * 32 * 2 - 4]) \
        == mb.MUON_ERR_ALIAS
    # two matrices reading one gradient is allowed by validation (then fails later
    # only for want of a GPU, or succeeds on one)
    st = _call(L, [_desc(16, 32), _desc(16, 32)], [p, p1], [g, g], [m, m + 0x100000])
    assert st != mb.MUON_ERR_ALIAS
    # update export overlapping a weight
    assert _call(L, [_desc(16, 32)], [p], [g], [m], updates=[p + 32]) == mb.MUON_ERR_ALIAS
    # strided rows are taken into account: ld = 64 makes param 0 reach further
    d = _desc(16, 32, ld=64)
    assert _call(L, [d], [p], [p + (15 * 64 + 32) * 2 - 2], [m]) == mb.MUON_ERR_ALIAS
    assert _call(L, [d], [p], [p + (15 * 64 + 32) * 2], [m]) != mb.MUON_ERR_ALIAS


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
@pytest.mark.parametrize("rows,cols,prec,status", [
    (32512, 32512, mb.NS_BF16, mb.MUON_ERR_HIP),          # 1.97 GiB working copy: accepted
    (32768, 32768, mb.NS_BF16, mb.MUON_ERR_UNSUPPORTED),  # 2 GiB
    (16128, 65536, mb.NS_BF16, mb.MUON_ERR_HIP),
    (65536, 16384, mb.NS_BF16, mb.MUON_ERR_UNSUPPORTED),  # tall: the same copy as 16384 x 65536
    (23040, 23040, mb.NS_F32, mb.MUON_ERR_HIP),
    (23296, 23296, mb.NS_F32, mb.MUON_ERR_UNSUPPORTED),
    (23296, 23296, mb.NS_BF16X3, mb.MUON_ERR_UNSUPPORTED),
    (23296, 23296, mb.NS_BF16, mb.MUON_ERR_HIP),
])
def test_working_copy_size_cap(L, rows, cols, prec, status):
    # the Newton-Schulz products address one working copy with 32-bit offsets;
    # accepted sizes get as far as the device (no GPU here: MUON_ERR_HIP)
    pdt = mb.DTYPE_F32 if prec != mb.NS_BF16 else mb.DTYPE_BF16
    d = _desc(rows, cols, pdt=pdt, prec=prec)
    p = BASE
    g, m = p + (1 << 36), p + (2 << 36)
    assert _call(L, [d], [p], [g], [m]) == status
    if status == mb.MUON_ERR_UNSUPPORTED:
        assert "2 GiB" in mb.muon_last_error()


def test_valid_call_without_gpu_reports_hip_error(L):
    p, g, m = _ptrs(0, 16, 32)
    assert _call(L, [_desc(16, 32)], [p], [g], [m]) == mb.MUON_ERR_HIP


def test_workspace_bytes(L):
    # workspace rows carry LDPAD (0) elements beyond their padded width
    pad = 0
    one = mb.muon_workspace_bytes([(1536, 1536)])
    # X and X' (2 x 1536 rows) plus A and B (2 x 1536 rows), bf16
    assert one == 4 * 1536 * (1536 + pad) * 2
    tall = mb.muon_workspace_bytes([(6144, 1536)])
    wide = mb.muon_workspace_bytes([(1536, 6144)])
    assert tall == wide == (2 * 1536 * (6144 + pad) + 2 * 1536 * (1536 + pad)) * 2
    assert mb.muon_workspace_bytes([(1536, 1536)], precision=mb.NS_BF16X3) == 2 * one
    assert mb.muon_workspace_bytes([(1536, 1536)], precision=mb.NS_F32) == 2 * one
    # padding to multiples of 256
    assert mb.muon_workspace_bytes([(1, 300)]) == (2 * 256 * (512 + pad) + 2 * 256 * (256 + pad)) * 2
    assert mb.muon_workspace_bytes([(0, 4)]) == 0


def test_python_binding_rejects_bad_tensors():
    w = torch.zeros(4, 4, dtype=torch.float16)
    with pytest.raises(TypeError):
        mb.StepArgs([w], [w], [w])
    with pytest.raises(ValueError):
        mb.StepArgs([torch.zeros(4)], [torch.zeros(4)], [torch.zeros(4)])


# ------------------------------------------------------------------ AdamW

def _adamw_desc(numel, pdt=mb.DTYPE_BF16, gdt=mb.DTYPE_BF16):
    d = mb.AdamwDesc()
    d.numel, d.param_dtype, d.grad_dtype = numel, pdt, gdt
    return d


def _hp(**kw):
    h = mb.AdamwHparams()
    h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.step = 1e-3, 0.9, 0.95, 1e-8, 0.0, 1
    keep = []
    for k, v in kw.items():
        if k in ("lr_per_tensor", "wd_per_tensor"):
            ptr, arr = _floats(*v)
            keep.append(arr)
            setattr(h, k, ptr)
        else:
            setattr(h, k, v)
    h._keep = keep
    return h


def _adamw_ptrs(i):
    p = BASE + 0x40000000 + i * 0x10000000
    return p, p + 0x1000000, p + 0x2000000, p + 0x3000000


def _call_adamw(L, descs, ptrs, hp):
    n = len(descs)
    D = (mb.AdamwDesc * max(n, 1))(*descs)
    cols = list(zip(*ptrs)) if ptrs else ([], [], [], [])
    arrs = [mb._ptr_array(list(c)) for c in cols]
    return L.muon_adamw_batched(arrs[0], arrs[1], arrs[2], arrs[3], D, n,
                                None if hp is None else ctypes.byref(hp), None)


def test_adamw_count_zero_and_empty_tensors(L):
    assert _call_adamw(L, [], [], _hp()) == mb.MUON_OK
    # tensors of zero elements are skipped (their pointers are not read)
    assert _call_adamw(L, [_adamw_desc(0), _adamw_desc(0)], [(0, 0, 0, 0), (0, 0, 0, 0)], _hp()) == mb.MUON_OK
    assert _call_adamw(L, [_adamw_desc(16)], [_adamw_ptrs(0)], None) == mb.MUON_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [
    dict(lr=float("nan")), dict(lr=float("inf")), dict(beta1=1.0), dict(beta2=-0.1), dict(beta1=float("nan")),
    dict(eps=-1e-8), dict(eps=float("nan")), dict(weight_decay=-0.1), dict(weight_decay=float("inf")),
    dict(step=0), dict(step=-3), dict(lr_per_tensor=(1e-3, float("nan"))), dict(wd_per_tensor=(0.0, -0.5)),
])
def test_adamw_hparam_errors(L, kw):
    st = _call_adamw(L, [_adamw_desc(16), _adamw_desc(16)], [_adamw_ptrs(0), _adamw_ptrs(1)], _hp(**kw))
    assert st == mb.MUON_ERR_INVALID_ARGUMENT
    assert mb.muon_last_error() != ""


@pytest.mark.parametrize("desc,status", [
    (dict(numel=-1), mb.MUON_ERR_INVALID_ARGUMENT),
    (dict(numel=(1 << 40) + 1), mb.MUON_ERR_UNSUPPORTED),
    (dict(pdt=7), mb.MUON_ERR_UNSUPPORTED),
    (dict(gdt=-1), mb.MUON_ERR_UNSUPPORTED),
])
def test_adamw_desc_errors(L, desc, status):
    d = _adamw_desc(desc.get("numel", 16), desc.get("pdt", mb.DTYPE_BF16), desc.get("gdt", mb.DTYPE_BF16))
    assert _call_adamw(L, [d], [_adamw_ptrs(0)], _hp()) == status


def test_adamw_pointer_errors_and_aliases(L):
    p, g, m, v = _adamw_ptrs(0)
    d = _adamw_desc(16)
    assert _call_adamw(L, [d], [(0, g, m, v)], _hp()) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _call_adamw(L, [d], [(p, g, m, 0)], _hp()) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _call_adamw(L, [d], [(p + 1, g, m, v)], _hp()) == mb.MUON_ERR_UNSUPPORTED
    assert _call_adamw(L, [d], [(p, g, m + 2, v)], _hp()) == mb.MUON_ERR_UNSUPPORTED
    # second moment overlapping the first
    assert _call_adamw(L, [d], [(p, g, m, m + 60)], _hp()) == mb.MUON_ERR_ALIAS
    # the gradient of tensor 1 inside the parameter of tensor 0 (bf16: 32 bytes)
    p1, g1, m1, v1 = _adamw_ptrs(1)
    assert _call_adamw(L, [d, d], [(p, g, m, v), (p1, p + 30, m1, v1)], _hp()) == mb.MUON_ERR_ALIAS
    assert _call_adamw(L, [d, d], [(p, g, m, v), (p1, p + 32, m1, v1)], _hp()) != mb.MUON_ERR_ALIAS
    # two tensors reading one gradient pass validation
    assert _call_adamw(L, [d, d], [(p, g, m, v), (p1, g, m1, v1)], _hp()) != mb.MUON_ERR_ALIAS


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_adamw_valid_call_without_gpu_reports_hip_error(L):
    assert _call_adamw(L, [_adamw_desc(16)], [_adamw_ptrs(0)], _hp(weight_decay=0.1, step=7)) == mb.MUON_ERR_HIP


def test_adamw_binding_rejects_bad_tensors():
    p = torch.zeros(8, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        mb.AdamwArgs([p], [p], [p.float().half()], [p.float()])
    with pytest.raises(ValueError):
        mb.AdamwArgs([p], [p], [torch.zeros(7)], [torch.zeros(8)])
    with pytest.raises(ValueError):
        mb.AdamwArgs([torch.zeros(4, 4).t()], [torch.zeros(16)], [torch.zeros(16)], [torch.zeros(16)])


def test_mfma_probe_argument_errors(L):
    flops = ctypes.c_double(0.0)
    sink = BASE
    assert L.muon_mfma_probe(0, sink, ctypes.byref(flops), None) == mb.MUON_ERR_INVALID_ARGUMENT
    assert L.muon_mfma_probe((1 << 30) + 1, sink, ctypes.byref(flops), None) == mb.MUON_ERR_INVALID_ARGUMENT
    assert L.muon_mfma_probe(10, None, ctypes.byref(flops), None) == mb.MUON_ERR_INVALID_ARGUMENT
    assert L.muon_mfma_probe(10, sink, None, None) == mb.MUON_ERR_INVALID_ARGUMENT
    assert L.muon_mfma_probe(10, sink + 2, ctypes.byref(flops), None) == mb.MUON_ERR_UNSUPPORTED


# ---------------------------------------------------------------- stream plans

def _create(L, descs, group_of, ngroups, tile_mode=0, out=True):
    n = len(descs)
    D = (mb.MatrixDesc * max(n, 1))(*descs)
    ptrs = [_ptrs(i, d.rows, d.cols) for i, d in enumerate(descs)]
    grp = (ctypes.c_int32 * max(n, 1))(*group_of)
    h = ctypes.c_void_p()
    return L.muon_stream_plan_create(mb._ptr_array([p for p, _, _ in ptrs]), mb._ptr_array([g for _, g, _ in ptrs]),
                                     mb._ptr_array([m for _, _, m in ptrs]), D, n, grp, ngroups, tile_mode, None,
                                     ctypes.byref(h) if out else None)


@pytest.mark.parametrize("group_of,ngroups,tile_mode,out", [
    ([0, 2], 2, 0, True),        # group index out of range
    ([0, -1], 2, 0, True),
    ([0, 0], 0, 0, True),        # no groups
    ([0, 1], 2, 5, True),        # unknown tile mode
    ([0, 1], 2, 0, False),       # no place for the plan
])
def test_stream_plan_create_errors(L, group_of, ngroups, tile_mode, out):
    descs = [_desc(16, 32), _desc(32, 16)]
    assert _create(L, descs, group_of, ngroups, tile_mode, out) == mb.MUON_ERR_INVALID_ARGUMENT
    assert mb.muon_last_error() != ""


def test_stream_plan_create_checks_matrices(L):
    # the matrices are checked as for a step call over the whole set
    d = _desc(16, 32)
    d.ld_grad = 8
    assert _create(L, [_desc(16, 32), d], [0, 1], 2) == mb.MUON_ERR_INVALID_ARGUMENT
    assert _create(L, [], [], 1) == mb.MUON_ERR_INVALID_ARGUMENT
    # valid arguments: without a GPU the call fails only at the device
    assert _create(L, [_desc(16, 32), _desc(32, 16)], [1, 1], 3) == mb.MUON_ERR_HIP


def test_stream_submit_and_destroy_arguments(L):
    hp = mb.StepHparams(0.02, 0.95, 1, mb.NsCoeffs(3.4445, -4.775, 2.0315), 5, 0, None)
    assert L.muon_stream_submit(None, 0, None, ctypes.byref(hp), None) == mb.MUON_ERR_INVALID_ARGUMENT
    assert L.muon_stream_plan_destroy(None) == mb.MUON_OK
