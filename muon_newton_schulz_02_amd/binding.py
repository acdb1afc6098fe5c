"""ctypes binding of libmuon_mi355x.so (declared in include/muon.h).

Argument marshalling only: tensors become device pointers, row strides and
dtype codes; the torch stream becomes a hipStream_t.  Every step of the
computation runs in the library's HIP kernels.  If the library is not
built, the first call raises `MuonLibraryMissing`; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmuon_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "muon.h")

MUON_OK = 0
MUON_ERR_INVALID_ARGUMENT = 1
MUON_ERR_UNSUPPORTED = 2
MUON_ERR_ALIAS = 3
MUON_ERR_OUT_OF_MEMORY = 4
MUON_ERR_HIP = 5

DTYPE_F32 = 0
DTYPE_BF16 = 1

NS_BF16 = 0
NS_BF16X3 = 1
NS_F32 = 2

SCALE_NONE = 0
SCALE_SQRT_ASPECT = 1
SCALE_RMS_MATCH = 2


class MuonLibraryMissing(RuntimeError):
    pass


class MuonError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_name(status)}: {detail}")
        self.status = status
        self.detail = detail


class MatrixDesc(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("ld_param", ctypes.c_int64), ("ld_grad", ctypes.c_int64), ("ld_mom", ctypes.c_int64),
        ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
        ("mom_dtype", ctypes.c_int32), ("precision", ctypes.c_int32),
    ]


class NsCoeffs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float)]


MOMENTUM_HEAVY_BALL = 0
MOMENTUM_EMA = 1


class StepOptions(ctypes.Structure):
    """muon_step_options (include/muon.h)."""
    _fields_ = [
        ("ns_schedule", ctypes.POINTER(NsCoeffs)), ("weight_decay", ctypes.c_float),
        ("momentum_kind", ctypes.c_int32), ("lr_per_matrix", ctypes.POINTER(ctypes.c_float)),
        ("scale_per_matrix", ctypes.POINTER(ctypes.c_float)), ("launch_mode", ctypes.c_int32),
        ("tile_mode", ctypes.c_int32),
    ]


TILES_AUTO = 0
TILES_LARGE = 1
TILES_SMALL = 2


LAUNCH_AUTO = 0
LAUNCH_PHASE_GRIDS = 1
LAUNCH_CHAIN = 2


class AdamwDesc(ctypes.Structure):
    """muon_adamw_desc (include/muon.h)."""
    _fields_ = [("numel", ctypes.c_int64), ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32)]


class AdamwHparams(ctypes.Structure):
    """muon_adamw_hparams (include/muon.h)."""
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64),
        ("lr_per_tensor", ctypes.POINTER(ctypes.c_float)), ("wd_per_tensor", ctypes.POINTER(ctypes.c_float)),
    ]


class StepHparams(ctypes.Structure):
    """muon_step_hparams (include/muon.h)."""
    _fields_ = [
        ("lr", ctypes.c_float), ("beta", ctypes.c_float), ("nesterov", ctypes.c_int32),
        ("ns_coeffs", NsCoeffs), ("ns_steps", ctypes.c_int32), ("scale_rule", ctypes.c_int32),
        ("options", ctypes.POINTER(StepOptions)),
    ]


_VP = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_lib = None


def exported_names() -> list[str]:
    """Function names declared in include/muon.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(muon_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MuonLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m muon_newton_schulz_02_amd.build` "
            "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    i32, f32, u64 = ctypes.c_int32, ctypes.c_float, ctypes.c_uint64
    D = ctypes.POINTER(MatrixDesc)
    L.muon_step_batched.argtypes = [_PP, _PP, _PP, D, i32, f32, f32, i32, NsCoeffs, i32, i32, _VP]
    L.muon_step_batched.restype = i32
    L.muon_step_batched_ex.argtypes = [_PP, _PP, _PP, D, i32, f32, f32, i32, NsCoeffs, i32, i32, _PP, _VP]
    L.muon_step_batched_ex.restype = i32
    L.muon_step_batched_noalloc.argtypes = [_PP, _PP, _PP, D, i32, f32, f32, i32, NsCoeffs, i32, i32, _PP, _VP]
    L.muon_step_batched_noalloc.restype = i32
    L.muon_step_batched_v2.argtypes = [_PP, _PP, _PP, D, i32, f32, f32, i32, NsCoeffs, i32, i32,
                                       ctypes.POINTER(StepOptions), _PP, _VP]
    L.muon_step_batched_v2.restype = i32
    L.muon_adamw_batched.argtypes = [_PP, _PP, _PP, _PP, ctypes.POINTER(AdamwDesc), i32,
                                     ctypes.POINTER(AdamwHparams), _VP]
    L.muon_adamw_batched.restype = i32
    L.muon_mfma_probe.argtypes = [ctypes.c_int64, _VP, ctypes.POINTER(ctypes.c_double), _VP]
    L.muon_mfma_probe.restype = i32
    L.muon_ns_batched.argtypes = [_PP, _PP, D, i32, NsCoeffs, i32, _VP]
    L.muon_ns_batched.restype = i32
    L.muon_frobenius_norms.argtypes = [_PP, D, i32, _VP, _VP]
    L.muon_frobenius_norms.restype = i32
    L.muon_workspace_bytes.argtypes = [D, i32]
    L.muon_workspace_bytes.restype = u64
    L.muon_release_workspace.argtypes = []
    L.muon_release_workspace.restype = i32
    L.muon_status_string.argtypes = [i32]
    L.muon_status_string.restype = ctypes.c_char_p
    L.muon_last_error.argtypes = []
    L.muon_last_error.restype = ctypes.c_char_p
    L.muon_timing_enable.argtypes = [i32]
    L.muon_timing_enable.restype = i32
    L.muon_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.muon_timing_read.restype = i32
    L.muon_abi_version.argtypes = []
    L.muon_abi_version.restype = i32
    L.muon_stream_plan_create.argtypes = [_PP, _PP, _PP, D, i32, ctypes.POINTER(i32), i32, i32, _PP, _PP]
    L.muon_stream_plan_create.restype = i32
    L.muon_stream_submit.argtypes = [_VP, i32, _VP, ctypes.POINTER(StepHparams), _VP]
    L.muon_stream_submit.restype = i32
    L.muon_stream_plan_destroy.argtypes = [_VP]
    L.muon_stream_plan_destroy.restype = i32
    _lib = L
    return L


def status_name(status: int) -> str:
    try:
        return lib().muon_status_string(int(status)).decode()
    except MuonLibraryMissing:
        return f"status {status}"


def muon_status_string(status: int) -> str:
    return lib().muon_status_string(int(status)).decode()


def muon_last_error() -> str:
    return lib().muon_last_error().decode()


def muon_abi_version() -> int:
    return int(lib().muon_abi_version())


def muon_release_workspace() -> None:
    _check(lib().muon_release_workspace())


KERNEL_CLASSES = ("momentum", "norm", "gram", "poly", "combine", "writeback", "adamw", "chain")


def muon_timing_enable(enable: bool) -> None:
    _check(lib().muon_timing_enable(1 if enable else 0))


def muon_timing_read() -> dict:
    """{class: (total_ms, launches)} of the launches recorded since the last read."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().muon_timing_read(ms, cnt))
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_CLASSES)}


def _check(status: int) -> None:
    if status != MUON_OK:
        raise MuonError(status, muon_last_error())


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return DTYPE_F32
    if dt == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")


def _row_stride(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D (got shape {tuple(t.shape)})")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have unit column stride")
    return max(int(t.stride(0)), int(t.shape[1])) if t.shape[0] == 1 else int(t.stride(0))


def _ptr_array(ptrs) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(len(ptrs), 1))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def _stream_handle(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _precisions(precision, n):
    if isinstance(precision, (list, tuple)):
        if len(precision) != n:
            raise ValueError("one precision per matrix")
        return [int(p) for p in precision]
    return [int(precision)] * n


class StepArgs:
    """Pointer and descriptor arrays for a fixed list of tensors, built once
    and reused by every call on the same tensors."""

    def __init__(self, params, grads, momenta, precision=NS_BF16, updates_out=None):
        n = len(grads)
        if len(params) != n or len(momenta) != n:
            raise ValueError("params, grads and momenta must have the same length")
        precs = _precisions(precision, n)
        self.count = n
        self.descs = (MatrixDesc * max(n, 1))()
        for i, (w, g, m) in enumerate(zip(params, grads, momenta)):
            d = self.descs[i]
            d.ld_param = _row_stride(w, "param")
            d.ld_grad = _row_stride(g, "grad")
            d.ld_mom = _row_stride(m, "momentum")
            if tuple(w.shape) != tuple(g.shape) or tuple(m.shape) != tuple(g.shape):
                raise ValueError(f"matrix {i}: param, grad and momentum shapes differ")
            d.rows, d.cols = int(g.shape[0]), int(g.shape[1])
            d.param_dtype = dtype_code(w.dtype)
            d.grad_dtype = dtype_code(g.dtype)
            d.mom_dtype = dtype_code(m.dtype)
            d.precision = precs[i]
        self.params = _ptr_array([t.data_ptr() for t in params])
        self.grads = _ptr_array([t.data_ptr() for t in grads])
        self.momenta = _ptr_array([t.data_ptr() for t in momenta])
        self.updates = None
        if updates_out is not None:
            if len(updates_out) != n:
                raise ValueError("one updates_out entry per matrix (None allowed)")
            for i, u in enumerate(updates_out):
                if u is not None and (u.dtype != torch.float32 or not u.is_contiguous()
                                      or tuple(u.shape) != (self.descs[i].rows, self.descs[i].cols)):
                    raise ValueError(f"updates_out[{i}] must be a contiguous float32 rows x cols tensor")
            self.updates = _ptr_array([0 if u is None else u.data_ptr() for u in updates_out])
        self._keep = (params, grads, momenta, updates_out)


def muon_step_batched(params, grads=None, momenta=None, *, lr, beta, nesterov, ns_coeffs, ns_steps,
                      scale_rule=SCALE_NONE, precision=NS_BF16, stream=None, updates_out=None):
    """One Muon step on lists of 2-D tensors (or on a prebuilt StepArgs)."""
    args = params if isinstance(params, StepArgs) else StepArgs(params, grads, momenta, precision, updates_out)
    a, b, c = ns_coeffs
    co = NsCoeffs(float(a), float(b), float(c))
    st = _stream_handle(stream)
    if args.updates is None:
        status = lib().muon_step_batched(args.params, args.grads, args.momenta, args.descs, args.count,
                                         float(lr), float(beta), int(nesterov), co, int(ns_steps),
                                         int(scale_rule), st)
    else:
        status = lib().muon_step_batched_ex(args.params, args.grads, args.momenta, args.descs, args.count,
                                            float(lr), float(beta), int(nesterov), co, int(ns_steps),
                                            int(scale_rule), args.updates, st)
    _check(status)


def muon_step_batched_v2(params, grads=None, momenta=None, *, lr, beta, nesterov, ns_coeffs, ns_steps,
                         scale_rule=SCALE_NONE, precision=NS_BF16, stream=None, updates_out=None,
                         ns_schedule=None, weight_decay=0.0, momentum_kind=MOMENTUM_HEAVY_BALL,
                         lr_per_matrix=None, scale_per_matrix=None, launch_mode=LAUNCH_AUTO,
                         tile_mode=TILES_AUTO):
    """muon_step_batched with the update variants of muon_step_options."""
    args = params if isinstance(params, StepArgs) else StepArgs(params, grads, momenta, precision, updates_out)
    a, b, c = ns_coeffs
    co = NsCoeffs(float(a), float(b), float(c))
    opt, keep = _step_options(args.count, ns_steps, ns_schedule, weight_decay, momentum_kind, lr_per_matrix,
                              scale_per_matrix, launch_mode, tile_mode)
    status = lib().muon_step_batched_v2(args.params, args.grads, args.momenta, args.descs, args.count,
                                        float(lr), float(beta), int(nesterov), co, int(ns_steps),
                                        int(scale_rule), ctypes.byref(opt), args.updates, _stream_handle(stream))
    del keep
    _check(status)


def _step_options(count, ns_steps, ns_schedule, weight_decay, momentum_kind, lr_per_matrix, scale_per_matrix,
                  launch_mode, tile_mode):
    """A muon_step_options and the ctypes arrays it points into (keep them alive)."""
    opt = StepOptions()
    keep = []
    if ns_schedule is not None:
        if len(ns_schedule) != int(ns_steps):
            raise ValueError("ns_schedule needs one triple per step")
        arr = (NsCoeffs * max(len(ns_schedule), 1))(*[NsCoeffs(*(float(v) for v in t)) for t in ns_schedule])
        keep.append(arr)
        opt.ns_schedule = ctypes.cast(arr, ctypes.POINTER(NsCoeffs))
    opt.weight_decay = float(weight_decay)
    opt.momentum_kind = int(momentum_kind)
    opt.launch_mode = int(launch_mode)
    opt.tile_mode = int(tile_mode)
    for name, vals in (("lr_per_matrix", lr_per_matrix), ("scale_per_matrix", scale_per_matrix)):
        if vals is not None:
            if len(vals) != count:
                raise ValueError(f"{name} needs one value per matrix")
            arr = (ctypes.c_float * max(len(vals), 1))(*[float(v) for v in vals])
            keep.append(arr)
            setattr(opt, name, ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)))
    return opt, keep


class StreamPlan:
    """A stream plan (muon_stream_plan_create): the step of each group of
    matrices is submitted on its own, behind the event that marks that
    group's gradients complete, so it can start while backward still runs.
    The results equal one muon_step_batched_v2 call over every matrix."""

    def __init__(self, params, grads, momenta, group_of, ngroups=None, *, precision=NS_BF16,
                 tile_mode=TILES_AUTO, updates_out=None):
        self.args = StepArgs(params, grads, momenta, precision, updates_out)
        if len(group_of) != self.args.count:
            raise ValueError("one group index per matrix")
        self.ngroups = int(ngroups) if ngroups is not None else (max(group_of) + 1 if len(group_of) else 0)
        grp = (ctypes.c_int32 * max(len(group_of), 1))(*[int(v) for v in group_of])
        self._h = ctypes.c_void_p()
        _check(lib().muon_stream_plan_create(self.args.params, self.args.grads, self.args.momenta, self.args.descs,
                                             self.args.count, grp, self.ngroups, int(tile_mode), self.args.updates,
                                             ctypes.byref(self._h)))

    def submit(self, group, ready_event=None, *, lr, beta, nesterov, ns_coeffs, ns_steps, scale_rule=SCALE_NONE,
               stream=None, ns_schedule=None, weight_decay=0.0, momentum_kind=MOMENTUM_HEAVY_BALL,
               lr_per_matrix=None, scale_per_matrix=None, launch_mode=LAUNCH_AUTO):
        """Enqueue group `group`'s step behind `ready_event` (a recorded
        torch.cuda.Event, a raw hipEvent_t as an int, or None)."""
        if self._h is None or not self._h.value:
            raise ValueError("the stream plan is closed")
        opt, keep = _step_options(self.args.count, ns_steps, ns_schedule, weight_decay, momentum_kind,
                                  lr_per_matrix, scale_per_matrix, launch_mode, TILES_AUTO)
        a, b, c = ns_coeffs
        hp = StepHparams(float(lr), float(beta), int(nesterov), NsCoeffs(float(a), float(b), float(c)),
                         int(ns_steps), int(scale_rule), ctypes.pointer(opt))
        if ready_event is None:
            ev = None
        elif isinstance(ready_event, int):
            ev = ready_event
        else:
            ev = ready_event.cuda_event
        status = lib().muon_stream_submit(self._h, int(group), ev, ctypes.byref(hp), _stream_handle(stream))
        del keep
        _check(status)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().muon_stream_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass


def muon_step_batched_ex(params, grads, momenta, updates_out, **kw):
    """muon_step_batched that also exports the binary32 update O of each matrix."""
    return muon_step_batched(params, grads, momenta, updates_out=updates_out, **kw)


class AdamwArgs:
    """Pointer and descriptor arrays of a fixed list of AdamW tensors, built
    once and reused by every call on the same tensors."""

    def __init__(self, params, grads, exp_avg, exp_avg_sq):
        n = len(params)
        if len(grads) != n or len(exp_avg) != n or len(exp_avg_sq) != n:
            raise ValueError("params, grads, exp_avg and exp_avg_sq must have the same length")
        self.count = n
        self.descs = (AdamwDesc * max(n, 1))()
        for i, (p, g, m, v) in enumerate(zip(params, grads, exp_avg, exp_avg_sq)):
            for name, t in (("param", p), ("grad", g), ("exp_avg", m), ("exp_avg_sq", v)):
                if not t.is_contiguous():
                    raise ValueError(f"tensor {i}: {name} must be contiguous")
            if not (p.numel() == g.numel() == m.numel() == v.numel()):
                raise ValueError(f"tensor {i}: param, grad and moments differ in size")
            if m.dtype != torch.float32 or v.dtype != torch.float32:
                raise TypeError(f"tensor {i}: the moments must be float32")
            d = self.descs[i]
            d.numel = int(p.numel())
            d.param_dtype = dtype_code(p.dtype)
            d.grad_dtype = dtype_code(g.dtype)
        self.params = _ptr_array([t.data_ptr() for t in params])
        self.grads = _ptr_array([t.data_ptr() for t in grads])
        self.exp_avg = _ptr_array([t.data_ptr() for t in exp_avg])
        self.exp_avg_sq = _ptr_array([t.data_ptr() for t in exp_avg_sq])
        self._keep = (params, grads, exp_avg, exp_avg_sq)


def muon_adamw_batched(params, grads=None, exp_avg=None, exp_avg_sq=None, *, lr, beta1, beta2, eps,
                       weight_decay=0.0, step, lr_per_tensor=None, wd_per_tensor=None, stream=None):
    """One AdamW step on lists of contiguous tensors (or on a prebuilt AdamwArgs)."""
    args = params if isinstance(params, AdamwArgs) else AdamwArgs(params, grads, exp_avg, exp_avg_sq)
    hp = AdamwHparams()
    hp.lr, hp.beta1, hp.beta2, hp.eps = float(lr), float(beta1), float(beta2), float(eps)
    hp.weight_decay = float(weight_decay)
    hp.step = int(step)
    keep = []
    for name, vals in (("lr_per_tensor", lr_per_tensor), ("wd_per_tensor", wd_per_tensor)):
        if vals is not None:
            if len(vals) != args.count:
                raise ValueError(f"{name} needs one value per tensor")
            arr = (ctypes.c_float * max(len(vals), 1))(*[float(v) for v in vals])
            keep.append(arr)
            setattr(hp, name, ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)))
    status = lib().muon_adamw_batched(args.params, args.grads, args.exp_avg, args.exp_avg_sq, args.descs,
                                      args.count, ctypes.byref(hp), _stream_handle(stream))
    del keep
    _check(status)


def muon_mfma_probe(iterations: int, sink: torch.Tensor, stream=None) -> float:
    """Enqueue the MFMA-rate probe; returns its floating-point operation count."""
    if sink.dtype != torch.float32 or sink.numel() < 1:
        raise ValueError("sink must be a float32 device tensor of at least one element")
    flops = ctypes.c_double(0.0)
    _check(lib().muon_mfma_probe(int(iterations), sink.data_ptr(), ctypes.byref(flops), _stream_handle(stream)))
    return float(flops.value)


def muon_ns_batched(x_in, x_out, *, ns_coeffs, ns_steps, precision=NS_BF16, stream=None):
    """x_out[i] (float32) = Newton-Schulz orthogonalisation of x_in[i]."""
    n = len(x_in)
    if len(x_out) != n:
        raise ValueError("x_in and x_out must have the same length")
    precs = _precisions(precision, n)
    descs = (MatrixDesc * max(n, 1))()
    for i, (x, y) in enumerate(zip(x_in, x_out)):
        if y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != tuple(x.shape):
            raise ValueError(f"x_out[{i}] must be a contiguous float32 tensor shaped like x_in[{i}]")
        d = descs[i]
        d.rows, d.cols = int(x.shape[0]), int(x.shape[1])
        d.ld_grad = _row_stride(x, "x_in")
        d.ld_param = d.ld_mom = d.cols
        d.grad_dtype = dtype_code(x.dtype)
        d.param_dtype = DTYPE_F32
        d.mom_dtype = DTYPE_F32
        d.precision = precs[i]
    a, b, c = ns_coeffs
    _check(lib().muon_ns_batched(_ptr_array([t.data_ptr() for t in x_in]),
                                 _ptr_array([t.data_ptr() for t in x_out]), descs, n,
                                 NsCoeffs(float(a), float(b), float(c)), int(ns_steps),
                                 _stream_handle(stream)))


def muon_frobenius_norms(x_in, norms_out, *, stream=None):
    """norms_out (float32 device tensor of len(x_in)) = Frobenius norms."""
    n = len(x_in)
    if norms_out.dtype != torch.float32 or norms_out.numel() < n:
        raise ValueError("norms_out must be float32 with one entry per matrix")
    descs = (MatrixDesc * max(n, 1))()
    for i, x in enumerate(x_in):
        d = descs[i]
        d.rows, d.cols = int(x.shape[0]), int(x.shape[1])
        d.ld_grad = _row_stride(x, "x_in")
        d.ld_param = d.ld_mom = d.cols
        d.grad_dtype = dtype_code(x.dtype)
    _check(lib().muon_frobenius_norms(_ptr_array([t.data_ptr() for t in x_in]), descs, n,
                                      norms_out.data_ptr(), _stream_handle(stream)))


def muon_workspace_bytes(shapes, precision=NS_BF16) -> int:
    """Workspace bytes for [(rows, cols), ...]."""
    n = len(shapes)
    precs = _precisions(precision, n)
    descs = (MatrixDesc * max(n, 1))()
    for i, (r, c) in enumerate(shapes):
        d = descs[i]
        d.rows, d.cols = int(r), int(c)
        d.ld_param = d.ld_grad = d.ld_mom = int(c)
        d.precision = precs[i]
        d.grad_dtype = DTYPE_BF16
    return int(lib().muon_workspace_bytes(descs, n))
