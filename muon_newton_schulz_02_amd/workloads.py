"""Seeded synthetic inputs for the Muon step: shapes, values and step settings.

This module draws random numbers and builds tensors; it holds none of the
optimizer's arithmetic, so both the HIP path (through the tests and the
benchmark) and the CPU oracle can take their inputs from it.

Workloads (shapes from the pages where they give them):

* ``single256_f32``   one 256x256 float32 matrix; W, G, M iid N(0,1) drawn in
  that order from numpy's default_rng(0); beta 0.95, Nesterov, lr 0.02,
  5 cubic steps (1.5, -0.5, 0), float32 Newton-Schulz.
* ``gpt2s_attn768_bf16``  12 square 768x768 bf16 matrices (GPT-2-small
  attention projections); W ~ N(0, 0.02^2), a fresh G ~ N(0, 1e-3^2) on each
  of 3 consecutive steps, M0 = 0, 5 quintic steps.
* ``d24_bf16``  the d24 model of "把 GPT-2 的训练租金估算从 4.3 万美元压到 40 美元…"
  (section "FLOPs 账"): 24 layers, width 1536, 12 heads of 128, so per layer
  Q, K, V, O 1536x1536, MLP up 1536x6144 and down 6144x1536 (144 matrices).
  G = alpha * A B^T + N with A (rows x 16), B (cols x 16), N iid N(0,1);
  alpha puts the top singular value of the rank-16 part at 1e3 times the
  edge of the noise bulk, sqrt(rows) + sqrt(cols).  M0 = 0, 5 quintic steps.
* ``lm3p8b_bf16``  32 layers of the little-lm 3.8B shapes of
  "开发者千美元训3.8B模型 击败GPT-2" (24 query / 8 KV heads, head_dim 128,
  width 3072, MLP 4x): Q, O 3072x3072, K, V 3072x1024, up 3072x12288, down
  12288x3072 (192 matrices).  G iid N(0,1), M0 = 0, 5 quintic steps.
* ``stress_mixed_bf16``  64 matrices with rows and cols drawn iid uniform
  from {512, 1024, 2048, 4096, 8192}; G = Q_u diag(i^-2) Q_v^T with Q_u, Q_v
  the orthonormal factors of Student-t(3) matrices; 10 quintic steps on the
  split-bf16 (BF16X3) path.

AdamW inputs (the non-matrix half of the hybrid optimizer):

* ``d24_adamw_bf16``  the d24 parameters that are not transformer matrices.
  The page gives 1,384,124,976 parameters in all, 679,481,856 in transformer
  matrices and 50,331,648 in the output head (vocab 32768 x 1536); the
  remaining 654,311,472 = 13 x 32768 x 1536 + 48 are read as the token
  embedding plus 12 value embeddings ("Karpathy 只花 $72 就訓練出 GPT-2…",
  section 那些讓 600 倍加速成為可能的技術, names value embeddings and
  learnable residual scalars) and two scalars per layer.  The head, the 13
  embeddings and two 24-element scalar tensors: 704,643,120 elements.
  bf16 p and g; p ~ N(0, 0.02^2) (scalars 1 + N(0, 0.01^2)), g ~ N(0,
  1e-3^2), m ~ N(0, 1e-3^2), v = (N(0, 1e-3^2))^2, as at a step well into
  training (t = 100).

Every tensor is drawn from a torch.Generator seeded from (workload seed,
matrix index, step, purpose), on the device asked for; CPU and GPU
generators give different streams, so a test that compares against the
oracle copies the very tensors it fed the GPU back to the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

CUBIC = (1.5, -0.5, 0.0)
# Textbook quintic Newton-Schulz (Higham, Functions of Matrices, ch. 8).
QUINTIC_TEXTBOOK = (15.0 / 8.0, -5.0 / 4.0, 3.0 / 8.0)
# The quintic commonly used with Muon (K. Jordan's 2024 Muon write-up); it is
# not printed on the pages and is passed in as a parameter like any triple.
QUINTIC_MUON = (3.4445, -4.7750, 2.0315)

PRECISION_BF16 = 0
PRECISION_BF16X3 = 1
PRECISION_F32 = 2


@dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    name: str = ""


@dataclass
class Workload:
    name: str
    specs: list
    param_dtype: torch.dtype
    grad_dtype: torch.dtype
    precision: int
    coeffs: tuple
    ns_steps: int
    lr: float = 0.02
    beta: float = 0.95
    nesterov: bool = True
    n_steps: int = 1
    scale_rule: int = 0
    seed: int = 0
    grad_kind: str = "gaussian"
    grad_std: float = 1.0
    w_std: float = 0.02
    m0_zero: bool = True
    notes: dict = field(default_factory=dict)

    @property
    def elements(self) -> int:
        return sum(s.rows * s.cols for s in self.specs)


def _d24_specs(layers: int = 24, width: int = 1536):
    out = []
    for layer in range(layers):
        for nm in ("q", "k", "v", "o"):
            out.append(MatrixSpec(width, width, f"h{layer}.attn.{nm}"))
        out.append(MatrixSpec(width, 4 * width, f"h{layer}.mlp.up"))
        out.append(MatrixSpec(4 * width, width, f"h{layer}.mlp.down"))
    return out


def _lm38_specs(layers: int = 32, width: int = 3072, kv_width: int = 1024):
    out = []
    for layer in range(layers):
        out.append(MatrixSpec(width, width, f"h{layer}.attn.q"))
        out.append(MatrixSpec(width, kv_width, f"h{layer}.attn.k"))
        out.append(MatrixSpec(width, kv_width, f"h{layer}.attn.v"))
        out.append(MatrixSpec(width, width, f"h{layer}.attn.o"))
        out.append(MatrixSpec(width, 4 * width, f"h{layer}.mlp.up"))
        out.append(MatrixSpec(4 * width, width, f"h{layer}.mlp.down"))
    return out


def _stress_specs(seed: int = 5, count: int = 64):
    rng = np.random.default_rng(seed)
    sizes = np.array([512, 1024, 2048, 4096, 8192])
    rows = rng.choice(sizes, size=count)
    cols = rng.choice(sizes, size=count)
    return [MatrixSpec(int(r), int(c), f"stress{i}") for i, (r, c) in enumerate(zip(rows, cols))]


def workload(name: str, layers: int | None = None) -> Workload:
    """The named workload; `layers` truncates the layer stacks (for parity runs)."""
    if name == "single256_f32":
        return Workload(name, [MatrixSpec(256, 256, "w")], torch.float32, torch.float32,
                        PRECISION_F32, CUBIC, 5, seed=0, grad_kind="iid_all_n01", m0_zero=False)
    if name == "gpt2s_attn768_bf16":
        specs = [MatrixSpec(768, 768, f"h{i // 4}.attn.{'qkvo'[i % 4]}") for i in range(12)]
        return Workload(name, specs, torch.bfloat16, torch.bfloat16, PRECISION_BF16,
                        QUINTIC_MUON, 5, n_steps=3, seed=2, grad_std=1e-3)
    if name == "d24_bf16":
        specs = _d24_specs(24 if layers is None else layers)
        return Workload(name, specs, torch.bfloat16, torch.bfloat16, PRECISION_BF16,
                        QUINTIC_MUON, 5, seed=3, grad_kind="rank16_plus_noise")
    if name == "lm3p8b_bf16":
        specs = _lm38_specs(32 if layers is None else layers)
        return Workload(name, specs, torch.bfloat16, torch.bfloat16, PRECISION_BF16,
                        QUINTIC_MUON, 5, seed=4)
    if name == "stress_mixed_bf16":
        specs = _stress_specs()
        if layers is not None:
            specs = specs[:layers]
        return Workload(name, specs, torch.bfloat16, torch.bfloat16, PRECISION_BF16X3,
                        QUINTIC_MUON, 10, seed=5, grad_kind="studentt_spectral")
    raise KeyError(name)


WORKLOAD_NAMES = ("single256_f32", "gpt2s_attn768_bf16", "d24_bf16", "lm3p8b_bf16",
                  "stress_mixed_bf16")


def _gen(device, seed: int, idx: int, step: int, purpose: int) -> torch.Generator:
    gen = torch.Generator(device=device)
    key = ((seed & 0xFFFF) << 40) ^ ((idx & 0xFFFFF) << 16) ^ ((step & 0xFFF) << 4) ^ (purpose & 0xF)
    gen.manual_seed(key)
    return gen


def _normal(shape, device, gen, std=1.0):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _rank16_plus_noise(rows, cols, device, seed, idx, step):
    """alpha * A B^T + N with sigma_1(alpha A B^T) = 1e3 * (sqrt(rows) + sqrt(cols))."""
    rng = np.random.default_rng([seed, idx, step, 7])
    a = rng.standard_normal((rows, 16))
    b = rng.standard_normal((cols, 16))
    ra = np.linalg.qr(a, mode="r")
    rb = np.linalg.qr(b, mode="r")
    top = float(np.linalg.svd(ra @ rb.T, compute_uv=False)[0])
    alpha = 1e3 * (math.sqrt(rows) + math.sqrt(cols)) / top
    gen = _gen(device, seed, idx, step, 1)
    g = _normal((rows, cols), device, gen)
    at = torch.from_numpy((alpha * a).astype(np.float32)).to(device)
    bt = torch.from_numpy(b.astype(np.float32)).to(device)
    g.addmm_(at, bt.t())
    return g


def _studentt_spectral(rows, cols, device, seed, idx):
    """Q_u diag(i^-2) Q_v^T with Q_u, Q_v from QR of Student-t(3) matrices."""
    r = min(rows, cols)
    gen = _gen(device, seed, idx, 0, 2)

    def student_t(shape):
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        chi = torch.randn((3,) + tuple(shape), generator=gen, device=device,
                          dtype=torch.float32).square_().sum(0)
        return z / torch.sqrt(chi / 3.0)

    qu, _ = torch.linalg.qr(student_t((rows, r)))
    qv, _ = torch.linalg.qr(student_t((cols, r)))
    s = torch.arange(1, r + 1, device=device, dtype=torch.float32).pow_(-2.0)
    return (qu * s) @ qv.t().contiguous()


def spectral_factors(rows, cols, seed, idx, device="cpu"):
    """The stress gradients' construction in float64 on `device`: (Q_u, s,
    Q_v) with Q_u (rows x r) and Q_v (cols x r) the orthonormal factors (QR)
    of Student-t(3) matrices, s_i = i^-2, r = min(rows, cols); G = Q_u
    diag(s) Q_v^T.  Float64 throughout, so G has the exact i^-2 spectrum to
    float64 accuracy.  (Not the stream the stack's float32 draw takes.)"""
    r = min(rows, cols)
    gen = _gen(device, seed, idx, 0, 2)

    def student_t(shape):
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float64)
        chi = torch.randn((3,) + tuple(shape), generator=gen, device=device, dtype=torch.float64).square_().sum(0)
        return z / torch.sqrt(chi / 3.0)

    qu, _ = torch.linalg.qr(student_t((rows, r)))
    qv, _ = torch.linalg.qr(student_t((cols, r)))
    s = torch.arange(1, r + 1, device=device, dtype=torch.float64).pow_(-2.0)
    return qu, s, qv


def initial_state(wl: Workload, idx: int, device="cpu"):
    """(W, M0) for matrix `idx`: W in the parameter dtype, M0 float32."""
    spec = wl.specs[idx]
    shape = (spec.rows, spec.cols)
    if wl.grad_kind == "iid_all_n01":
        rng = np.random.default_rng(wl.seed)
        w = rng.standard_normal(shape)
        rng.standard_normal(shape)          # G is the second draw
        m = rng.standard_normal(shape)
        return (torch.from_numpy(w.astype(np.float32)).to(device),
                torch.from_numpy(m.astype(np.float32)).to(device))
    gen = _gen(device, wl.seed, idx, 0, 0)
    w = _normal(shape, device, gen, wl.w_std).to(wl.param_dtype)
    m = torch.zeros(shape, dtype=torch.float32, device=device)
    return w, m


def gradient(wl: Workload, idx: int, step: int = 0, device="cpu") -> torch.Tensor:
    """Gradient of matrix `idx` at step `step`, in the gradient dtype."""
    spec = wl.specs[idx]
    shape = (spec.rows, spec.cols)
    if wl.grad_kind == "iid_all_n01":
        rng = np.random.default_rng(wl.seed)
        rng.standard_normal(shape)
        g = rng.standard_normal(shape)
        return torch.from_numpy(g.astype(np.float32)).to(device)
    if wl.grad_kind == "gaussian":
        g = _normal(shape, device, _gen(device, wl.seed, idx, step, 1), wl.grad_std)
    elif wl.grad_kind == "rank16_plus_noise":
        g = _rank16_plus_noise(spec.rows, spec.cols, device, wl.seed, idx, step)
    elif wl.grad_kind == "studentt_spectral":
        g = _studentt_spectral(spec.rows, spec.cols, device, wl.seed, idx)
    else:
        raise KeyError(wl.grad_kind)
    return g.to(wl.grad_dtype)


def random_matrix(rows, cols, seed, dtype=torch.float32, device="cpu", std=1.0):
    """A plain seeded N(0, std^2) matrix for edge-case and shape tests."""
    gen = _gen(device, seed, rows * 131 + cols, 0, 3)
    return _normal((rows, cols), device, gen, std).to(dtype)


# ---------------------------------------------------------------- AdamW inputs

@dataclass(frozen=True)
class AdamwSpec:
    numel: int
    name: str
    group: int      # index into AdamwWorkload.lr / .wd


@dataclass
class AdamwWorkload:
    name: str
    specs: list
    param_dtype: torch.dtype
    grad_dtype: torch.dtype
    lr: tuple           # per group: head, embeddings, scalars
    wd: tuple
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    step: int = 100
    seed: int = 13

    @property
    def elements(self) -> int:
        return sum(s.numel for s in self.specs)

    def lr_per_tensor(self):
        return [self.lr[s.group] for s in self.specs]

    def wd_per_tensor(self):
        return [self.wd[s.group] for s in self.specs]


def adamw_workload(name: str = "d24_adamw_bf16", vocab: int = 32768, width: int = 1536, layers: int = 24,
                   value_embeddings: int = 12) -> AdamwWorkload:
    """The AdamW tensors of the d24 model (see the module docstring); the
    keyword arguments shrink it for parity runs.  The rates are illustrative
    (the pages give none): three groups, decay on the head only."""
    if name != "d24_adamw_bf16":
        raise KeyError(name)
    table = vocab * width
    specs = [AdamwSpec(table, "lm_head", 0), AdamwSpec(table, "wte", 1)]
    specs += [AdamwSpec(table, f"value_embed{i}", 1) for i in range(value_embeddings)]
    specs += [AdamwSpec(layers, "resid_lambdas", 2), AdamwSpec(layers, "x0_lambdas", 2)]
    return AdamwWorkload(name, specs, torch.bfloat16, torch.bfloat16, lr=(4e-3, 2e-2, 5e-3), wd=(0.1, 0.0, 0.0))


def adamw_state(wl: AdamwWorkload, idx: int, device="cpu"):
    """(p, m, v) of tensor `idx`: p in the parameter dtype, m and v float32."""
    spec = wl.specs[idx]
    gen = _gen(device, wl.seed, idx, 0, 4)
    if spec.group == 2:
        p = _normal((spec.numel,), device, gen, 0.01).add_(1.0)
    else:
        p = _normal((spec.numel,), device, gen, 0.02)
    m = _normal((spec.numel,), device, gen, 1e-3)
    v = _normal((spec.numel,), device, gen, 1e-3).square_()
    return p.to(wl.param_dtype), m, v


def adamw_gradient(wl: AdamwWorkload, idx: int, step: int = 0, device="cpu") -> torch.Tensor:
    spec = wl.specs[idx]
    return _normal((spec.numel,), device, _gen(device, wl.seed, idx, step, 5), 1e-3).to(wl.grad_dtype)
