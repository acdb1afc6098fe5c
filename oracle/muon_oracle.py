"""Plain CPU oracle for one Muon optimizer step on 2-D weight matrices.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the HIP path is checked against.  Only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library or its Python binding and
imports nothing from them; the only thing both sides share is the seeded
input generator module, which holds none of the method's arithmetic.

Sources
-------
[P3]  "把 GPT-2 的训练租金估算从 4.3 万美元压到 40 美元：nanochat「time-to-GPT-2」
      排行榜背后的成本算术与工程堆栈" (magicnetworld.com), table 符号与约定,
      row "Muon": Muon is an optimizer for matrix-shaped parameters that
      orthogonalises the momentum.
[P4]  "开发者千美元训3.8B模型 击败GPT-2" (aiproducthub.cn), paragraph 影响:
      Muon orthogonalises the matrix parameters' update with Newton-Schulz;
      every other parameter goes to AdamW.
[H]   N. J. Higham, *Functions of Matrices*, SIAM 2008, ch. 8 (the polar
      decomposition and its Newton-Schulz iteration).  The pages name the
      iteration but print no formula; the odd-polynomial form used here,
      X <- a X + (b A + c A^2) X with A = X X^T, is the general polynomial
      Newton-Schulz step of which the textbook cubic (3/2, -1/2, 0) and
      quintic (15/8, -5/4, 3/8) are special cases.

Where the pages are silent the plainest reading is taken; each reading is
named R<n> below and listed with its reason in the design notes.

  R1  momentum is the heavy-ball buffer M <- beta*M + g (no dampening).
  R2  Nesterov uses the updated buffer: U = g + beta*M_new.
  R3  momentum runs in IEEE binary32, one rounding per operation, no fused
      multiply-add; beta enters as its binary32 value.
  R4  normalisation X0 = U / (||U||_F + eps) with eps = 1e-7, in float64.
  R5  a matrix with rows > cols is iterated on its transpose, so that the
      Gram matrix X X^T is the smaller side; the result is transposed back.
  R6  the write-back is W <- W - t*O with t = fl32(lr * s), s from the scale
      rule, each operation rounded to binary32, then to the parameter dtype
      (bfloat16 round-to-nearest-even).
  R7  scale rules: NONE s = 1; SQRT_ASPECT s = sqrt(max(1, rows/cols));
      RMS_MATCH s = 0.2*sqrt(max(rows, cols)).

Update variants (the pages describe none of them; they are the forms
commonly used with Muon, offered as options):
  R14 EMA momentum: M <- beta*M + (1-beta)*g, with (1-beta) rounded to
      binary32 and each product and sum rounded once; its Nesterov
      direction is U = (1-beta)*g + beta*M_new.
  R15 a Newton-Schulz schedule: step k uses its own triple (a_k, b_k, c_k).
  R16 decoupled weight decay: W <- rnd(fl32(fl32(W*d) - fl32(t*O))) with
      d = fl32(1 - fl32(lr*wd)); wd = 0 gives d = 1 and R6 exactly.
  R17 a per-matrix learning rate and a per-matrix scale s replace lr and the
      scale rule of R6/R7 for that matrix.

Parity of every function here is pinned by tests/test_oracle_pins.py
against closed forms, invariants, exact rational arithmetic and LAPACK; see
that file for which pin covers which function.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

EPS = 1e-7

SCALE_NONE = 0
SCALE_SQRT_ASPECT = 1
SCALE_RMS_MATCH = 2


# ---------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even) on binary32 values
# ---------------------------------------------------------------------------

def to_bf16(x) -> np.ndarray:
    """Round to bfloat16 (RNE) and return the values as float32.

    Float64 input is first rounded to binary32 (the GPU rounds its binary32
    accumulators), then the low 16 bits of the binary32 pattern are rounded
    away with ties to even.  NaN stays NaN; overflow rounds to +-inf as IEEE
    round-to-nearest prescribes.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(f)
    if np.any(nan):
        out = np.where(nan, np.float32(np.nan), out)
    return out.reshape(f.shape)


def split_bf16x2(x) -> tuple[np.ndarray, np.ndarray]:
    """Split binary32 values into hi = bf16(x) and lo = bf16(x - hi)."""
    f = np.asarray(x, dtype=np.float32)
    hi = to_bf16(f)
    lo = to_bf16(f - hi)          # binary32 subtraction, exact (Sterbenz)
    return hi, lo


# ---------------------------------------------------------------------------
# the step, one stage at a time
# ---------------------------------------------------------------------------

MOMENTUM_HEAVY_BALL = 0
MOMENTUM_EMA = 1


def momentum(m, g, beta: float, nesterov: bool, kind: int = MOMENTUM_HEAVY_BALL):
    """Momentum buffer update and the update direction U ([P3]; R1-R3, R14).

    m: float32 buffer, g: gradient (bf16 values held in float32, or float32).
    Returns (m_new, u), both float32.  numpy float32 arithmetic rounds each
    operation once to nearest-even and never fuses, which is R3 exactly.
    """
    m = np.asarray(m, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    b = np.float32(beta)
    if kind == MOMENTUM_HEAVY_BALL:
        gin = g
    elif kind == MOMENTUM_EMA:
        gin = (np.float32(1.0) - b) * g
    else:
        raise ValueError(f"unknown momentum kind {kind}")
    m_new = (b * m) + gin
    if nesterov:
        u = gin + (b * m_new)
    else:
        u = m_new.copy()
    return m_new, u


def frobenius_norm(u) -> float:
    """||U||_F = sqrt(sum of squares), summed in float64 ([P3] 'orthogonalised';
    the Frobenius scaling bounds every singular value by 1 so the iteration
    converges, [H] ch. 8)."""
    v = np.asarray(u, dtype=np.float64)
    return float(math.sqrt(float(np.sum(v * v))))


def normalise(u, eps: float = EPS) -> np.ndarray:
    """X0 = U / (||U||_F + eps) in float64 (R4)."""
    v = np.asarray(u, dtype=np.float64)
    return v / (frobenius_norm(v) + eps)


def orient(x):
    """R5: return (x_wide, transposed) with x_wide having rows <= cols."""
    x = np.asarray(x)
    if x.shape[0] > x.shape[1]:
        return x.T, True
    return x, False


def schedule(coeffs, steps: int) -> list:
    """The triple of each of `steps` steps: one triple for all (a, b, c), or a
    sequence of `steps` triples (R15)."""
    c = np.asarray(coeffs, dtype=np.float64)
    if c.shape == (3,):
        return [tuple(float(v) for v in c)] * steps
    if c.shape != (steps, 3):
        raise ValueError(f"a schedule needs {steps} triples, got shape {c.shape}")
    return [tuple(float(v) for v in row) for row in c]


def newton_schulz(x0, coeffs, steps: int) -> np.ndarray:
    """`steps` polynomial Newton-Schulz steps on a wide float64 matrix ([P4], [H]).

    Each step forms the Gram matrix A = X X^T, the polynomial B = b A + c A A
    and the new iterate X <- a X + B X.  All in float64.  `coeffs` is one
    triple or a schedule of `steps` triples (R15).
    """
    x = np.array(x0, dtype=np.float64)
    for a, b, c in schedule(coeffs, steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x


def orthogonalise(u, coeffs, steps: int, eps: float = EPS) -> np.ndarray:
    """O = NS^steps(U / (||U||_F + eps)), oriented per R5 and transposed back."""
    xw, tr = orient(np.asarray(u, dtype=np.float64))
    o = newton_schulz(normalise(xw, eps), coeffs, steps)
    return o.T if tr else o


def scale_factor(rule: int, rows: int, cols: int) -> float:
    """Per-matrix update scale s (R7)."""
    if rule == SCALE_NONE:
        return 1.0
    if rule == SCALE_SQRT_ASPECT:
        return math.sqrt(max(1.0, rows / cols))
    if rule == SCALE_RMS_MATCH:
        return 0.2 * math.sqrt(max(rows, cols))
    raise ValueError(f"unknown scale rule {rule}")


def write_back(w, o, lr: float, s: float, param_bf16: bool, weight_decay: float = 0.0) -> np.ndarray:
    """W <- rnd(fl32(fl32(W*d) - fl32(t*O))) with t = fl32(lr*s) and
    d = fl32(1 - fl32(lr*wd)) (R6, R16; wd = 0 leaves W*d = W exactly).

    o is rounded to binary32 first (the update leaves the GPU's epilogue in
    binary32); returns float32 values (bf16-representable when param_bf16).
    """
    t = np.float32(np.float64(lr) * np.float64(s))
    w32 = np.asarray(w, dtype=np.float32)
    o32 = np.asarray(o, dtype=np.float32)
    if weight_decay != 0.0:
        d = np.float32(1.0) - np.float32(np.float32(lr) * np.float32(weight_decay))
        w32 = w32 * d
    out = w32 - (t * o32)
    return to_bf16(out) if param_bf16 else out


# ---------------------------------------------------------------------------
# the whole step
# ---------------------------------------------------------------------------

@dataclass
class StepResult:
    w: np.ndarray      # new weight (float32 values; bf16-representable for bf16 params)
    m: np.ndarray      # new momentum buffer (float32)
    o: np.ndarray      # orthogonalised update O, rows x cols, float64
    u: np.ndarray      # update direction U (float32)


def muon_step(w, g, m, *, lr, beta, nesterov, coeffs, steps, scale_rule=SCALE_NONE,
              param_bf16=False, eps=EPS, storage="fp64", momentum_kind=MOMENTUM_HEAVY_BALL,
              weight_decay=0.0, scale=None) -> StepResult:
    """One Muon step on one matrix: momentum, normalise, Newton-Schulz, write-back.

    storage="fp64" is the reference definition.  storage="bf16" evaluates the
    same step with the intermediates rounded where a bf16 GPU path stores
    them (see `orthogonalise_bf16_storage`); it is an aid for separating the
    bf16 storage error from other error, not a different method.
    Variants: momentum_kind (R14), a schedule in `coeffs` (R15), weight_decay
    (R16), and `scale` replacing the scale rule (R17; `lr` is per matrix
    already, one matrix per call).
    """
    m_new, u = momentum(m, g, beta, nesterov, momentum_kind)
    if storage == "fp64":
        o = orthogonalise(u, coeffs, steps, eps)
    elif storage == "bf16":
        o = orthogonalise_bf16_storage(u, coeffs, steps, eps)
    else:
        raise ValueError(storage)
    rows, cols = np.asarray(w).shape
    s = scale_factor(scale_rule, rows, cols) if scale is None else float(scale)
    w_new = write_back(w, o, lr, s, param_bf16, weight_decay)
    return StepResult(w=w_new, m=m_new, o=o, u=u)


def orthogonalise_bf16_storage(u, coeffs, steps: int, eps: float = EPS, rnd=None) -> np.ndarray:
    """The same map as `orthogonalise`, with bf16 rounding at the storage points.

    A bf16 GPU path cannot keep its intermediates in float64; it stores
    them in bfloat16 between the matrix products and accumulates each
    product in binary32.  The storage points, in order:

      1. U (before scaling) is stored; 1/(||U||_F + eps) is applied later as
         a scalar s, with ||U||_F taken from the binary32 U.
      2. With G = s^2 X X^T (s on the first step, 1 afterwards):
         c != 0: A = G is stored, then B = b A + c A A is stored;
         c == 0: B = b G is stored.
      3. X_new = s (a X + B X) is stored, except after the last step, whose
         value is the update O.  a X is added in full precision.

    All arithmetic between the storage points is float64 here, so the
    result differs from a binary32-accumulating GPU only by accumulation
    rounding, which is far below the bf16 storage error.  `rnd` replaces
    the rounding function (default `to_bf16`); with the identity it must
    reduce to `orthogonalise`.
    """
    if rnd is None:
        rnd = to_bf16
    triples = schedule(coeffs, steps)
    u32 = np.asarray(u, dtype=np.float32)
    xw, tr = orient(u32)
    inv = 1.0 / (frobenius_norm(u32) + eps)
    x = np.asarray(rnd(xw), dtype=np.float64)
    s = inv
    if steps == 0:
        o = s * x
        return o.T if tr else o
    for k in range(steps):
        a, b, c = triples[k]
        gram = (s * s) * (x @ x.T)
        if c != 0.0:
            a_st = np.asarray(rnd(gram), dtype=np.float64)
            b_st = np.asarray(rnd(b * a_st + c * (a_st @ a_st)), dtype=np.float64)
        else:
            b_st = np.asarray(rnd(b * gram), dtype=np.float64)
        xn = s * (a * x + b_st @ x)
        s = 1.0
        x = xn if k == steps - 1 else np.asarray(rnd(xn), dtype=np.float64)
    return x.T if tr else x


# ---------------------------------------------------------------------------
# reference quantities used by the parity gates
# ---------------------------------------------------------------------------

def polar_factor(g) -> np.ndarray:
    """The orthogonal polar factor U V^T of G = U S V^T (LAPACK SVD)."""
    uu, _, vt = np.linalg.svd(np.asarray(g, dtype=np.float64), full_matrices=False)
    return uu @ vt


def rel_frobenius(x, ref) -> float:
    """||x - ref||_F / ||ref||_F in float64 (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


def nominal_ns_flops(rows: int, cols: int, steps: int, c_nonzero: bool = True) -> float:
    """Nominal Newton-Schulz FLOPs: per step 4 m^2 n + 2 m^3 (m <= n), 4 m^2 n when c == 0."""
    m, n = min(rows, cols), max(rows, cols)
    per = 4.0 * m * m * n + (2.0 * m ** 3 if c_nonzero else 0.0)
    return per * steps
