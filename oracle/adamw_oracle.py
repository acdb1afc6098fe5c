"""Plain CPU oracle for the AdamW half of the hybrid optimizer.

TEST INFRASTRUCTURE ONLY.  Like muon_oracle, this module is the slow,
obviously-correct definition that the HIP path is checked against; only the
test-suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import it.  It shares no code with the HIP library or its binding.

Sources
-------
[P4]  "开发者千美元训3.8B模型 击败GPT-2" (aiproducthub.cn), paragraph 影响: the
      hybrid optimizer gives the matrix parameters to Muon and every other
      parameter to AdamW.
[P2]  "Karpathy 只花 $72 就訓練出 GPT-2 — 7 年前 OpenAI 花了 $43,000"
      (gu-log.vercel.app), section 那些讓 600 倍加速成為可能的技術: the model
      has learnable scalars on its residual pathways and value embeddings,
      i.e. parameters that are not projection matrices.
[KB]  D. P. Kingma and J. Ba, "Adam: A Method for Stochastic Optimization",
      ICLR 2015, Algorithm 1 (moment estimates, bias correction, the update
      m_hat / (sqrt(v_hat) + eps)).
[LH]  I. Loshchilov and F. Hutter, "Decoupled Weight Decay Regularization",
      ICLR 2019, Algorithm 2 (AdamW: the decay multiplies the weight and is
      not folded into the gradient).

The pages name AdamW and print nothing else about it.  Readings (listed with
their reasons in the design notes):

  R18 AdamW runs per element in IEEE binary32, one rounding per operation,
      no fused multiply-add, division and square root correctly rounded:
          m  <- beta1*m + c1*g            c1 = fl32(1 - beta1)
          v  <- beta2*v + c2*(g*g)        c2 = fl32(1 - beta2)
          mh =  m / bc1                   bc1 = fl32(1 - beta1^t)
          vh =  v / bc2                   bc2 = fl32(1 - beta2^t)
          u  =  mh / (sqrt(vh) + eps)
          p  <- rnd(fl32(p*d) - fl32(lr*u))   d = fl32(1 - fl32(lr*wd))
      beta^t is taken in binary64 (the C library's pow) from the binary32
      beta and the step number t >= 1; m and v are binary32 buffers; p is
      rounded to its storage type (bfloat16 to nearest-even) at the end.
"""
from __future__ import annotations

import math

import numpy as np

from .muon_oracle import to_bf16


def adamw_constants(beta1: float, beta2: float, step: int):
    """(c1, c2, bc1, bc2) of R18 as binary32 values."""
    if step < 1:
        raise ValueError("the step number t starts at 1")
    b1 = np.float32(beta1)
    b2 = np.float32(beta2)
    c1 = np.float32(1.0) - b1
    c2 = np.float32(1.0) - b2
    bc1 = np.float32(1.0 - math.pow(float(b1), step))
    bc2 = np.float32(1.0 - math.pow(float(b2), step))
    return c1, c2, bc1, bc2


def adamw(p, g, m, v, *, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
          step: int, param_bf16: bool = False):
    """One AdamW step ([KB] Algorithm 1 with [LH]'s decoupled decay; R18).

    p: weights (float32, or bf16 values held in float32); g: gradient (bf16
    values in float32, or float32); m, v: float32 moment buffers.
    Returns (p_new, m_new, v_new) as float32 arrays.  numpy float32
    arithmetic rounds every operation once to nearest-even (sqrt and
    division included) and never fuses.
    """
    p = np.asarray(p, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    b1 = np.float32(beta1)
    b2 = np.float32(beta2)
    c1, c2, bc1, bc2 = adamw_constants(beta1, beta2, step)
    lr32 = np.float32(lr)
    e32 = np.float32(eps)

    # first and second moment estimates
    m_new = (b1 * m) + (c1 * g)
    v_new = (b2 * v) + (c2 * (g * g))
    # bias-corrected estimates and the update direction
    m_hat = m_new / bc1
    v_hat = v_new / bc2
    u = m_hat / (np.sqrt(v_hat) + e32)
    # decoupled weight decay, then the step
    d = np.float32(1.0) - (lr32 * np.float32(weight_decay))
    p_new = (p * d) - (lr32 * u)
    if param_bf16:
        p_new = to_bf16(p_new)
    return p_new.astype(np.float32), m_new.astype(np.float32), v_new.astype(np.float32)
