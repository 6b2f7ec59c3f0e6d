"""CPU oracle for the transformer-block pipeline around the quantized LoRA
linear (TEST INFRASTRUCTURE ONLY, like the rest of this package).

Sources: nlp-lineage milestone page on QLoRA, "The idea" (adapters must go on
every linear layer of each Transformer block; only L1 and L2 get weight
gradients); inferensys glossary entry "QLoRA", frozen-base paragraph (the 4-bit
base is never updated and the optimizer keeps momentum and variance for the
adapters only).

Readings:
  * Linears that read the same input (q, k, v; gate, up) may be stacked along
    the output dimension into one quantized matrix of G segments.  Each keeps
    its own adapter (L1_g, L2_g) and its own rounding points, so the stacked
    forward is exactly the concatenation of the separate forwards.  In the
    backward the input gradient is the sum over segments, rounded once:
    dX = bf16(sum_g (dY_g W'_g + G_g L1_g^T)).
  * The optimizer is AdamW (decoupled weight decay) over the adapters only,
    on fp32 master copies whose bf16 rounding is what the layer multiplies
    with:  theta <- theta (1 - lr wd);  m <- b1 m + (1 - b1) g;
    v <- b2 v + (1 - b2) g^2;  theta <- theta - lr (m / (1 - b1^t)) /
    (sqrt(v / (1 - b2^t)) + eps).
"""
from __future__ import annotations

import numpy as np

from .qlora_oracle import _f64, bf16_bits, qlora_backward, qlora_forward


def qlora_group_forward(X, Wq_list, L1_list, L2_list, lora_scale: float = 1.0):
    """Stacked forward of G linears sharing X: Y_cat = [Y_0 | ... | Y_{G-1}]
    (bf16 bits [M, G N]) and the list of T_g."""
    Ys, Ts = [], []
    for Wq, L1, L2 in zip(Wq_list, L1_list, L2_list):
        Y, T = qlora_forward(X, Wq, L1, L2, lora_scale)
        Ys.append(Y)
        Ts.append(T)
    return np.concatenate(Ys, axis=1), Ts


def qlora_group_backward(X, dY_cat, Wq_list, L1_list, L2_list, lora_scale: float = 1.0, T_list=None):
    """Backward of the stacked linears: (dX, [dL1_g], [dL2_g], [G_g]).  Each
    segment's adapter gradients are those of the separate layer; dX is the
    float64 sum of the segments' unrounded input gradients, rounded once."""
    G = len(Wq_list)
    N = np.asarray(dY_cat).shape[1] // G
    ident = lambda x: np.asarray(x, np.float64)
    dX_sum, dL1s, dL2s, Gs = 0.0, [], [], []
    for g in range(G):
        dYg = np.asarray(dY_cat)[:, g * N:(g + 1) * N]
        T = None if T_list is None else T_list[g]
        # adapter gradients and G_g with the layer's own rounding points
        _, dL1, dL2, Gg, _ = qlora_backward(X, dYg, Wq_list[g], L1_list[g], L2_list[g], lora_scale, T=T,
                                            compute_dx=False)
        dX_sum = dX_sum + _f64(dYg) @ _f64(Wq_list[g]) + _f64(Gg) @ _f64(L1_list[g]).T
        dL1s.append(dL1)
        dL2s.append(dL2)
        Gs.append(Gg)
    return bf16_bits(dX_sum), dL1s, dL2s, Gs


def adamw_step(theta, m, v, grad, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
               step: int):
    """One AdamW step in float64 from the given (fp32) state.  Returns
    (theta, m, v) as float64 arrays; the caller compares them with the fp32
    state the device keeps."""
    theta, m, v, g = (np.asarray(a, np.float64) for a in (theta, m, v, grad))
    theta = theta * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    theta = theta - lr * m_hat / (np.sqrt(v_hat) + eps)
    return theta, m, v
