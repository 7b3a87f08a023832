"""Length-head oracle -- TEST INFRASTRUCTURE ONLY.

A plain float64 reference for the adaptive length head, in numpy.  Only the
tests, the package smoke check and the benchmark's CPU-baseline leg may import
it; it shares nothing with the GPU library and never imports it.

Sources (pages as titled; citations name the section or algorithm):
  * "AdaFlash：基于在策略蒸馏扩散草稿器的自适应投机解码" (review, ZH), section 2.2
    "Adaptive Length Head": per-position linear projection and SiLU, mean over
    the k positions of the block, linear layer and sigmoid giving the predicted
    accept rate a_hat; verify length k_hat = clamp(floor(gamma a_hat k), 1, k);
    online loss (a_hat - a*)^2 with a* the accepted count over the candidate
    length; the drafter is detached (no gradient into the hidden states).
  * "AdaFlash: Taming Variance in Diffusion Speculative Decoding" (review, EN),
    Algorithm 3 "Adaptive Length Head, Forward Pass" (the same steps, gamma as
    a rescaling of a_hat before the floor) and "Online Update of the Length
    Head, Derived" (a* = fraction of the verified tokens that were accepted).

Readings where the pages leave a step open (each is listed in the design doc):
  * The label is a* = A / L with L the verify length actually used (the
    tokens sent to the target) and A the accepted count among them.
  * The squared error is taken on the sigmoid output before gamma: gamma is a
    serving-time scale applied only to form k_hat.
  * The projection width H' and the weights are free parameters (synthetic
    here); the second layer maps H' to one logit with a bias.
  * Gradients are of the SUM of the per-request losses over the batch, with
    respect to the head parameters only (W1, b1, w2, b2).

Every step is a plain array operation in float64 (one library matmul for the
projection and one for the weight gradient), in the order the pages give.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _silu(x):
    return x * _sigmoid(x)


def forward(h: np.ndarray, W1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: float, gamma: float) -> dict:
    """Algorithm 3 of the EN review / section 2.2 of the ZH review.

    h: [B, k, H] hidden states; W1: [H', H]; b1: [H']; w2: [H']; b2 scalar.
    Returns z1 [B, k, H'] (pre-activation), hbar [B, H'], s [B] (logit),
    a_hat [B] (sigmoid output), k_hat [B] (int)."""
    h = np.asarray(h, np.float64)
    W1 = np.asarray(W1, np.float64)
    b1 = np.asarray(b1, np.float64)
    w2 = np.asarray(w2, np.float64)
    B, k, H = h.shape
    # Step 1: per-position projection and SiLU, h'_i = SiLU(W1 h_i + b1).
    z1 = h @ W1.T + b1
    hp = _silu(z1)
    # Step 2: mean over the k positions of the block.
    hbar = hp.mean(axis=1)
    # Step 3: linear layer to one logit and sigmoid: predicted accept rate.
    s = hbar @ w2 + float(b2)
    a_hat = _sigmoid(s)
    # Steps 4-5: k_hat = clamp(floor(gamma * a_hat * k), 1, k).
    k_hat = np.clip(np.floor(gamma * a_hat * k), 1, k).astype(np.int64)
    return {"z1": z1, "hbar": hbar, "s": s, "a_hat": a_hat, "k_hat": k_hat}


def label(accept_len: np.ndarray, verify_len: np.ndarray) -> np.ndarray:
    """a* = accepted count / verified length (EN review, online update)."""
    return np.asarray(accept_len, np.float64) / np.asarray(verify_len, np.float64)


def loss_backward(h, W1, b1, w2, b2, accept_len, verify_len) -> dict:
    """Per-request loss (a_hat - a*)^2 and the gradient of its sum over the
    batch with respect to W1, b1, w2, b2 (chain rule; the pages print no
    gradient).  The hidden states get no gradient (drafter detached)."""
    f = forward(h, W1, b1, w2, b2, 1.0)
    h = np.asarray(h, np.float64)
    w2 = np.asarray(w2, np.float64)
    B, k, H = h.shape
    a_star = label(accept_len, verify_len)
    a = f["a_hat"]
    loss = (a - a_star) ** 2
    ds = 2.0 * (a - a_star) * a * (1.0 - a)                  # d loss / d s
    dw2 = f["hbar"].T @ ds                                     # [H']
    db2 = ds.sum()
    dhbar = ds[:, None] * w2[None, :]                          # [B, H']
    z1 = f["z1"]
    sg = _sigmoid(z1)
    dsilu = sg * (1.0 + z1 * (1.0 - sg))                       # SiLU'(z)
    dz1 = (dhbar[:, None, :] / k) * dsilu                      # [B, k, H']
    dz1m = dz1.reshape(B * k, -1)
    dW1 = dz1m.T @ h.reshape(B * k, H)                         # [H', H]
    db1 = dz1m.sum(axis=0)
    return {"loss": loss, "a_hat": a, "a_star": a_star, "dW1": dW1, "db1": db1, "dw2": dw2, "db2": db2}
