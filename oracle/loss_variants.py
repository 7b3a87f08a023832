"""Supervision-loss variants oracle -- TEST INFRASTRUCTURE ONLY.

Plain float64 numpy reference for the per-row losses the pages compare, and
their gradients with respect to the draft logits.  Only the tests, the package
smoke check and the benchmark's CPU-baseline leg may import it; it shares
nothing with the GPU library and never imports it.

Sources (pages as titled; citations name the section, equation or table):
  * "AdaFlash: Taming Variance in Diffusion Speculative Decoding" (review, EN),
    "Forward KL vs. Reverse KL" (the two divergences; forward KL is the OSD
    baseline's objective), "The Reverse-KL + Hard-Label Mixture Loss,
    Derived", "Entry-Wise Divergence Clipping, Derived", and the ablation
    Table 2 (rows: plain reverse KL; with entry-wise clipping; with the
    mixture).
  * "AdaFlash：基于在策略蒸馏扩散草稿器的自适应投机解码" (review, ZH), section 2.1:
    l_OPD = alpha l_hard + (1 - alpha) l_rkl^clip, alpha = 0.8, delta = 0.01.
  * "DFlash 阅读笔记：并行起草、目标特征与精确验证" (DFlash notes), section 7.3,
    eq. 12: cross entropy weighted by exp(-(k-1)/lambda) for the k-th predicted
    position of a block (lambda = 7 at block size 16).

Per row (p = softmax(z_p), q = softmax(z_q) at temperature 1, x* = argmax z_p
with the lowest index on ties):
  CE   = -log q(x*)                                  (hard label, l_hard)
  R_c  = sum_v min(q_v log(q_v / p_v), c)            (c = inf: plain reverse KL)
  FKL  = sum_v p_v log(p_v / q_v)
Variants (w = 1 unless stated):
  rkl       loss = R_inf
  rkl_clip  loss = R_delta
  mixture   loss = alpha CE + (1 - alpha) R_delta
  fkl       loss = FKL
  wce       loss = w_i CE, w_i = exp(-i / lam) for draft position i = 0, 1, ...
            (the first predicted position has weight 1)
Gradients (chain rule; the pages print none), with f_v = q_v (log q_v - log p_v):
  d CE / d z_v  = q_v - [v == x*]
  d R_c / d z_v = q_v ([f_v <= c](log q_v - log p_v + 1) - S),
                  S = sum_{f_w <= c} (f_w + q_w)
  d FKL / d z_v = q_v - p_v
Conventions as in the main oracle: a term with q_v = 0 is 0; p_v = 0 < q_v
gives +inf (always clipped).
"""
from __future__ import annotations

import numpy as np

VARIANTS = ("rkl", "rkl_clip", "mixture", "fkl", "wce")


def _softmax_log(z):
    z = np.asarray(z, np.float64)
    m = np.max(z)
    lse = m + np.log(np.sum(np.exp(z - m)))
    return np.exp(z - lse), z - lse


def row_terms(zp, zq, c):
    """CE, R_c, FKL of one row and their gradients with respect to z_q."""
    p, lp = _softmax_log(zp)
    q, lq = _softmax_log(zq)
    xs = int(np.argmax(zp))  # numpy's argmax takes the lowest index on ties
    ce = -lq[xs]
    with np.errstate(divide="ignore", invalid="ignore"):
        f = np.where(q > 0, q * (lq - lp), 0.0)
    inU = f <= c
    R = float(np.sum(np.where(inU, f, c)))
    S = float(np.sum(np.where(inU, f + q, 0.0)))
    with np.errstate(invalid="ignore"):
        gR = q * (np.where(inU, lq - lp + 1.0, 0.0) - S)
    gR = np.where(q > 0, gR, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        fk = np.where(p > 0, p * (lp - lq), 0.0)
    fkl = float(np.sum(fk))
    gce = q.copy()
    gce[xs] -= 1.0
    return {"ce": ce, "R": R, "fkl": fkl, "g_ce": gce, "g_R": gR, "g_fkl": q - p, "xstar": xs}


def variant_row(zp, zq, variant, i, p1=0.0, p2=0.0):
    """Loss and gradient of one row for `variant` (see the module docstring)."""
    if variant == "rkl":
        t = row_terms(zp, zq, np.inf)
        return t["R"], t["g_R"]
    if variant == "rkl_clip":
        t = row_terms(zp, zq, p1)
        return t["R"], t["g_R"]
    if variant == "mixture":
        a, d = p1, p2
        t = row_terms(zp, zq, d)
        return a * t["ce"] + (1 - a) * t["R"], a * t["g_ce"] + (1 - a) * t["g_R"]
    if variant == "fkl":
        t = row_terms(zp, zq, np.inf)
        return t["fkl"], t["g_fkl"]
    if variant == "wce":
        w = np.exp(-i / p1)
        t = row_terms(zp, zq, np.inf)
        return w * t["ce"], w * t["g_ce"]
    raise ValueError(variant)


def batch(target, draft, verify_len, variant, p1=0.0, p2=0.0):
    """All verified rows of a batch, packed in request order (row n = the
    i-th draft position of request b, i < L_b).  target [B, k+1, V] and draft
    [B, k, V] as float64 logits (convert bf16 first).  Returns loss [N],
    grad [N, V]."""
    B, k1, V = target.shape
    k = k1 - 1
    L = np.full(B, k) if verify_len is None else np.clip(np.asarray(verify_len), 1, k)
    losses, grads = [], []
    for b in range(B):
        for i in range(int(L[b])):
            l, g = variant_row(target[b, i], draft[b, i], variant, i, p1, p2)
            losses.append(l)
            grads.append(g)
    return np.array(losses), np.array(grads).reshape(len(losses), V)
