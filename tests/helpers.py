"""Shared helpers for the GPU parity tests: device transfer, running the
library through its C ABI binding, and comparing against the oracle."""
from __future__ import annotations

import numpy as np

NEAR_TIE = 1e-5   # |p - u q| band for accept tests; relative band for draws


def to_dev(a: np.ndarray, bf16: bool):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if bf16 else a))
    if bf16:
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def gpu_verify(bt, T, opd=False, clip_c=10.0, lam=1.0, verify_len=None, tokens=None, grad_rows=None):
    """Runs adaflash_verify on the batch; returns numpy outputs.  Only the
    gradient rows in ``grad_rows`` (default: all written rows) are copied back."""
    import torch
    import diffusion_drafter_verification_amd as ada
    bf16 = bt.target.dtype == np.uint16
    t = to_dev(bt.target, bf16)
    d = to_dev(bt.draft, bf16) if bt.draft is not None else None
    tok = torch.from_numpy(bt.tokens if tokens is None else tokens).to("cuda")
    vl = torch.from_numpy(bt.verify_len if verify_len is None else verify_len).to("cuda")
    uni = torch.from_numpy(bt.uniforms).to("cuda")
    out = ada.verify(t, d, tok, vl, uni, T=T, opd=opd, clip_c=clip_c, lam=lam)
    torch.cuda.synchronize()
    grad = out.pop("grad")
    res = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    res["grad"] = None
    if grad is not None:
        N = int(res["row_offsets"][-1])
        sel = torch.arange(N, device="cuda") if grad_rows is None else torch.as_tensor(
            np.asarray(grad_rows), device="cuda")
        res["grad_rows"] = sel.cpu().numpy()
        res["grad"] = grad[sel].float().cpu().numpy()
    return res


def gpu_opd(target, draft, verify_len, clip_c, lam, grad_rows=None):
    """Runs adaflash_opd_loss_fwd_bwd; copies back only ``grad_rows`` of the gradient."""
    import torch
    import diffusion_drafter_verification_amd as ada
    bf16 = target.dtype == np.uint16
    t = to_dev(target, bf16)
    d = to_dev(draft, bf16)
    vl = None if verify_len is None else torch.from_numpy(verify_len).to("cuda")
    out = ada.opd_loss_fwd_bwd(t, d, vl, clip_c=clip_c, lam=lam)
    torch.cuda.synchronize()
    grad = out.pop("grad")
    res = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    N = int(res["row_offsets"][-1])
    sel = torch.arange(N, device="cuda") if grad_rows is None else torch.as_tensor(
        np.asarray(grad_rows), device="cuda")
    res["grad"] = grad[sel].float().cpu().numpy()
    return res


def compare_verify(g, r, T, tokens, verify_len, k):
    """Exact comparison of accept lengths and emitted tokens; in sampled mode a
    difference is allowed only where the oracle puts the deciding quantity
    inside the near-tie band.  Returns (n_requests, n_in_band, n_flips)."""
    A_g, A_r = g["accept_len"], r["accept_len"]
    tok_g, tok_r = g["out_tokens"], r["out_tokens"]
    B = A_r.shape[0]
    if T == 0:
        assert np.array_equal(A_g, A_r), np.nonzero(A_g != A_r)[0][:10]
        assert np.array_equal(tok_g, tok_r)
        return B, 0, 0
    mr = r["margins"]
    L = np.clip(verify_len, 1, k)
    in_band = 0
    flips = 0
    for b in range(B):
        near_acc = np.abs(mr[b, :L[b]]) < NEAR_TIE
        near_draw = mr[b, k] < NEAR_TIE
        if near_acc[: min(A_r[b], A_g[b]) + 1].any() or near_draw:
            in_band += 1
        same = A_g[b] == A_r[b] and np.array_equal(tok_g[b], tok_r[b])
        if same:
            continue
        flips += 1
        a = min(A_g[b], A_r[b])
        if A_g[b] != A_r[b]:
            assert near_acc[a], f"request {b}: accept length {A_g[b]} vs oracle {A_r[b]}, margin {mr[b, a]}"
        else:
            assert near_draw, (f"request {b}: token {tok_g[b, a]} vs oracle {tok_r[b, a]} "
                               f"(draw margin {mr[b, k]})")
    # The structure holds regardless.
    for b in range(B):
        a = A_g[b]
        assert 0 <= a <= L[b]
        assert np.array_equal(tok_g[b, :a], tokens[b, :a])
        assert (tok_g[b, a + 1:] == -1).all()
    return B, in_band, flips


def compare_margins(g, r, verify_len, k, T):
    if T == 0:
        assert np.isnan(g["margins"]).all()
        return
    L = np.clip(verify_len, 1, k)
    for b in range(g["margins"].shape[0]):
        m_g = g["margins"][b, :L[b]].astype(np.float64)
        m_r = r["margins"][b, :L[b]]
        assert np.abs(m_g - m_r).max() < 2e-6, (b, m_g, m_r)
        assert np.isnan(g["margins"][b, L[b]:k]).all()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _loss_excess(g, r):
    """Error beyond 1e-3 relative + 1e-6 absolute; equal infinities match."""
    g = g.astype(np.float64)
    same_inf = np.isinf(r) & (g == r)
    with np.errstate(invalid="ignore"):
        e = np.abs(g - r) - (1e-3 * np.abs(r) + 1e-6)
    e = np.where(same_inf, -1.0, e)
    return np.where(np.isnan(e), np.inf, e)


def compare_losses(ce_g, rk_g, ce_r, rk_r):
    e1 = _loss_excess(ce_g, ce_r)
    e2 = _loss_excess(rk_g, rk_r)
    assert (e1 <= 0).all(), (np.argmax(e1), ce_g[np.argmax(e1)], ce_r[np.argmax(e1)])
    assert (e2 <= 0).all(), (np.argmax(e2), rk_g[np.argmax(e2)], rk_r[np.argmax(e2)])


def compare_grad(g_gpu, g_ref, bf16=True):
    """2e-3 absolute, or one bf16 ulp of the reference where that is larger."""
    err = np.abs(g_gpu.astype(np.float64) - g_ref)
    tol = np.maximum(2e-3, bf16_ulp(g_ref)) if bf16 else 2e-5 + 1e-5 * np.abs(g_ref)
    bad = err > tol
    assert not bad.any(), (np.argwhere(bad)[:5], err.max())
    assert abs(float(g_ref.sum())) < 1e-9 * g_ref.shape[-1] + 1e-9
    return int((np.abs(g_ref) >= 0.5).sum())
