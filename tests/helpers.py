"""Shared helpers for the GPU parity tests: device transfer, running the
library through its C ABI binding, and comparing against the oracle."""
from __future__ import annotations

import numpy as np

from parity import grad_tolerance, loss_excess, loss_rel_error, margin_error, verify_counts


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
    difference is allowed only inside the relative near-tie band of the accept
    test where the two decisions part, or the draw band (tests/parity.py).
    Returns the counts (requests, in_abs_band, in_rel_band, near_draw, flips)."""
    return verify_counts(g, r, T, tokens, verify_len, k)


def compare_margins(g, r, verify_len, k, T):
    """GPU accept-test margins p(x) - u q(x) against the oracle's (2e-6
    absolute: fp32 probabilities); NaN past the verify length and in greedy mode."""
    if T == 0:
        assert np.isnan(g["margins"]).all()
        return 0.0
    worst = margin_error(g["margins"], r["margins"], verify_len, k)
    assert worst < 2e-6, worst
    return worst


def compare_losses(ce_g, rk_g, ce_r, rk_r):
    e1 = loss_excess(ce_g, ce_r)
    e2 = loss_excess(rk_g, rk_r)
    assert (e1 <= 0).all(), (np.argmax(e1), ce_g[np.argmax(e1)], ce_r[np.argmax(e1)])
    assert (e2 <= 0).all(), (np.argmax(e2), rk_g[np.argmax(e2)], rk_r[np.argmax(e2)])
    return max(loss_rel_error(ce_g, ce_r), loss_rel_error(rk_g, rk_r))


def compare_grad(g_gpu, g_ref, bf16=True):
    """2e-3 absolute, or one bf16 ulp of the reference where that is larger.
    Returns the largest absolute error."""
    err = np.abs(g_gpu.astype(np.float64) - g_ref)
    bad = ~(err <= grad_tolerance(g_ref, bf16))  # (an undefined entry counts as an error)
    assert not bad.any(), (np.argwhere(bad)[:5], err.max())
    assert abs(float(g_ref.sum())) < 1e-9 * g_ref.shape[-1] + 1e-9
    return float(err.max()) if err.size else 0.0
