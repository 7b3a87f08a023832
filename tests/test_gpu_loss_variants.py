"""GPU parity of the supervision-loss variants (adaflash_loss_variant_fwd_bwd
through the C ABI) against the float64 oracle (oracle/loss_variants.py) on the
same seeded inputs.  Losses within 1e-3 relative + 1e-5 absolute (the
divergences are differences of row sums); gradients as the main supervision
path: 2e-3 absolute or one bf16 ulp (bf16), 2e-5 + 1e-5 relative (fp32)."""
import numpy as np
import pytest

import workloads as W
from oracle import loss_variants as LV
from helpers import compare_grad, to_dev

pytestmark = pytest.mark.gpu

CASES = [("rkl", 0.0, 0.0), ("rkl_clip", 0.05, 0.0), ("rkl_clip", 10.0, 0.0), ("mixture", 0.8, 0.01),
         ("mixture", 0.8, 10.0), ("fkl", 0.0, 0.0), ("wce", 7.0, 0.0)]


def _wl(B, k, V, bf16, seed):
    return W.Workload("variant", B=B, k=k, V=V, bf16=bf16, model=W.WL_ZIPF, T=1.0, p_scale=2.0, q_coef=0.7,
                      zipf_s=1.1, ragged=True, sigma_choice=True, sigmas=(0.3, 1.0, 2.0), seed=seed)


def _f64(a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _gpu(bt, variant, p1, p2, rows=None):
    import torch
    import diffusion_drafter_verification_amd as ada
    bf16 = bt.target.dtype == np.uint16
    out = ada.loss_variant_fwd_bwd(to_dev(bt.target, bf16), to_dev(bt.draft, bf16),
                                   torch.from_numpy(bt.verify_len).cuda(), variant, p1, p2)
    torch.cuda.synchronize()
    N = int(out["row_offsets"][-1].item())
    sel = torch.arange(N, device="cuda") if rows is None else torch.as_tensor(np.asarray(rows), device="cuda")
    return (int(out["status"].item()), out["loss"][:N].cpu().numpy(), out["grad"][sel].float().cpu().numpy(),
            out["row_offsets"].cpu().numpy())


def _check_losses(g, r):
    g = g.astype(np.float64)
    assert np.all(np.abs(g - r) <= 1e-3 * np.abs(r) + 1e-5), (np.argmax(np.abs(g - r)), g, r)


@pytest.mark.parametrize("variant,p1,p2", CASES)
@pytest.mark.parametrize("V,bf16", [(10000, True), (4097, True), (300, False)])
def test_variant_small(variant, p1, p2, V, bf16):
    bt = W.generate(_wl(5, 4, V, bf16, seed=V + 11), with_tokens=False)
    st, loss, grad, ro = _gpu(bt, variant, p1, p2)
    assert st == 0
    rl, rg = LV.batch(_f64(bt.target), _f64(bt.draft), bt.verify_len, variant, p1, p2)
    assert ro[-1] == len(rl)
    _check_losses(loss, rl)
    compare_grad(grad, rg, bf16=bf16)


@pytest.mark.parametrize("variant,p1,p2", [("mixture", 0.8, 0.01), ("fkl", 0.0, 0.0), ("wce", 7.0, 0.0)])
def test_variant_full_size_sampled_rows(variant, p1, p2):
    # B=128, k=16, V=151936 (the bench's workload); every loss, and the
    # gradient of 12 sampled rows, against the oracle row by row.
    bt = W.generate(W.WORKLOADS[4], round=0, with_tokens=False)
    L = np.clip(bt.verify_len, 1, 16)
    starts = np.concatenate([[0], np.cumsum(L)])
    rng = np.random.default_rng(9)
    pairs = sorted({(int(b), int(rng.integers(0, L[b]))) for b in rng.integers(0, 128, size=12)})
    rows = [int(starts[b] + i) for b, i in pairs]
    st, loss, grad, ro = _gpu(bt, variant, p1, p2, rows=rows)
    assert st == 0 and ro[-1] == starts[-1]
    tgt, drf = bt.target, bt.draft
    for (b, i), g in zip(pairs, grad):
        rl, rgr = LV.variant_row(_f64(tgt[b, i]), _f64(drf[b, i]), variant, i, p1, p2)
        _check_losses(loss[starts[b] + i:starts[b] + i + 1], np.array([rl]))
        compare_grad(g[None, :], rgr[None, :], bf16=True)
