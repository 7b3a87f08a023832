"""Vocabularies of more than 64 chunks of 8192 entries: V = 2^20 (the largest
accepted, 128 chunks) and V = 600,001 (74 chunks, a ragged tail, unaligned
rows).  The finaliser holds up to two chunk records of a row per lane, and
only these sizes use the second.  Gaussian logits with no rank prior spread
the probability mass over the whole row, so the emitted tokens fall in both
halves of the chunk range; the test checks that they do.  Same bar as
test_gpu_parity.py."""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import compare_grad, compare_losses, compare_margins, compare_verify, gpu_verify

CASES = [  # (V, bf16, T, supervision, seed)
    (1 << 20, True, 1.0, True, 7001),
    (1 << 20, True, 0.0, False, 7002),
    (600001, True, 1.0, False, 7003),
    (600001, False, 0.7, True, 7004),
]
HALF = 64 * 8192  # first vocabulary index of the second half of the chunk records


def batch(V, bf16, T, seed):
    wl = W.Workload("wide", B=4, k=3, V=V, bf16=bf16, model=W.WL_GAUSS, T=T, p_scale=2.0, q_coef=0.7,
                    ragged=True, sigma_choice=True, sigmas=(0.3, 1.0, 2.0), seed=seed)
    return W.generate(wl, T=T)


def emitted(out_tokens, accept_len):
    return np.array([out_tokens[b, accept_len[b]] for b in range(out_tokens.shape[0])])


@pytest.mark.gpu
@pytest.mark.parametrize("V,bf16,T,opd,seed", CASES)
def test_wide_vocabulary(V, bf16, T, opd, seed):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("wide vocab", V, bf16, T, opd, seed, flush=True)
    bt = batch(V, bf16, T, seed)
    k = 3
    g = gpu_verify(bt, T, opd=opd, clip_c=0.05, lam=1.0)
    r = oracle.verify(bt.target, bt.draft if T > 0 else None, bt.tokens, bt.verify_len, bt.uniforms, T=T)
    assert g["status"][0] == 0, g["status"]
    compare_verify(g, r, T, bt.tokens, bt.verify_len, k)
    compare_margins(g, r, bt.verify_len, k, T)
    if opd:
        ro = oracle.opd(bt.target, bt.draft, bt.verify_len, 0.05, 1.0, with_grad=True)
        N = ro["N"]
        compare_losses(g["loss_ce"][:N], g["loss_rkl"][:N], ro["loss_ce"], ro["loss_rkl"])
        compare_grad(g["grad"][:N], ro["grad"], bf16=bf16)


def test_cases_reach_the_upper_chunks():
    """The oracle's emitted tokens over the sampled cases (the draws that
    search the chunk records) lie on both sides of chunk 64 (a CPU test: it
    checks the inputs, not the kernels)."""
    lo = hi = 0
    for V, bf16, T, _, seed in CASES:
        if T == 0:
            continue
        bt = batch(V, bf16, T, seed)
        r = oracle.verify(bt.target, bt.draft if T > 0 else None, bt.tokens, bt.verify_len, bt.uniforms, T=T)
        e = emitted(r["out_tokens"], r["accept_len"])
        lo += int((e < HALF).sum())
        hi += int((e >= HALF).sum())
    assert lo > 0 and hi > 0, (lo, hi)
