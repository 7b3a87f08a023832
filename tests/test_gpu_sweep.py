"""Seeded sweep of 96 small configurations through the C ABI against the oracle:
vocabulary sizes around the 8192-entry chunk boundary (and 1, 7), bf16 and
fp32 rows, draft lengths 1 to 16, ragged and full verify lengths, greedy and
sampled temperatures, with and without fused supervision (clip thresholds on
either path, lambda 0 to 2.5), padded and packed logits.  Same bar as
test_gpu_parity.py."""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import compare_grad, compare_losses, compare_margins, compare_verify, gpu_verify, to_dev

pytestmark = pytest.mark.gpu

VS = [1, 7, 3000, 8191, 8192, 8193, 16384, 16385, 24577]


def _cases(n=96, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for q in range(n):
        V = int(VS[q % len(VS)])
        out.append(dict(V=V, bf16=bool(rng.integers(0, 2)), k=int(rng.choice([1, 3, 8, 16])),
                        B=int(rng.choice([1, 2, 5, 9])), T=float(rng.choice([0.0, 0.6, 1.0])),
                        opd=bool(rng.integers(0, 2)), c=float(rng.choice([10.0, 0.02])),
                        lam=float(rng.choice([0.0, 1.0, 2.5])), packed=bool(rng.integers(0, 2)),
                        ragged=bool(rng.integers(0, 2)), seed=int(rng.integers(1, 1 << 30))))
    return out


def _packed_verify(bt, T, opd, c, lam):
    import torch
    import diffusion_drafter_verification_amd as ada
    bf16 = bt.target.dtype == np.uint16
    B, k1, V = bt.target.shape
    L = np.clip(bt.verify_len, 1, k1 - 1)
    tp = np.concatenate([bt.target[b, :L[b] + 1] for b in range(B)])
    dp = np.concatenate([bt.draft[b, :L[b]] for b in range(B)])
    out = ada.verify_packed(to_dev(tp, bf16), to_dev(dp, bf16), torch.from_numpy(bt.tokens).cuda(),
                            torch.from_numpy(bt.verify_len).cuda(), torch.from_numpy(bt.uniforms).cuda(),
                            T=T, opd=opd, clip_c=c, lam=lam)
    torch.cuda.synchronize()
    grad = out.pop("grad")
    res = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    res["grad"] = grad.float().cpu().numpy() if grad is not None else None
    return res


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "V{V}-{k}x{B}-T{T}-{opd}-{packed}".format(**c))
def test_sweep(case):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("sweep", case, flush=True)
    c = case
    wl = W.Workload("sweep", B=c["B"], k=c["k"], V=c["V"], bf16=c["bf16"], model=W.WL_ZIPF, T=c["T"],
                    p_scale=2.0, q_coef=0.7, zipf_s=1.1, ragged=c["ragged"], sigma_choice=True,
                    sigmas=(0.3, 1.0, 2.0), seed=c["seed"])
    bt = W.generate(wl, T=c["T"])
    T, k = c["T"], c["k"]
    if c["packed"]:
        g = _packed_verify(bt, T, c["opd"], c["c"], c["lam"])
    else:
        g = gpu_verify(bt, T, opd=c["opd"], clip_c=c["c"], lam=c["lam"])
    r = oracle.verify(bt.target, bt.draft if T > 0 else None, bt.tokens, bt.verify_len, bt.uniforms, T=T)
    assert g["status"][0] == 0, g["status"]
    compare_verify(g, r, T, bt.tokens, bt.verify_len, k)
    compare_margins(g, r, bt.verify_len, k, T)
    L = np.clip(bt.verify_len, 1, k)
    assert np.array_equal(g["row_offsets"], np.concatenate([[0], np.cumsum(L)]))
    if c["opd"]:
        ro = oracle.opd(bt.target, bt.draft, bt.verify_len, c["c"], c["lam"], with_grad=True)
        N = ro["N"]
        compare_losses(g["loss_ce"][:N], g["loss_rkl"][:N], ro["loss_ce"], ro["loss_rkl"])
        compare_grad(g["grad"][:N], ro["grad"], bf16=c["bf16"])
