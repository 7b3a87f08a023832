"""The measurement hook (adaflash_timing_enable / adaflash_timing_read):
while it is on, the dominant kernel of every call is launched with events
attached to its dispatch.  The outputs must not change (bit for bit against
the same calls with the hook off), one duration is recorded per call up to
the capacity, the calls past it run unrecorded, and a read starts a new
series."""
import numpy as np
import pytest

import workloads as W
from helpers import to_dev

pytestmark = pytest.mark.gpu


def _wl(seed):
    return W.Workload("hook", B=6, k=5, V=20000, bf16=True, model=W.WL_ZIPF, T=1.0, p_scale=2.0, q_coef=0.7,
                      zipf_s=1.1, ragged=True, sigma_choice=True, sigmas=(0.3, 1.0, 2.0), seed=seed)


def _bits(out, N):
    import torch
    res = {}
    for key, v in out.items():
        if v is None:
            continue
        if key == "grad":
            v = v[:N].view(torch.int16)
        elif key in ("loss_ce", "loss_rkl"):
            v = v[:N]
        res[key] = v.cpu().numpy().copy()
    return res


@pytest.mark.parametrize("mode", ["fused", "verify", "greedy", "opd"])
def test_hook_records_and_leaves_outputs_unchanged(mode):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_drafter_verification_amd as ada
    print("timing hook", mode, flush=True)
    T = 0.0 if mode == "greedy" else 1.0
    bt = W.generate(_wl(91), T=T) if mode != "opd" else W.generate(_wl(91), with_tokens=False)
    N = int(np.clip(bt.verify_len, 1, 5).sum())
    t, d = to_dev(bt.target, True), to_dev(bt.draft, True)
    vl = torch.from_numpy(bt.verify_len).cuda()

    def call():
        if mode == "opd":
            return ada.opd_loss_fwd_bwd(t, d, vl, clip_c=0.05, lam=1.0)
        tok = torch.from_numpy(bt.tokens).cuda()
        uni = torch.from_numpy(bt.uniforms).cuda()
        return ada.verify(t, d, tok, vl, uni, T=T, opd=mode == "fused", clip_c=0.05, lam=1.0)

    ada.adaflash_timing_enable(0)
    ref = _bits(call(), N)
    torch.cuda.synchronize()
    try:
        ada.adaflash_timing_enable(2)
        outs = [_bits(call(), N) for _ in range(3)]  # the third call runs past the capacity
        torch.cuda.synchronize()
        ms = ada.adaflash_timing_read(8)
        assert len(ms) == 2, ms
        assert all(np.isfinite(x) and 0.0 < x < 1000.0 for x in ms), ms
        assert ada.adaflash_timing_read(8) == []  # a read starts a new series
        call()
        torch.cuda.synchronize()
        assert len(ada.adaflash_timing_read(8)) == 1
    finally:
        ada.adaflash_timing_enable(0)
    for o in outs:
        assert o.keys() == ref.keys()
        for key in ref:
            assert np.array_equal(o[key].view(np.uint8), ref[key].view(np.uint8)), key


def test_hook_samples_every_nth_call():
    """adaflash_timing_every(n): events on calls 0, n, 2n, ... only, up to the
    capacity; adaflash_timing_enable restores every call."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_drafter_verification_amd as ada
    print("timing hook stride", flush=True)
    bt = W.generate(_wl(92), with_tokens=False)
    t, d = to_dev(bt.target, True), to_dev(bt.draft, True)
    vl = torch.from_numpy(bt.verify_len).cuda()
    with pytest.raises(ada.AdaflashError):
        ada.adaflash_timing_every(0)
    try:
        ada.adaflash_timing_enable(8)
        ada.adaflash_timing_every(3)
        for _ in range(7):  # calls 0, 3 and 6 carry events
            ada.opd_loss_fwd_bwd(t, d, vl, clip_c=10.0, lam=1.0)
        torch.cuda.synchronize()
        assert len(ada.adaflash_timing_read(8)) == 3
        ada.adaflash_timing_enable(8)  # back to every call
        for _ in range(2):
            ada.opd_loss_fwd_bwd(t, d, vl, clip_c=10.0, lam=1.0)
        torch.cuda.synchronize()
        assert len(ada.adaflash_timing_read(8)) == 2
    finally:
        ada.adaflash_timing_enable(0)
