"""Repeated calls at the full size (B=128, k=16, V=151936 bf16) with the
outputs filled with NaN before every call: every gradient entry and loss of
the rows in use must be written, and bit-identical from call to call, on the
fast path (c = 10) and on the exact two-barrier path (c = 0.01), fused with
verification, supervision alone, and a loss variant."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_drafter_verification_amd as ada
    wl = W.WORKLOADS[4]
    B, k, V = wl.B, wl.k, wl.V
    bt = W.generate(wl, round=3)
    dev = "cuda"
    t = torch.from_numpy(bt.target.view(np.int16)).view(torch.bfloat16).to(dev)
    d = torch.from_numpy(bt.draft.view(np.int16)).view(torch.bfloat16).to(dev)
    inp = dict(t=t, d=d, tok=torch.from_numpy(bt.tokens).to(dev), vl=torch.from_numpy(bt.verify_len).to(dev),
               u=torch.from_numpy(bt.uniforms).to(dev))
    out = dict(acc=torch.empty(B, dtype=torch.int32, device=dev),
               outt=torch.empty(B, k + 1, dtype=torch.int32, device=dev),
               mg=torch.empty(B, k + 1, dtype=torch.float32, device=dev),
               ro=torch.empty(B + 1, dtype=torch.int32, device=dev),
               ce=torch.empty(B * k, dtype=torch.float32, device=dev),
               rk=torch.empty(B * k, dtype=torch.float32, device=dev),
               grad=torch.empty(B * k, V, dtype=torch.bfloat16, device=dev),
               st=torch.zeros(1, dtype=torch.int32, device=dev), ws=ada.workspace(B, k, V, dev))
    N = int(np.clip(bt.verify_len, 1, k).sum())
    return ada, inp, out, N


@pytest.mark.parametrize("mode,c", [("fused", 10.0), ("fused", 0.01), ("opd", 0.01), ("mixture", 0.01)])
def test_every_entry_written_and_repeatable(setup, mode, c):
    import torch
    ada, i, o, N = setup
    print("repeat", mode, c, flush=True)
    first = None
    for rep in range(3):
        o["grad"].fill_(float("nan"))
        o["ce"].fill_(float("nan"))
        o["rk"].fill_(float("nan"))
        if mode == "fused":
            ada.adaflash_verify(i["t"], i["d"], i["tok"], i["vl"], i["u"], 1.0, o["acc"], o["outt"], o["mg"], c, 1.0,
                                o["ro"], o["ce"], o["rk"], o["grad"], o["st"], o["ws"])
        elif mode == "opd":
            ada.adaflash_opd_loss_fwd_bwd(i["t"], i["d"], i["vl"], c, 1.0, o["ro"], o["ce"], o["rk"], o["grad"],
                                          o["st"], o["ws"])
        else:
            ada.adaflash_loss_variant_fwd_bwd(i["t"], i["d"], i["vl"], "mixture", 0.8, c, o["ro"], o["ce"],
                                              o["grad"], o["st"], o["ws"])
        torch.cuda.synchronize()
        assert int(o["st"].item()) == 0
        g = o["grad"][:N]
        assert not bool(torch.isnan(g).any()), "unwritten gradient entries"
        assert not bool(torch.isnan(o["ce"][:N]).any()), "unwritten losses"
        snap = (g.view(torch.int16).clone(), o["ce"][:N].clone(), o["acc"].clone(), o["outt"].clone())
        if first is None:
            first = snap
        else:
            assert torch.equal(first[0], snap[0]), "gradient differs between identical calls"
            assert torch.equal(first[1], snap[1])
            if mode == "fused":
                assert torch.equal(first[2], snap[2]) and torch.equal(first[3], snap[3])


def test_prepared_call_repeats_the_direct_call(setup):
    """A prepared call (checked and marshalled once) gives the direct call's
    outputs bit for bit, on every repetition, with the outputs cleared in
    between."""
    import torch
    ada, i, o, N = setup
    print("prepared call", flush=True)
    args = (i["t"], i["d"], i["tok"], i["vl"], i["u"], 1.0, o["acc"], o["outt"], o["mg"], 10.0, 1.0, o["ro"],
            o["ce"], o["rk"], o["grad"], o["st"], o["ws"])
    ada.adaflash_verify(*args)
    torch.cuda.synchronize()
    ref = {kk: o[kk].clone() for kk in ("acc", "outt", "mg", "ro", "ce", "rk")}
    ref_grad = o["grad"][:N].clone()
    prep = ada.adaflash_verify(*args, prepare=True)
    for rep in range(3):
        for kk in ("ce", "rk", "mg"):
            o[kk].fill_(float("nan"))
        o["grad"].fill_(float("nan"))
        o["acc"].fill_(-7)
        prep.run()
        torch.cuda.synchronize()
        assert int(o["st"].item()) == 0
        for kk, v in ref.items():
            g, r = (o[kk][:N], v[:N]) if kk in ("ce", "rk") else (o[kk], v)
            if g.dtype == torch.float32:  # bit patterns (margins hold NaN past each verify length)
                g, r = g.view(torch.int32), r.view(torch.int32)
            assert torch.equal(g, r), kk
        assert torch.equal(o["grad"][:N].view(torch.int16), ref_grad.view(torch.int16))
