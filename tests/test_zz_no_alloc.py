"""adaflash_verify_noalloc (the entry point for callers that cannot allocate)
against adaflash_verify with a caller workspace: every output bit-identical on
two calls in a row, the second with a smaller input, and a batch too large for
the library's own array rejected with nothing written."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ada():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_drafter_verification_amd as ada
    ada.load_library()
    return ada


def _inputs(bt, bf16):
    import torch
    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if bf16 else a))
        return (t.view(torch.bfloat16) if bf16 else t).cuda()
    return dict(t=dev(bt.target), d=dev(bt.draft), tok=torch.from_numpy(bt.tokens).cuda(),
                vl=torch.from_numpy(bt.verify_len).cuda(), u=torch.from_numpy(bt.uniforms).cuda())


def _outputs(B, k, V, dtype):
    import torch
    nan = float("nan")
    return dict(acc=torch.full((B,), -9, dtype=torch.int32, device="cuda"),
                outt=torch.full((B, k + 1), -9, dtype=torch.int32, device="cuda"),
                mg=torch.full((B, k + 1), nan, device="cuda"),
                ro=torch.full((B + 1,), -9, dtype=torch.int32, device="cuda"),
                ce=torch.full((B * k,), nan, device="cuda"), rk=torch.full((B * k,), nan, device="cuda"),
                grad=torch.full((B * k, V), nan, dtype=dtype, device="cuda"),
                st=torch.full((1,), -9, dtype=torch.int32, device="cuda"))


def _call(ada, fn, i, o, T, c, ws=None):
    args = (i["t"], i["d"], i["tok"], i["vl"], i["u"], T, o["acc"], o["outt"], o["mg"], c, 1.0, o["ro"], o["ce"],
            o["rk"], o["grad"], o["st"])
    if ws is None:
        fn(*args)
    else:
        fn(*args, ws)


def _same(o1, o2, N):
    import torch
    for key in ("acc", "outt", "ro", "st"):
        assert torch.equal(o1[key], o2[key]), key
    assert torch.equal(o1["mg"].view(torch.int32), o2["mg"].view(torch.int32))
    for key in ("ce", "rk"):
        assert torch.equal(o1[key][:N].view(torch.int32), o2[key][:N].view(torch.int32)), key
    g1, g2 = o1["grad"][:N], o2["grad"][:N]
    assert torch.equal(g1.view(torch.int16) if g1.dtype == torch.bfloat16 else g1.view(torch.int32),
                       g2.view(torch.int16) if g2.dtype == torch.bfloat16 else g2.view(torch.int32)), "grad"


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_the_workspace_entry_point(ada, order):
    import torch
    print("no-alloc: c128 fused, then a small fp32 call", flush=True)
    cases = [(W.WORKLOADS[4], 1.0, 10.0, 0),
             (W.Workload("s", B=8, k=5, V=10000, bf16=False, model=W.WL_ZIPF, T=0.7, p_scale=2.0, q_coef=0.7,
                         zipf_s=1.1, ragged=True, sigma_choice=True, sigmas=(0.3, 1.0, 2.0), seed=91), 0.7, 0.01, 1)]
    for wl, T, c, rnd in cases:
        bt = W.generate(wl, round=rnd, T=T)
        bf16 = wl.bf16
        dtype = torch.bfloat16 if bf16 else torch.float32
        i = _inputs(bt, bf16)
        N = int(np.clip(bt.verify_len, 1, wl.k).sum())
        ref = _outputs(wl.B, wl.k, wl.V, dtype)
        _call(ada, ada.adaflash_verify, i, ref, T, c, ada.workspace(wl.B, wl.k, wl.V))
        got = _outputs(wl.B, wl.k, wl.V, dtype)
        _call(ada, ada.adaflash_verify_noalloc, i, got, T, c)
        torch.cuda.synchronize()
        assert int(ref["st"].item()) == 0
        _same(ref, got, N)
        print(f"  B={wl.B} V={wl.V} T={T} c={c}: identical ({N} rows)", flush=True)


def test_noalloc_rejects_a_batch_beyond_its_array(ada):
    import torch
    B, k, V = 4096, 16, 151936
    assert ada.adaflash_workspace_bytes(B, k, V) > ada.NOALLOC_WORKSPACE_BYTES
    t = torch.zeros(B, k + 1, 8, dtype=torch.bfloat16, device="cuda")  # shapes only; nothing may be read
    o = _outputs(B, k, 8, torch.bfloat16)
    tv = t.expand(B, k + 1, 8)
    with pytest.raises(ada.AdaflashError) as err:
        lib = ada.load_library()
        rc = lib.adaflash_verify_noalloc(1, tv.data_ptr(), tv.data_ptr(), o["outt"].data_ptr(), o["acc"].data_ptr(),
                                         o["mg"].data_ptr(), B, k, V, 1.0, o["acc"].data_ptr(), o["outt"].data_ptr(),
                                         None, 10.0, 1.0, o["ro"].data_ptr(), None, None, None, None, None)
        ada._check(rc)
    assert err.value.code == -4
    torch.cuda.synchronize()
    assert bool((o["acc"] == -9).all()) and bool((o["ro"] == -9).all())
