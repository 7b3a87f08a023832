"""GPU parity of the adaptive length head (adaflash_length_head_forward and
adaflash_length_head_backward through the C ABI) against the float64 oracle
(oracle/length_head.py) on the same seeded inputs.

Tolerances (fp32 accumulation of exact bf16 products on the matrix cores):
a_hat within 2e-5 absolute; k_hat exactly the fp32 rule applied to the GPU's
a_hat, and equal to the oracle's wherever gamma a k is not within 1e-4 of an
integer; loss within 1e-5 absolute; each gradient element within
1e-4 x (the sum of the absolute values of its terms) + 1e-9."""
import numpy as np
import pytest

import workloads as W
from oracle import length_head as LH

pytestmark = pytest.mark.gpu


def _dev(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def _run(lb: W.LengthHeadBatch, gamma: float):
    import torch
    import diffusion_drafter_verification_amd as ada
    h = _dev(lb.hidden.view(np.int16), torch.bfloat16)
    W1 = _dev(lb.W1.view(np.int16), torch.bfloat16)
    b1, w2 = _dev(lb.b1), _dev(lb.w2)
    fwd = ada.length_head_forward(h, W1, b1, w2, lb.b2, gamma)
    bwd = ada.length_head_backward(h, W1, b1, w2, lb.b2, _dev(lb.accept_len), _dev(lb.verify_len))
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in fwd.items()}, {k: v.cpu().numpy() for k, v in bwd.items()})


def _check(lb: W.LengthHeadBatch, gamma: float):
    fwd, bwd = _run(lb, gamma)
    h = LH.bf16_to_f64(lb.hidden)
    W1 = LH.bf16_to_f64(lb.W1)
    B, k, H = h.shape
    ref = LH.forward(h, W1, lb.b1, lb.w2, lb.b2, gamma)
    assert np.max(np.abs(fwd["a_hat"] - ref["a_hat"])) < 2e-5
    # k_hat: the GPU's fp32 decision from its own a_hat; the oracle's wherever it is not a near tie.
    x = np.floor(np.float32(gamma) * fwd["a_hat"].astype(np.float32) * np.float32(k))
    assert np.array_equal(fwd["k_hat"], np.clip(x, 1, k).astype(np.int32))
    t = gamma * ref["a_hat"] * k
    clear = np.abs(t - np.round(t)) > 1e-4
    assert np.array_equal(fwd["k_hat"][clear], ref["k_hat"][clear])
    g = LH.loss_backward(h, W1, lb.b1, lb.w2, lb.b2, lb.accept_len, lb.verify_len)
    assert np.max(np.abs(bwd["loss"] - g["loss"])) < 1e-5
    # Scale of each gradient element: the sum of |terms| of its reduction.
    f = LH.forward(h, W1, lb.b1, lb.w2, lb.b2, 1.0)
    z = f["z1"]
    sg = 1.0 / (1.0 + np.exp(-z))
    a = f["a_hat"]
    ds = 2.0 * (a - g["a_star"]) * a * (1.0 - a)
    dz = (ds[:, None, None] * lb.w2.astype(np.float64)[None, None, :] / k) * sg * (1 + z * (1 - sg))
    dzm = np.abs(dz.reshape(B * k, -1))
    sW1 = dzm.T @ np.abs(h.reshape(B * k, H))
    sb1 = dzm.sum(axis=0)
    sw2 = np.abs(f["hbar"]).T @ np.abs(ds)
    sb2 = np.abs(ds).sum()
    for key, scale in (("dW1", sW1), ("db1", sb1), ("dw2", sw2)):
        err = np.abs(bwd[key] - g[key])
        assert np.all(err <= 1e-4 * scale + 1e-9), (key, float(err.max()), float(scale.max()))
    assert abs(bwd["db2"][0] - g["db2"]) <= 1e-4 * sb2 + 1e-9


@pytest.mark.parametrize("B,k,H,Hp,gamma", [
    (5, 16, 64, 48, 1.0),      # ragged column tile, one row tile
    (9, 16, 128, 100, 1.3),    # ragged rows (M = 144) and columns
    (1, 1, 16, 1, 0.7),        # smallest shapes
    (3, 7, 32, 70, 0.9),       # k not a divisor of the tile, M = 21
    (40, 16, 256, 64, 1.0),    # several row tiles; the weight product in two slices
    (37, 16, 400, 200, 1.1),   # every tile edge ragged: M = 592, H' = 200, H = 400
])
def test_length_head_small(B, k, H, Hp, gamma):
    _check(W.length_head_inputs(B, k, H, Hp, seed=1000 + B * 7 + Hp), gamma)


def test_length_head_full_size():
    # B = 128 requests, k = 16 positions, H = 4096, H' = 256: the size the bench times.
    _check(W.length_head_inputs(128, 16, 4096, 256), 1.0)


def test_length_head_empty_batch():
    import torch
    import diffusion_drafter_verification_amd as ada
    h = torch.zeros(0, 16, 64, dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    b1 = torch.zeros(8, device="cuda")
    out = ada.length_head_forward(h, W1, b1, b1, 0.0)
    torch.cuda.synchronize()
    assert out["a_hat"].numel() == 0 and out["k_hat"].numel() == 0


@pytest.mark.parametrize("B", [128, 7])
def test_cached_projection_equals_recomputed(B):
    """The forward's kept projection fed to the backward gives the same
    outputs, bit for bit, as the backward that recomputes it; the forward's
    own outputs do not change either; and the kept projection matches the
    oracle's h W1^T."""
    import torch
    import diffusion_drafter_verification_amd as ada
    lb = W.length_head_inputs(B)
    h = _dev(lb.hidden.view(np.int16), torch.bfloat16)
    W1 = _dev(lb.W1.view(np.int16), torch.bfloat16)
    b1, w2 = _dev(lb.b1), _dev(lb.w2)
    A, L = _dev(lb.accept_len), _dev(lb.verify_len)
    f0 = ada.length_head_forward(h, W1, b1, w2, lb.b2, 1.0)
    f1 = ada.length_head_forward(h, W1, b1, w2, lb.b2, 1.0, keep_projection=True)
    g0 = ada.length_head_backward(h, W1, b1, w2, lb.b2, A, L)
    g1 = ada.length_head_backward(h, W1, b1, w2, lb.b2, A, L, z1=f1["z1"])
    torch.cuda.synchronize()
    for key in ("a_hat", "k_hat"):
        assert torch.equal(f0[key], f1[key]), key
    for key in ("loss", "dW1", "db1", "dw2", "db2"):
        assert torch.equal(g0[key], g1[key]), key
    hh = LH.bf16_to_f64(lb.hidden).reshape(B * lb.hidden.shape[1], -1)
    ref = hh @ LH.bf16_to_f64(lb.W1).T
    z = f1["z1"].double().cpu().numpy()
    scale = np.abs(hh) @ np.abs(LH.bf16_to_f64(lb.W1)).T
    assert np.all(np.abs(z - ref) <= 1e-4 * scale + 1e-9)


@pytest.mark.parametrize("B", [128, 9])
def test_unaligned_weight_gradient_output(B):
    """A dW1 that is not 16-byte aligned takes the workspace and the slice sum
    instead of the weight product's direct 16-byte stores (one slice at these
    sizes); its values equal those of an aligned dW1, and so do the other
    outputs."""
    import torch
    import diffusion_drafter_verification_amd as ada
    lb = W.length_head_inputs(B, 16, 4096 if B == 128 else 128, 256 if B == 128 else 100, seed=77 + B)
    h = _dev(lb.hidden.view(np.int16), torch.bfloat16)
    W1 = _dev(lb.W1.view(np.int16), torch.bfloat16)
    b1, w2 = _dev(lb.b1), _dev(lb.w2)
    A, L = _dev(lb.accept_len), _dev(lb.verify_len)
    Bn, k, H = lb.hidden.shape
    Hp = lb.W1.shape[0]
    ws = ada.length_head_workspace(Bn, k, H, Hp)
    outs = []
    for offset in (0, 1):
        store = torch.full((Hp * H + 4,), float("nan"), dtype=torch.float32, device="cuda")
        dW1 = store[offset:offset + Hp * H].view(Hp, H)
        assert (dW1.data_ptr() % 16 == 0) == (offset == 0)
        o = {"loss": torch.empty(Bn, device="cuda"), "dW1": dW1, "db1": torch.empty(Hp, device="cuda"),
             "dw2": torch.empty(Hp, device="cuda"), "db2": torch.empty(1, device="cuda")}
        ada.adaflash_length_head_backward(h, W1, b1, w2, lb.b2, A, L, o["loss"], o["dW1"], o["db1"], o["dw2"],
                                          o["db2"], ws)
        torch.cuda.synchronize()
        outs.append({key: v.clone() for key, v in o.items()})
    assert torch.isfinite(outs[1]["dW1"]).all()
    for key in ("loss", "dW1", "db1", "dw2", "db2"):
        assert torch.equal(outs[0][key], outs[1][key]), key
