"""Seeded input generator: Philox known answers, determinism, shapes and value recipes."""
import json
import os

import numpy as np
import pytest

import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLD, "philox_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["ctr"]]
        key = [int(x, 16) for x in vec["key"]]
        out = [int(x, 16) for x in vec["out"]]
        assert list(W.philox4x32_10(ctr, key)) == out


def test_bf16_rounding_helpers():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: round to even (1.0)
    assert back[0] == 1.0 and back[1] == 1.0
    assert back[2] == np.float32(1.0078125)
    assert back[3] == -2.5


def test_shapes_and_determinism():
    wl = W.WORKLOADS[3]
    small = W.Workload("s", B=6, k=16, V=1000, bf16=True, model=W.WL_ZIPF, T=1.0, p_scale=2.0,
                       q_coef=0.7, zipf_s=1.1, ragged=True, sigma_choice=True, sigmas=wl.sigmas,
                       seed=wl.seed)
    a = W.generate(small, round=3)
    b = W.generate(small, round=3, nthreads=1)
    c = W.generate(small, round=4)
    assert a.target.shape == (6, 17, 1000) and a.draft.shape == (6, 16, 1000)
    assert a.target.dtype == np.uint16
    for name in ("target", "draft", "tokens", "verify_len", "uniforms", "sigma"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert not np.array_equal(a.target, c.target)
    assert a.verify_len.min() >= 1 and a.verify_len.max() <= 16
    assert set(np.unique(a.sigma)).issubset({np.float32(0.3), np.float32(1.0), np.float32(2.0)})
    assert ((a.uniforms >= 0) & (a.uniforms < 1)).all()
    assert ((a.tokens >= 0) & (a.tokens < 1000)).all()


def test_verify_len_and_sigma_are_roughly_uniform():
    wl = W.Workload("s", B=20000, k=16, V=4, bf16=True, model=W.WL_ZIPF, T=1.0, ragged=True,
                    sigma_choice=True, sigmas=(0.3, 1.0, 2.0), seed=77)
    bt = W.generate(wl, with_tokens=False)
    counts = np.bincount(bt.verify_len, minlength=17)[1:]
    assert counts.min() > 0.8 * 20000 / 16 and counts.max() < 1.2 * 20000 / 16
    s = np.unique(bt.sigma, return_counts=True)[1]
    assert s.min() > 0.9 * 20000 / 3


def test_normal_moments_and_zipf_prior():
    wl = W.Workload("g", B=64, k=1, V=4096, bf16=False, model=W.WL_GAUSS, T=1.0, p_scale=1.0,
                    q_coef=0.0, sigmas=(1.0, 1.0, 1.0), seed=5)
    bt = W.generate(wl, with_tokens=False)
    z = bt.target.astype(np.float64).ravel()
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    # The prior is -1.1 ln(v+1): averaging rows removes the noise.
    wz = W.Workload("z", B=256, k=1, V=512, bf16=False, model=W.WL_ZIPF, T=1.0, p_scale=2.0,
                    q_coef=0.7, zipf_s=1.1, seed=9)
    bz = W.generate(wz, with_tokens=False)
    mean_row = bz.target.astype(np.float64).mean(axis=(0, 1))
    prior = -1.1 * np.log(np.arange(512) + 1.0)
    assert np.abs(mean_row - prior).max() < 0.35


def test_two_level_case_has_requested_overlap():
    wl = W.two_level(0.8)
    bt = W.generate(wl)
    zp = bt.target[0, 0].astype(np.float64)
    zq = bt.draft[0, 0].astype(np.float64)
    p = np.exp(zp) / np.exp(zp).sum()
    q = np.exp(zq) / np.exp(zq).sum()
    assert abs(np.minimum(p, q).sum() - 0.8) < 1e-6


def test_draft_tokens_follow_the_draft_distribution():
    # Gumbel-max sampling from softmax(z_q / T): compare frequencies with the softmax.
    wl = W.Workload("t", B=1, k=1, V=8, bf16=False, model=W.WL_GAUSS, T=0.7, p_scale=1.0,
                    q_coef=0.5, sigmas=(1.0, 1.0, 1.0), seed=21)
    toks = []
    for r in range(4000):
        bt = W.generate(wl, round=r, logits_round=0)
        toks.append(int(bt.tokens[0, 0]))
    zq = bt.draft[0, 0].astype(np.float64) / 0.7
    q = np.exp(zq - zq.max())
    q /= q.sum()
    freq = np.bincount(toks, minlength=8) / 4000.0
    assert np.abs(freq - q).max() < 4 * np.sqrt(q.max() / 4000.0)


def test_greedy_draft_tokens_are_argmax():
    wl = W.Workload("g0", B=3, k=4, V=50, bf16=True, model=W.WL_ZIPF, T=0.0, p_scale=2.0,
                    q_coef=0.7, zipf_s=1.1, seed=3)
    bt = W.generate(wl)
    zq = W.bf16_bits_to_f32(bt.draft)
    assert np.array_equal(bt.tokens, zq.argmax(axis=-1))
