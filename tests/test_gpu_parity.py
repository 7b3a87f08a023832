"""GPU parity: the gfx950 library, called through its C ABI binding, against the
CPU oracle on the same seeded inputs.

Bar: greedy outputs bit-exact; sampled accept lengths and tokens exact except
where the oracle puts the accept test inside the relative near-tie band
|p - u q| < 1e-5 max(p, u q), or the draw's threshold within 1e-5 of the total
mass from a CDF boundary (both bands and the flips are counted and printed);
losses within 1e-3 relative (1e-6 absolute floor); gradients within 2e-3
absolute or one bf16 ulp of the reference.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import (compare_grad, compare_losses, compare_margins, compare_verify, gpu_opd,
                     gpu_verify)
from parity import add_counts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_drafter_verification_amd as ada
    ada.load_library()   # raises if the library is missing: there is no fallback


def say(*a):
    print(*a, flush=True)


def small(name, B, k, V, bf16=True, T=1.0, ragged=True, seed=7, model=W.WL_ZIPF):
    return W.Workload(name, B=B, k=k, V=V, bf16=bf16, model=model, T=T, p_scale=2.0, q_coef=0.7,
                      zipf_s=1.1 if model == W.WL_ZIPF else 0.0, ragged=ragged, sigma_choice=True,
                      sigmas=(0.3, 1.0, 2.0), seed=seed)


def check_verify(bt, T, opd=False, c=10.0, lam=1.0, grad_rows=None):
    k = bt.tokens.shape[1]
    g = gpu_verify(bt, T, opd=opd, clip_c=c, lam=lam, grad_rows=grad_rows)
    r = oracle.verify(bt.target, bt.draft if T > 0 else None, bt.tokens, bt.verify_len, bt.uniforms, T=T)
    assert g["status"][0] == 0, g["status"]
    counts = compare_verify(g, r, T, bt.tokens, bt.verify_len, k)
    compare_margins(g, r, bt.verify_len, k, T)
    assert np.array_equal(g["row_offsets"], np.concatenate([[0], np.cumsum(np.clip(bt.verify_len, 1, k))]))
    if opd:
        ro = oracle.opd(bt.target, bt.draft, bt.verify_len, c, lam, rows=grad_rows,
                        with_grad=True)
        N = int(g["row_offsets"][-1])
        rows = np.arange(N) if grad_rows is None else np.asarray(grad_rows)
        compare_losses(g["loss_ce"][rows], g["loss_rkl"][rows], ro["loss_ce"], ro["loss_rkl"])
        compare_grad(g["grad"], ro["grad"], bf16=bt.target.dtype == np.uint16)
    return counts


def report(name, counts):
    say(f"{name}: {counts['requests']} requests, {counts['in_abs_band']} in the absolute band, "
        f"{counts['in_rel_band']} in the relative band, {counts['near_draw']} near a draw boundary, "
        f"{counts['flips']} flips")


# ------------------------------------------------------------ small shapes

@pytest.mark.parametrize("V,bf16", [(10000, True), (4096, True), (4097, True), (37, False), (9000, False)])
def test_greedy_small(V, bf16):
    say("greedy", V, bf16)
    bt = W.generate(small("g", B=6, k=5, V=V, bf16=bf16, T=0.0, seed=V), T=0.0)
    check_verify(bt, 0.0)


@pytest.mark.parametrize("V,bf16,T", [(10000, True, 1.0), (4097, True, 1.0), (37, False, 1.0),
                                      (12288, True, 0.7), (9000, False, 1.3)])
def test_sampled_small(V, bf16, T):
    say("sampled", V, bf16, T)
    bt = W.generate(small("s", B=16, k=6, V=V, bf16=bf16, T=T, seed=V + 1), T=T)
    check_verify(bt, T)


@pytest.mark.parametrize("T,c,lam", [(1.0, 10.0, 1.0), (1.0, 0.01, 1.0), (1.0, 0.05, 2.0),
                                     (0.7, 0.01, 0.25), (0.0, 0.02, 1.0), (1.0, 10.0, 0.0)])
def test_fused_small(T, c, lam):
    say("fused", T, c, lam)
    bt = W.generate(small("f", B=8, k=4, V=10000, T=T, seed=int(c * 1000) + 3), T=T)
    check_verify(bt, T, opd=True, c=c, lam=lam)


@pytest.mark.parametrize("V,bf16,ragged", [(10000, True, True), (4097, True, False), (300, False, True)])
def test_opd_only_small(V, bf16, ragged):
    say("opd", V, bf16, ragged)
    bt = W.generate(small("o", B=5, k=4, V=V, bf16=bf16, ragged=ragged, seed=V + 5), with_tokens=False)
    for c in (10.0, 0.01):
        vl = bt.verify_len if ragged else None
        g = gpu_opd(bt.target, bt.draft, vl, c, 1.0)
        r = oracle.opd(bt.target, bt.draft, vl, c, 1.0)
        N = r["N"]
        assert g["status"][0] == 0
        assert g["row_offsets"][-1] == N
        compare_losses(g["loss_ce"][:N], g["loss_rkl"][:N], r["loss_ce"], r["loss_rkl"])
        compare_grad(g["grad"][:N], r["grad"], bf16=bf16)


# -------------------------------------------------------------- edge cases

def test_empty_batch():
    import torch
    import diffusion_drafter_verification_amd as ada
    say("empty batch")
    t = torch.zeros(0, 5, 64, dtype=torch.bfloat16, device="cuda")
    d = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    e = torch.zeros(0, 4, dtype=torch.int32, device="cuda")
    out = ada.verify(t, d, e, torch.zeros(0, dtype=torch.int32, device="cuda"),
                     torch.zeros(0, 5, device="cuda"), T=1.0, opd=True)
    torch.cuda.synchronize()
    assert out["row_offsets"].cpu().tolist() == [0]
    o2 = ada.opd_loss_fwd_bwd(t, d, None)
    torch.cuda.synchronize()
    assert o2["row_offsets"].cpu().tolist() == [0]


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_vocabulary_of_one_and_single_draft(T):
    say("V=1", T)
    B, k = 3, 1
    bt = W.Batch(wl=None, round=0, target=np.zeros((B, k + 1, 1), np.float32),
                 draft=np.zeros((B, k, 1), np.float32), tokens=np.zeros((B, k), np.int32),
                 verify_len=np.ones(B, np.int32), uniforms=np.full((B, k + 1), 0.99, np.float32),
                 sigma=np.ones(B, np.float32))
    g = gpu_verify(bt, T, opd=True)
    assert list(g["accept_len"]) == [1, 1, 1]
    assert (g["out_tokens"] == 0).all()
    assert np.allclose(g["loss_ce"][:3], 0) and np.allclose(g["loss_rkl"][:3], 0)
    assert (g["grad"][:3] == 0).all()


def test_maximum_draft_length():
    say("k=64")
    bt = W.generate(small("k64", B=3, k=64, V=5000, seed=64), T=1.0)
    check_verify(bt, 1.0, opd=True)
    bt0 = W.generate(small("k64g", B=3, k=64, V=5000, T=0.0, seed=65), T=0.0)
    # long greedy prefixes: copy the target argmax into the drafts
    am = W.bf16_bits_to_f32(bt0.target[:, :64]).argmax(-1).astype(np.int32)
    bt0.tokens[:] = am
    bt0.tokens[1, 40] = (am[1, 40] + 1) % 5000
    bt0.verify_len[:] = [64, 64, 17]
    check_verify(bt0, 0.0)
    g = gpu_verify(bt0, 0.0)
    assert list(g["accept_len"]) == [64, 40, 17]


def test_bad_verify_len_and_tokens_are_clamped_and_flagged():
    say("clamping")
    bt = W.generate(small("c", B=4, k=5, V=3000, seed=9), T=1.0)
    vl = np.array([0, 9, -2, 3], np.int32)
    g = gpu_verify(bt, 1.0, verify_len=vl)
    assert g["status"][0] & 1
    r = oracle.verify(bt.target, bt.draft, bt.tokens, vl, bt.uniforms, T=1.0)
    compare_verify(g, r, 1.0, bt.tokens, vl, 5)
    tok = bt.tokens.copy()
    tok[2, 0] = 3000
    tok[3, 1] = -7
    g2 = gpu_verify(bt, 1.0, tokens=tok)
    assert g2["status"][0] & 2


@pytest.mark.parametrize("case", ["bonus", "residual_lo", "residual_hi", "zero_residual"])
def test_hand_worked_draws(case):
    """The V = 4 cases worked by hand in the oracle pins (tests/test_oracle_pins.py):
    accept margin, draw and draw margin of the bonus row, of a residual, and of
    the Z == 0 fallback to the target row."""
    say("hand-worked draw", case)
    rows = {"bonus": ([[0.1, 0.2, 0.3, 0.4], [0.1, 0.2, 0.3, 0.4]], [0.1, 0.2, 0.3, 0.4], 3, 0.5, 0.35),
            "residual_lo": ([[0.1, 0.4, 0.2, 0.3]] * 2, [0.3, 0.1, 0.4, 0.2], 0, 0.9, 0.6),
            "residual_hi": ([[0.1, 0.4, 0.2, 0.3]] * 2, [0.3, 0.1, 0.4, 0.2], 0, 0.9, 0.9),
            "zero_residual": ([[0.1, 0.2, 0.7, 0.0], [0.25] * 4], [0.1, 0.2, 0.7, 0.0], 3, 0.5, 0.25)}[case]
    p_rows, q_row, token, u_acc, u_draw = rows
    with np.errstate(divide="ignore"):
        target = np.log(np.asarray(p_rows, np.float64)).astype(np.float32)[None]
        draft = np.log(np.asarray([q_row], np.float64)).astype(np.float32)[None]
    # the same request many times over, so that it runs as a batch
    B = 64
    bt = W.Batch(wl=None, round=0, target=np.repeat(target, B, 0), draft=np.repeat(draft, B, 0),
                 tokens=np.full((B, 1), token, np.int32), verify_len=np.ones(B, np.int32),
                 uniforms=np.tile(np.array([[u_acc, u_draw]], np.float32), (B, 1)), sigma=np.ones(B, np.float32))
    g = gpu_verify(bt, 1.0)
    r = oracle.verify(bt.target, bt.draft, bt.tokens, bt.verify_len, bt.uniforms, T=1.0)
    assert g["status"][0] == 0
    assert np.array_equal(g["accept_len"], r["accept_len"]) and np.array_equal(g["out_tokens"], r["out_tokens"])
    assert np.abs(g["margins"][:, 0] - r["margins"][:, 0]).max() < 1e-6
    assert np.abs(g["margins"][:, 1] - r["margins"][:, 1]).max() < 1e-6


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("rows", ["both", "draft", "target"])
def test_masked_vocabulary_entries(rows, bf16):
    """-inf logits (probability 0) in 30% of the entries of the draft rows,
    the target rows or both: a draft entry at -inf makes an undefined term
    0 * inf in the chunk sums of the supervision pass, a target entry at -inf
    an infinite KL term that is always clipped."""
    say("masked entries", rows, "bf16" if bf16 else "fp32")
    bt = W.generate(small("m", B=6, k=4, V=8192, bf16=bf16, seed=11), T=1.0)
    ninf = np.uint16(0xFF80) if bf16 else np.float32(-np.inf)
    rng = np.random.default_rng(0)
    mask_t = rng.random(bt.target.shape) < 0.3
    mask_d = rng.random(bt.draft.shape) < 0.3
    if rows != "draft":
        bt.target[mask_t] = ninf
    if rows != "target":
        bt.draft[mask_d] = ninf
    # keep the drafts on tokens the drafter can produce
    zq = W.bf16_bits_to_f32(bt.draft) if bf16 else bt.draft
    bt.tokens[:] = zq.argmax(-1)
    for c in (10.0, 0.01):
        check_verify(bt, 1.0, opd=True, c=c)


@pytest.mark.parametrize("c", [3.0, 4.5, 8.0])
def test_clipped_entries_at_large_c(c):
    """Entries clipped at a large threshold: in half of the rows one token
    the drafter is sure of (z_q = 12) is one the target rules out (z_p =
    -12), so q (log q - log p) there is about 24 > c.  From c = 4 the
    supervision kernel takes its looser per-thread clip bound, below it the
    tighter one; both must send these rows to the exact path and match the
    oracle's clipped losses and gradients."""
    say("clipped at large c", c)
    bt = W.generate(small("x", B=6, k=4, V=8192, seed=21), T=1.0)
    zt = W.bf16_bits_to_f32(bt.target).astype(np.float32)
    zd = W.bf16_bits_to_f32(bt.draft).astype(np.float32)
    rng = np.random.default_rng(5)
    hit = rng.random(bt.draft.shape[:2]) < 0.5
    v = rng.integers(0, bt.draft.shape[2], size=bt.draft.shape[:2])
    for b, i in zip(*np.nonzero(hit)):
        zd[b, i, v[b, i]] = 12.0
        zt[b, i, v[b, i]] = -12.0
    bt.target[:] = W.f32_to_bf16_bits(zt)
    bt.draft[:] = W.f32_to_bf16_bits(zd)
    zq = W.bf16_bits_to_f32(bt.draft).astype(np.float64)
    zp = W.bf16_bits_to_f32(bt.target[:, :-1]).astype(np.float64)
    lq = zq - np.logaddexp.reduce(zq, axis=-1, keepdims=True)
    lp = zp - np.logaddexp.reduce(zp, axis=-1, keepdims=True)
    f = np.exp(lq) * (lq - lp)
    assert (f.max(-1) > c)[hit].all()  # (the clip is real in every such row)
    check_verify(bt, 1.0, opd=True, c=c)


def test_ties_take_the_lowest_index():
    say("ties")
    B, k, V = 4, 3, 9000
    t = np.zeros((B, k + 1, V), np.float32)
    t[1, :, 7000] = 3.0
    t[1, :, 4100] = 3.0        # tie across chunks: 4100 < 7000
    t[2, :, 5] = 1.0
    t[2, :, 4] = 1.0           # tie inside a thread's entries
    t[3] = np.round(np.random.default_rng(3).normal(0, 1, (k + 1, V)))  # many integer ties
    tok = np.argmax(t[:, :k], -1).astype(np.int32)
    tok[3, 1] = (tok[3, 1] + 1) % V
    bt = W.Batch(wl=None, round=0, target=t, draft=t[:, :k].copy(), tokens=tok,
                 verify_len=np.full(B, k, np.int32), uniforms=np.full((B, k + 1), 0.5, np.float32),
                 sigma=np.ones(B, np.float32))
    check_verify(bt, 0.0)
    g = gpu_verify(bt, 0.0)
    assert g["out_tokens"][0, 0] == 0 and g["out_tokens"][1, 0] == 4100 and g["out_tokens"][2, 0] == 4
    check_verify(bt, 1.0, opd=True, c=0.01)


def test_deterministic():
    say("determinism")
    bt = W.generate(small("d", B=12, k=8, V=20000, seed=12), T=1.0)
    first = gpu_verify(bt, 1.0, opd=True, clip_c=0.01)
    for _ in range(10):
        again = gpu_verify(bt, 1.0, opd=True, clip_c=0.01)
        for key in ("accept_len", "out_tokens", "row_offsets", "loss_ce", "loss_rkl", "grad"):
            assert np.array_equal(first[key], again[key]), key
        assert np.array_equal(first["margins"], again["margins"], equal_nan=True)


# ----------------------------------------------- tiny workload and statistics

def test_tiny_workload_parity():
    """20,000 rounds of the tiny workload (B=4, 15 drafts, V=64, fp32), as one
    batch of 80,000 requests."""
    wl = W.WORKLOADS[1]
    say("tiny workload")
    big = W.Workload(wl.name, B=4 * 20000, k=wl.k, V=wl.V, bf16=False, model=wl.model, T=1.0,
                     p_scale=wl.p_scale, q_coef=wl.q_coef, sigmas=wl.sigmas, seed=wl.seed)
    bt = W.generate(big)
    report("tiny", check_verify(bt, 1.0))


@pytest.mark.parametrize("a", [0.8, 0.9])
def test_closed_form_accept_length_on_gpu(a):
    say("closed form", a)
    m = 15
    exact = (1 - a ** (m + 1)) / (1 - a)
    bt = W.generate(W.two_level(a, B=80000, k=m))
    g = gpu_verify(bt, 1.0)
    A = g["accept_len"].astype(np.float64)
    tau = (A + 1).mean()
    se = (A + 1).std() / np.sqrt(A.size)
    assert abs(tau - exact) < 4 * se, (tau, exact, se)
    rate = (g["margins"][:, :m] > 0).mean(axis=0)
    assert np.abs(rate - a).max() < 4 * np.sqrt(a * (1 - a) / A.size)


@pytest.mark.parametrize("V", [8, 64])
def test_emitted_tokens_follow_the_target_on_gpu(V):
    from scipy import special, stats
    say("chi-square", V)
    k, T, n = 3, 1.0, 20000
    wl = W.Workload("chi", B=1, k=k, V=V, bf16=False, model=W.WL_GAUSS, T=T, p_scale=1.5, q_coef=0.3,
                    sigmas=(1.2, 1.2, 1.2), seed=300 + V, ragged=True)
    bts = [W.generate(wl, round=r, logits_round=0) for r in range(n)]
    bt = W.Batch(wl=wl, round=0, target=np.concatenate([b.target for b in bts]),
                 draft=np.concatenate([b.draft for b in bts]), tokens=np.concatenate([b.tokens for b in bts]),
                 verify_len=np.concatenate([b.verify_len for b in bts]),
                 uniforms=np.concatenate([b.uniforms for b in bts]), sigma=np.ones(n, np.float32))
    g = gpu_verify(bt, T)
    p_all = special.softmax(bts[0].target[0].astype(np.float64) / T, axis=-1)
    pvals = []
    for j in range(k + 1):
        reached = g["accept_len"] >= j
        cnt = int(reached.sum())
        if cnt < 200:
            continue
        obs = np.bincount(g["out_tokens"][reached, j], minlength=V).astype(np.float64)
        exp = cnt * p_all[j]
        keep = exp >= 5
        o = np.append(obs[keep], obs[~keep].sum())
        e = np.append(exp[keep], exp[~keep].sum())
        if e[-1] < 5:
            o[-2] += o[-1]
            e[-2] += e[-1]
            o, e = o[:-1], e[:-1]
        pvals.append(stats.chisquare(o, e).pvalue)
    assert len(pvals) >= 2 and min(pvals) > 1e-3 / len(pvals), pvals


# --------------------------------------------------------- full-size workloads

def _rounds(wl, rounds, T, with_draft=True):
    for r in range(rounds):
        yield W.generate(wl, round=r, T=T)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_single_request_workload(T):
    """B=1, k=16, V=151936 bf16; 1,000 seeded rounds, one call per round."""
    wl = W.WORKLOADS[2]
    say("single request", T)
    tot = {}
    for blk in range(20):
        bts = [W.generate(wl, round=r, T=T) for r in range(blk * 50, blk * 50 + 50)]
        gs = [gpu_verify(bt, T) for bt in bts]
        for g in gs:
            assert g["status"][0] == 0
        stack = lambda name: np.concatenate([getattr(b, name) for b in bts])
        r = oracle.verify(stack("target"), stack("draft") if T > 0 else None, stack("tokens"),
                          stack("verify_len"), stack("uniforms"), T=T)
        gcat = {key: np.concatenate([g[key] for g in gs]) for key in ("accept_len", "out_tokens", "margins")}
        add_counts(tot, compare_verify(gcat, r, T, stack("tokens"), stack("verify_len"), wl.k))
        compare_margins(gcat, r, stack("verify_len"), wl.k, T)
    report(f"single T={T}", tot)


@pytest.mark.parametrize("block", range(8))
def test_c32_workload(block):
    """B=32 ragged, T=1: 200 rounds in 8 blocks of 25."""
    wl = W.WORKLOADS[3]
    say("c32 block", block)
    tot = {}
    for r in range(block * 25, block * 25 + 25):
        bt = W.generate(wl, round=r)
        add_counts(tot, check_verify(bt, 1.0))
    report(f"c32 block {block}", tot)


GRAD_BLOCK = 128  # gradient rows copied back and compared at a time


def _compare_grad_blocks(g_grad_dev, bt, c, lam, rows):
    """Every listed packed row's gradient against the oracle, GRAD_BLOCK rows
    at a time (host memory stays bounded at V = 151936)."""
    import torch
    worst = 0.0
    for a in range(0, len(rows), GRAD_BLOCK):
        blk = np.asarray(rows[a:a + GRAD_BLOCK])
        gg = g_grad_dev[torch.as_tensor(blk, device="cuda")].float().cpu().numpy()
        ref = oracle.opd(bt.target, bt.draft, bt.verify_len, c, lam, rows=blk)
        worst = max(worst, compare_grad(gg, ref["grad"]))
    return worst


@pytest.mark.parametrize("c,rounds,full_rounds", [(10.0, 10, 2), (0.01, 5, 2)])
def test_c128_fused_workload(c, rounds, full_rounds):
    """B=128 ragged fused verify + supervision, as bench.py times it: accept
    lengths, tokens and margins of every request, losses of every row; the
    gradient of EVERY row in the first ``full_rounds`` rounds, of 48 sampled
    rows in the others."""
    import torch
    import diffusion_drafter_verification_amd as ada
    from helpers import to_dev
    wl = W.WORKLOADS[4]
    say("c128", c)
    rng = np.random.default_rng(int(c * 100))
    tot = {}
    worst_loss = worst_grad = 0.0
    for r in range(rounds):
        bt = W.generate(wl, round=r)
        N = int(np.clip(bt.verify_len, 1, wl.k).sum())
        out = ada.verify(to_dev(bt.target, True), to_dev(bt.draft, True), torch.from_numpy(bt.tokens).cuda(),
                         torch.from_numpy(bt.verify_len).cuda(), torch.from_numpy(bt.uniforms).cuda(), T=1.0,
                         opd=True, clip_c=c, lam=wl.lam)
        torch.cuda.synchronize()
        g = {key: out[key].cpu().numpy() for key in ("accept_len", "out_tokens", "margins", "row_offsets",
                                                      "loss_ce", "loss_rkl", "status")}
        assert g["status"][0] == 0
        ro = oracle.verify(bt.target, bt.draft, bt.tokens, bt.verify_len, bt.uniforms, T=1.0)
        add_counts(tot, compare_verify(g, ro, 1.0, bt.tokens, bt.verify_len, wl.k))
        compare_margins(g, ro, bt.verify_len, wl.k, 1.0)
        full = oracle.opd(bt.target, bt.draft, bt.verify_len, c, wl.lam, with_grad=False)
        worst_loss = max(worst_loss, compare_losses(g["loss_ce"][:N], g["loss_rkl"][:N], full["loss_ce"],
                                                    full["loss_rkl"]))
        rows = np.arange(N) if r < full_rounds else np.sort(rng.choice(N, size=48, replace=False))
        worst_grad = max(worst_grad, _compare_grad_blocks(out["grad"], bt, c, wl.lam, rows))
        del out
    report(f"c128 c={c}", tot)
    say(f"c128 c={c}: largest loss error {worst_loss:.2e} (relative), gradient {worst_grad:.2e} (absolute)")


@pytest.mark.parametrize("seed_off", [0, 1, 2])
def test_replay_workload(seed_off):
    """8192 rows x V=151936, supervision only: the losses of all 8192 rows and
    the gradients of 1,024 rows (every eighth row) against the oracle."""
    wl = W.WORKLOADS[5]
    say("replay", seed_off)
    wl = W.Workload(wl.name, B=wl.B, k=wl.k, V=wl.V, bf16=True, model=wl.model, T=1.0, p_scale=wl.p_scale,
                    q_coef=wl.q_coef, zipf_s=wl.zipf_s, sigmas=wl.sigmas, seed=wl.seed + 1000 * seed_off)
    bt = W.generate(wl, with_tokens=False)
    import torch
    import diffusion_drafter_verification_amd as ada
    from helpers import to_dev
    out = ada.opd_loss_fwd_bwd(to_dev(bt.target, True), to_dev(bt.draft, True), None, clip_c=wl.clip_c,
                               lam=wl.lam)
    torch.cuda.synchronize()
    assert int(out["status"][0]) == 0
    assert int(out["row_offsets"][-1]) == wl.B * wl.k
    N = wl.B * wl.k
    ce = out["loss_ce"][:N].cpu().numpy()
    rk = out["loss_rkl"][:N].cpu().numpy()
    ro = oracle.opd(bt.target, bt.draft, None, wl.clip_c, wl.lam, with_grad=False)
    worst_loss = compare_losses(ce, rk, ro["loss_ce"], ro["loss_rkl"])
    rows = np.arange(seed_off, N, 8)
    worst_grad = 0.0
    for a in range(0, len(rows), GRAD_BLOCK):
        blk = rows[a:a + GRAD_BLOCK]
        gg = out["grad"][torch.as_tensor(blk, device="cuda")].float().cpu().numpy()
        rg = oracle.opd(bt.target, bt.draft, None, wl.clip_c, wl.lam, rows=blk)
        worst_grad = max(worst_grad, compare_grad(gg, rg["grad"]))
    say(f"replay {seed_off}: {N} losses (largest error {worst_loss:.2e} relative), {len(rows)} gradient rows "
        f"(largest error {worst_grad:.2e})")


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_c128_verify_only_workload(T):
    """B=128, k=16, V=151936 bf16 verification without supervision (the
    statistics and residual kernels at T=1, the greedy statistics kernel at
    T=0, as bench.py --mode verify / --mode greedy time them): every
    request's accept length, tokens and margins against the oracle, 3
    rounds."""
    wl = W.WORKLOADS[4]
    say("c128 verify only", T)
    tot = {}
    for r in range(3):
        bt = W.generate(wl, round=r, T=T) if T == 0 else W.generate(wl, round=r)
        add_counts(tot, check_verify(bt, T))
    report(f"c128 verify only T={T}", tot)
