"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one part of the oracle to something other than itself: a value
printed on a page (tests/golden/, cited there), a closed form, a textbook or
library routine, an invariant, brute force on tiny inputs, or a statistical
law.  The negative controls plant known-wrong samplers in the oracle (its
ORACLE_NEG_* flags) and check that the statistical tests catch them.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _one_row_opd(q, p, c, lam=1.0):
    """Supervision loss for one row whose distributions are given as probabilities."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    V = q.size
    target = np.zeros((1, 2, V), dtype=np.float32)
    draft = np.zeros((1, 1, V), dtype=np.float32)
    with np.errstate(divide="ignore"):
        target[0, 0] = np.log(p)
        draft[0, 0] = np.log(q)
    return oracle.opd(target, draft, None, c, lam)


# ---------------------------------------------------------------- OPD forward


def test_worked_example_hard_label_and_reverse_kl():
    g = _gold("opd_worked_example.json")
    out = _one_row_opd(g["q"], g["p"], c=10.0)
    assert abs(out["loss_ce"][0] - g["l_hard"]) < 5e-4
    assert abs(out["loss_rkl"][0] - g["l_rkl"]) < 5e-4
    # Mixture alpha*l_hard + (1-alpha)*l_rkl as alpha*(CE + lambda*R), lambda=(1-alpha)/alpha.
    a = g["alpha"]
    mix = _one_row_opd(g["q"], g["p"], c=10.0, lam=(1 - a) / a)
    l = a * (mix["loss_ce"][0] + (1 - a) / a * mix["loss_rkl"][0])
    assert abs(l - g["l_opd"]) < 2.5e-4


@pytest.mark.parametrize("c", [0.1, 0.09, 0.085, 0.05, 0.01])
def test_worked_example_entrywise_clip_sweep(c):
    # Sweeping the clip threshold between the printed per-entry terms pins every
    # term: R(c) = sum_y min(term_y, c), negative terms never clipped.
    g = _gold("opd_worked_example.json")
    out = _one_row_opd(g["q"], g["p"], c=c)
    expect = sum(min(t, c) for t in g["terms"])
    assert abs(out["loss_rkl"][0] - expect) < 2.5e-3


def test_single_outlier_term():
    g = _gold("opd_worked_example.json")["outlier"]
    q = [g["q"], 1 - g["q"]]
    p = [g["p"], 1 - g["p"]]
    full = _one_row_opd(q, p, c=1e30)["loss_rkl"][0]
    neg_only = _one_row_opd(q, p, c=1e-12)["loss_rkl"][0]
    # R(inf) - R(0+) is the sum of the positive terms: here the single outlier.
    assert abs((full - neg_only) - g["term"]) < 5e-4


def test_unclipped_equals_textbook_kl_and_ce_equals_log_softmax():
    rng = np.random.default_rng(0)
    for V in (2, 7, 64, 1000):
        zp = rng.normal(0, 2, V).astype(np.float32)
        zq = rng.normal(0, 2, V).astype(np.float32)
        target = np.zeros((1, 2, V), np.float32)
        target[0, 0] = zp
        draft = zq.reshape(1, 1, V)
        out = oracle.opd(target, draft, None, clip_c=1e30, lam=1.0)
        p = special.softmax(zp.astype(np.float64))
        q = special.softmax(zq.astype(np.float64))
        assert abs(out["loss_rkl"][0] - special.rel_entr(q, p).sum()) < 1e-10
        assert out["loss_rkl"][0] >= 0
        xs = int(np.argmax(zp))
        assert abs(out["loss_ce"][0] + special.log_softmax(zq.astype(np.float64))[xs]) < 1e-10


def test_kl_zero_when_distributions_match():
    z = np.random.default_rng(1).normal(0, 1, 300).astype(np.float32)
    target = np.zeros((1, 2, 300), np.float32)
    target[0, 0] = z
    out = oracle.opd(target, z.reshape(1, 1, 300), None, clip_c=10.0, lam=1.0)
    assert abs(out["loss_rkl"][0]) < 1e-12
    # With p == q and lam == 0 the gradient is softmax - onehot(argmax).
    out0 = oracle.opd(target, z.reshape(1, 1, 300), None, clip_c=10.0, lam=0.0)
    ref = special.softmax(z.astype(np.float64))
    ref[np.argmax(z)] -= 1
    assert np.abs(out0["grad"][0] - ref).max() < 1e-12


def test_masked_entries():
    # p == 0 < q gives an infinite term: always clipped (adds c).  q == 0 gives 0.
    V = 5
    zp = np.array([0.0, 1.0, -np.inf, 0.5, 0.2], np.float32)
    zq = np.array([0.3, -np.inf, 0.1, 0.4, 0.0], np.float32)
    target = np.zeros((1, 2, V), np.float32)
    target[0, 0] = zp
    c = 0.7
    out = oracle.opd(target, zq.reshape(1, 1, V), None, clip_c=c, lam=1.0)
    p = special.softmax(zp.astype(np.float64))
    q = special.softmax(zq.astype(np.float64))
    terms = []
    for v in range(V):
        if q[v] == 0:
            terms.append(0.0)
        elif p[v] == 0:
            terms.append(np.inf)
        else:
            terms.append(q[v] * np.log(q[v] / p[v]))
    assert abs(out["loss_rkl"][0] - sum(min(t, c) for t in terms)) < 1e-12
    assert np.isfinite(out["grad"]).all()
    # The masked draft entry has no gradient except a possible hard-label -1.
    assert out["grad"][0, 1] == 0.0 or np.argmax(zp) == 1


def test_bf16_and_fp32_inputs_agree():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 3, (2, 3, 257)).astype(np.float32)
    zb = W.f32_to_bf16_bits(z)
    zr = W.bf16_bits_to_f32(zb)
    a = oracle.opd(zb, zb[:, :2].copy(), None, 0.05, 1.0)
    b = oracle.opd(zr, zr[:, :2].copy(), None, 0.05, 1.0)
    for key in ("loss_ce", "loss_rkl", "grad"):
        assert np.array_equal(a[key], b[key])


# --------------------------------------------------------------- OPD gradient


def _fd_logits(rng, V):
    # Multiples of 2^-12 so that z +- 2^-10 stays exact in fp32.
    return (np.round(rng.normal(0, 1.5, V) * 4096) / 4096).astype(np.float32)


@pytest.mark.parametrize("c,lam", [(10.0, 1.0), (0.05, 1.0), (0.02, 0.25), (1e30, 2.0)])
def test_gradient_matches_central_differences(c, lam):
    rng = np.random.default_rng(int(c * 1000) + 7)
    V = 24
    h = 2.0 ** -10
    for trial in range(30):
        zp = _fd_logits(rng, V)
        zq = _fd_logits(rng, V)
        # Keep every entry away from the clip kink (input selection only).
        p = special.softmax(zp.astype(np.float64))
        q = special.softmax(zq.astype(np.float64))
        f = q * np.log(q / p)
        if np.min(np.abs(f - c)) > 5e-3:
            break
    target = np.zeros((1, 2, V), np.float32)
    target[0, 0] = zp
    base = oracle.opd(target, zq.reshape(1, 1, V), None, c, lam)
    g = base["grad"][0]
    fd = np.zeros(V)
    for v in range(V):
        zplus = zq.copy()
        zminus = zq.copy()
        zplus[v] += h
        zminus[v] -= h
        lp_ = oracle.opd(target, zplus.reshape(1, 1, V), None, c, lam, with_grad=False)
        lm_ = oracle.opd(target, zminus.reshape(1, 1, V), None, c, lam, with_grad=False)
        Lp = lp_["loss_ce"][0] + lam * lp_["loss_rkl"][0]
        Lm = lm_["loss_ce"][0] + lam * lm_["loss_rkl"][0]
        fd[v] = (Lp - Lm) / (2 * h)
    assert np.abs(fd - g).max() < 2e-5
    assert abs(g.sum()) < 1e-12


def test_worked_example_gradient_by_differences():
    g = _gold("opd_worked_example.json")
    for c in (10.0, 0.01):
        out = _one_row_opd(g["q"], g["p"], c=c)
        grad = out["grad"][0]
        zq = np.log(np.asarray(g["q"])).astype(np.float32)
        zp = np.log(np.asarray(g["p"])).astype(np.float32)
        target = np.zeros((1, 2, 4), np.float32)
        target[0, 0] = zp
        h = 1e-3
        for v in range(4):
            d = np.zeros(4, np.float32)
            d[v] = h
            hi = oracle.opd(target, (zq + d).reshape(1, 1, 4), None, c, 1.0, with_grad=False)
            lo = oracle.opd(target, (zq - d).reshape(1, 1, 4), None, c, 1.0, with_grad=False)
            hh = float((zq + d)[v]) - float(zq[v])
            hl = float(zq[v]) - float((zq - d)[v])
            fd = ((hi["loss_ce"][0] + hi["loss_rkl"][0]) - (lo["loss_ce"][0] + lo["loss_rkl"][0])) / (hh + hl)
            assert abs(fd - grad[v]) < 2e-4


def test_packed_rows_and_row_selection():
    rng = np.random.default_rng(3)
    B, k, V = 3, 4, 33
    t = rng.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    d = rng.normal(0, 2, (B, k, V)).astype(np.float32)
    vl = np.array([2, 4, 1], np.int32)
    full = oracle.opd(t, d, vl, 0.1, 1.0)
    assert full["N"] == 7 and full["loss_ce"].shape == (7,)
    sel = oracle.opd(t, d, vl, 0.1, 1.0, rows=np.array([6, 0, 3]))
    for j, n in enumerate([6, 0, 3]):
        assert sel["loss_ce"][j] == full["loss_ce"][n]
        assert np.array_equal(sel["grad"][j], full["grad"][n])
    # Packed row 6 is request 2, position 0.
    one = oracle.opd(t[2:3], d[2:3], vl[2:3], 0.1, 1.0)
    assert one["loss_rkl"][0] == full["loss_rkl"][6]


# ------------------------------------------------------------------- verify


def _stack(batches):
    return (np.concatenate([b.target for b in batches]), np.concatenate([b.draft for b in batches]),
            np.concatenate([b.tokens for b in batches]), np.concatenate([b.verify_len for b in batches]),
            np.concatenate([b.uniforms for b in batches]))


def _check_structure(out, tokens, verify_len, k):
    A = out["accept_len"]
    toks = out["out_tokens"]
    assert ((A >= 0) & (A <= np.clip(verify_len, 1, k))).all()
    for b in range(A.shape[0]):
        a = A[b]
        assert np.array_equal(toks[b, :a], tokens[b, :a])
        assert toks[b, a] >= 0
        assert (toks[b, a + 1:] == -1).all()


@pytest.mark.parametrize("a", [0.8, 0.9])
def test_closed_form_accept_length(a):
    """DFlash notes eq. 3: tau = (1 - a^(m+1)) / (1 - a) for m = 15 drafts."""
    gold = _gold("tau_closed_form.json")
    m = gold["m"]
    exact = (1 - a ** (m + 1)) / (1 - a)
    printed = [cse["tau"] for cse in gold["cases"] if cse["a"] == a][0]
    assert abs(exact - printed) < 0.005
    wl = W.two_level(a, B=80000, k=m)
    bt = W.generate(wl)
    out = oracle.verify(bt.target, bt.draft, bt.tokens, bt.verify_len, bt.uniforms, T=1.0)
    _check_structure(out, bt.tokens, bt.verify_len, m)
    A = out["accept_len"].astype(np.float64)
    tau = (A + 1).mean()
    se = (A + 1).std() / np.sqrt(A.size)
    assert abs(tau - exact) < 4 * se
    # T1: tau = 1 + sum_j Pr(A >= j), exactly on the counts.
    assert abs(tau - (1 + sum((A >= j).mean() for j in range(1, m + 1)))) < 1e-9
    # T3: every accept test passes with probability sum_v min(p, q) = a.
    acc = out["margins"][:, :m] > 0
    rate = acc.mean(axis=0)
    assert np.abs(rate - a).max() < 4 * np.sqrt(a * (1 - a) / A.size)


def test_random_logits_accept_length_matches_exact_expectation():
    """Paired test on the tiny workload: A+1 against 1 + sum_j prod_{i<j} a_i."""
    wl = W.WORKLOADS[1]
    big = W.Workload(wl.name, B=20000, k=wl.k, V=wl.V, bf16=False, model=wl.model, T=wl.T,
                     p_scale=wl.p_scale, q_coef=wl.q_coef, sigmas=wl.sigmas, seed=wl.seed)
    bt = W.generate(big)
    out = oracle.verify(bt.target, bt.draft, bt.tokens, bt.verify_len, bt.uniforms, T=1.0)
    _check_structure(out, bt.tokens, bt.verify_len, wl.k)
    p = special.softmax(bt.target[:, :wl.k].astype(np.float64), axis=-1)
    q = special.softmax(bt.draft.astype(np.float64), axis=-1)
    a = np.minimum(p, q).sum(-1)                       # [B, k]
    surv = np.cumprod(a, axis=1)                        # Pr(A >= j), j = 1..k
    expect = 1 + surv.sum(axis=1)
    d = (out["accept_len"] + 1) - expect
    assert abs(d.mean()) < 4 * d.std() / np.sqrt(d.size)


def _fixed_logit_rounds(V, k, T, rounds, seed, q_coef=0.3, flags=0, ragged=False):
    wl = W.Workload("chi", B=1, k=k, V=V, bf16=False, model=W.WL_GAUSS, T=T, p_scale=1.5,
                    q_coef=q_coef, sigmas=(1.2, 1.2, 1.2), seed=seed, ragged=ragged)
    bts = [W.generate(wl, round=r, logits_round=0) for r in range(rounds)]
    t, d, tok, vl, uni = _stack(bts)
    out = oracle.verify(t, d, tok, vl, uni, T=T, flags=flags)
    return t, out


def _chi_square_pvalues(t, out, T):
    k = t.shape[1] - 1
    A = out["accept_len"]
    toks = out["out_tokens"]
    p_all = special.softmax(t[0].astype(np.float64) / T, axis=-1)
    pvals = []
    for j in range(k + 1):
        reached = A >= j
        n = int(reached.sum())
        if n < 200:
            continue
        obs = np.bincount(toks[reached, j], minlength=p_all.shape[1]).astype(np.float64)
        exp = n * p_all[j]
        order = np.argsort(exp)
        # merge the smallest bins until each expected count is >= 5
        o_m, e_m, acc_o, acc_e = [], [], 0.0, 0.0
        for v in order:
            acc_o += obs[v]
            acc_e += exp[v]
            if acc_e >= 5:
                o_m.append(acc_o)
                e_m.append(acc_e)
                acc_o = acc_e = 0.0
        if acc_e > 0:
            if e_m:
                o_m[-1] += acc_o
                e_m[-1] += acc_e
        if len(e_m) < 2:
            continue
        pvals.append(stats.chisquare(o_m, e_m).pvalue)
    return pvals


@pytest.mark.parametrize("V,T,ragged", [(8, 1.0, False), (64, 1.0, False), (8, 0.5, False),
                                         (8, 1.0, True)])
def test_emitted_tokens_follow_the_target(V, T, ragged):
    """Losslessness (DFlash notes eq. 8): each emitted token ~ p at its position.
    With ragged verify lengths the bonus comes from target row L, not row k."""
    t, out = _fixed_logit_rounds(V, k=3, T=T, rounds=20000, seed=101 + V, ragged=ragged)
    pv = _chi_square_pvalues(t, out, T)
    assert len(pv) >= 2
    assert min(pv) > 1e-3 / len(pv)


@pytest.mark.parametrize("flags", [oracle.NEG_RESAMPLE_TARGET, oracle.NEG_ARGMAX])
def test_negative_controls_fail_the_chi_square(flags):
    t, out = _fixed_logit_rounds(8, k=3, T=1.0, rounds=20000, seed=109, flags=flags)
    pv = _chi_square_pvalues(t, out, 1.0)
    assert min(pv) < 1e-6


def test_residual_example_always_corrects_to_the_missing_mass():
    g = _gold("residual_example.json")
    n = 20000
    V = 3
    target = np.zeros((n, 2, V), np.float32)
    draft = np.zeros((n, 1, V), np.float32)
    target[:, 0] = np.log(g["p"])
    target[:, 1] = np.log(g["p"])
    draft[:, 0] = np.log(g["q"])
    wl = W.Workload("r", B=n, k=1, V=V, bf16=False, model=W.WL_GAUSS, T=1.0, seed=55)
    bt = W.generate(wl, with_tokens=False)          # verifier uniforms only
    # draft tokens ~ q, drawn with numpy (inputs only)
    tokens = np.random.default_rng(5).choice(V, size=(n, 1), p=g["q"]).astype(np.int32)
    out = oracle.verify(target, draft, tokens, None, bt.uniforms, T=1.0)
    rejected = out["accept_len"] == 0
    assert rejected.any()
    assert (out["out_tokens"][rejected, 0] == g["correction_token"]).all()
    rate = 1 - rejected.mean()
    assert abs(rate - g["accepted_mass"]) < 4 * np.sqrt(0.21 / n)


def test_inverse_cdf_edges():
    # Residual with mass on ids 2 and 4 only; bonus row with zero mass at both ends.
    V = 6
    p = np.array([0.1, 0.1, 0.4, 0.1, 0.3, 0.0])
    q = np.array([0.2, 0.2, 0.1, 0.2, 0.1, 0.2])
    target = np.zeros((2, 2, V), np.float32)
    with np.errstate(divide="ignore"):
        target[:, 0] = np.log(p)
        target[:, 1] = np.log([0.0, 0.25, 0.25, 0.25, 0.25, 0.0])
    draft = np.zeros((2, 1, V), np.float32)
    draft[:, 0] = np.log(q)
    top = np.float32(1.0) - np.float32(2.0 ** -24)
    # rejection of token 5 (p=0) is certain
    tokens = np.array([[5], [5]], np.int32)
    uni = np.array([[0.5, 0.0], [0.5, top]], np.float32)
    out = oracle.verify(target, draft, tokens, None, uni, T=1.0)
    assert list(out["accept_len"]) == [0, 0]
    assert out["out_tokens"][0, 0] == 2 and out["out_tokens"][1, 0] == 4
    # bonus: token 2 has p == q so it is always accepted
    tokens = np.array([[2], [2]], np.int32)
    target[:, 0] = np.log(q)
    uni = np.array([[0.99, 0.0], [0.99, top]], np.float32)
    out = oracle.verify(target, draft, tokens, None, uni, T=1.0)
    assert list(out["accept_len"]) == [1, 1]
    assert out["out_tokens"][0, 1] == 1 and out["out_tokens"][1, 1] == 4


def test_degenerate_vocabulary_of_one():
    target = np.zeros((3, 5, 1), np.float32)
    draft = np.zeros((3, 4, 1), np.float32)
    tokens = np.zeros((3, 4), np.int32)
    uni = np.full((3, 5), 0.999, np.float32)
    for T in (0.0, 1.0):
        out = oracle.verify(target, draft, tokens, np.array([1, 4, 2], np.int32), uni, T=T)
        assert list(out["accept_len"]) == [1, 4, 2]
        assert (out["out_tokens"][0] == [0, 0, -1, -1, -1]).all()


def test_verify_len_is_clamped():
    rng = np.random.default_rng(4)
    t = rng.normal(0, 1, (2, 4, 10)).astype(np.float32)
    d = t[:, :3].copy()
    tok = np.argmax(d, -1).astype(np.int32)
    uni = np.full((2, 4), 0.5, np.float32)
    out = oracle.verify(t, d, tok, np.array([0, 99], np.int32), uni, T=1.0)
    # identical distributions always accept: A = clamped L
    assert list(out["accept_len"]) == [1, 3]


# -------------------------------------------------------------------- greedy


def _ar_greedy(target, tokens, L):
    """Brute-force autoregressive greedy decoding with the drafts as proposals."""
    emitted = []
    for j in range(L + 1):
        choice = int(np.argmax(target[j]))   # numpy: first maximum on ties
        if j < L and tokens[j] == choice:
            emitted.append(choice)
            continue
        emitted.append(choice)
        break
    return emitted


def test_greedy_matches_brute_force():
    rng = np.random.default_rng(11)
    B, k, V = 400, 6, 12
    # Coarse logits so that ties happen often; drafts copy the target argmax with
    # probability 0.7 per position so long prefixes occur.
    t = rng.integers(-3, 4, (B, k + 1, V)).astype(np.float32)
    am = np.argmax(t[:, :k], -1)
    noise = rng.integers(0, V, (B, k))
    tok = np.where(rng.random((B, k)) < 0.7, am, noise).astype(np.int32)
    vl = rng.integers(1, k + 1, B).astype(np.int32)
    uni = rng.random((B, k + 1)).astype(np.float32)
    out = oracle.verify(t, None, tok, vl, uni, T=0.0)
    lens = []
    for b in range(B):
        em = _ar_greedy(t[b], tok[b], int(vl[b]))
        a = int(out["accept_len"][b])
        lens.append(a)
        assert list(out["out_tokens"][b, :a + 1]) == em
        assert (out["out_tokens"][b, a + 1:] == -1).all()
    assert max(lens) == k and min(lens) == 0


def test_greedy_ties_take_the_lowest_index():
    t = np.zeros((2, 3, 5), np.float32)          # all-equal rows: argmax is 0
    t[1, :, 3] = 2.0
    t[1, :, 1] = 2.0                             # duplicate maxima at 1 and 3
    tok = np.array([[0, 0], [1, 3]], np.int32)
    out = oracle.verify(t, None, tok, None, np.zeros((2, 3), np.float32), T=0.0)
    assert list(out["out_tokens"][0]) == [0, 0, 0]
    assert list(out["accept_len"]) == [2, 1]
    assert list(out["out_tokens"][1]) == [1, 1, -1]


# ------------------------------------ hand-computed margins and the Z == 0 case
#
# DFlash reading notes, section 5.2: accept iff u q(x) < p(x) (eq. 6); on a
# rejection draw from the residual [p - q]_+ / Z (eq. 7), with no rejection
# possible when Z = 0; the bonus token comes from the target row after the last
# draft (Algorithm 1, step 9).  The inverse CDF takes the smallest id whose
# running sum exceeds u Z.  The values below are worked by hand on V = 4.

def _one_request(p_rows, q_row, token, u_acc, u_draw):
    """One request, k = 1: target rows (position 0, bonus row), one draft row."""
    with np.errstate(divide="ignore"):
        target = np.log(np.asarray(p_rows, np.float64)).astype(np.float32)[None]
        draft = np.log(np.asarray([q_row], np.float64)).astype(np.float32)[None]
    tok = np.array([[token]], np.int32)
    uni = np.array([[u_acc, u_draw]], np.float32)
    return oracle.verify(target, draft, tok, None, uni, T=1.0)


def test_bonus_draw_margin_by_hand():
    # q = p on row 0, so the draft is accepted; the bonus row has cumulative
    # mass 0.1, 0.3, 0.6, 1.0 and u = 0.35 lands in token 2's interval (0.3, 0.6]:
    # distance to its nearer boundary 0.05, total mass 1.
    p0 = [0.1, 0.2, 0.3, 0.4]
    out = _one_request([p0, [0.1, 0.2, 0.3, 0.4]], p0, token=3, u_acc=0.5, u_draw=0.35)
    assert out["accept_len"][0] == 1 and list(out["out_tokens"][0]) == [3, 2]
    assert abs(out["margins"][0, 0] - (0.4 - 0.5 * 0.4)) < 1e-7            # p(x) - u q(x) = 0.2
    assert np.allclose(out["accept_pq"][0, 0], [0.4, 0.2], atol=1e-7)
    assert abs(out["margins"][0, 1] - 0.05) < 1e-7
    assert np.allclose(out["sample_info"][0], [1.0, 0.35, 0.3, 0.6], atol=1e-7)


@pytest.mark.parametrize("u_draw,token,margin,before,after", [(0.6, 1, 0.15, 0.0, 0.3), (0.9, 3, 0.1, 0.3, 0.4)])
def test_residual_draw_margin_by_hand(u_draw, token, margin, before, after):
    # p = (0.1, 0.4, 0.2, 0.3), q = (0.3, 0.1, 0.4, 0.2): residual (0, 0.3, 0, 0.1),
    # Z = 0.4.  Draft token 0 with u = 0.9: 0.9 * 0.3 = 0.27 > 0.1, rejected with
    # margin -0.17.  u_draw = 0.6: threshold 0.24 falls in token 1's interval
    # (0, 0.3], margin min(0.24, 0.06) / 0.4 = 0.15; u_draw = 0.9: threshold 0.36
    # in token 3's interval (0.3, 0.4], margin min(0.06, 0.04) / 0.4 = 0.1.
    p = [0.1, 0.4, 0.2, 0.3]
    q = [0.3, 0.1, 0.4, 0.2]
    out = _one_request([p, p], q, token=0, u_acc=0.9, u_draw=u_draw)
    assert out["accept_len"][0] == 0 and list(out["out_tokens"][0]) == [token, -1]
    assert abs(out["margins"][0, 0] - (-0.17)) < 1e-7
    assert np.allclose(out["accept_pq"][0, 0], [0.1, 0.27], atol=1e-7)
    assert abs(out["margins"][0, 1] - margin) < 1e-6
    assert np.allclose(out["sample_info"][0], [0.4, 0.4 * u_draw, before, after], atol=1e-7)


def test_zero_residual_falls_back_to_the_target_row():
    # p == q exactly with the draft on a token of zero mass: the test 0 < 0
    # fails, so the draft is rejected although Z = sum [p - q]_+ = 0.  The draw
    # then comes from p itself (total mass 1): u = 0.25 in token 1's interval
    # (0.1, 0.3], margin min(0.15, 0.05) = 0.05.
    p = [0.1, 0.2, 0.7, 0.0]
    out = _one_request([p, [0.25, 0.25, 0.25, 0.25]], p, token=3, u_acc=0.5, u_draw=0.25)
    assert out["accept_len"][0] == 0 and list(out["out_tokens"][0]) == [1, -1]
    assert out["margins"][0, 0] == 0.0
    assert abs(out["margins"][0, 1] - 0.05) < 1e-7
    assert np.allclose(out["sample_info"][0], [1.0, 0.25, 0.1, 0.3], atol=1e-7)
