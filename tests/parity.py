"""Comparison of GPU outputs with the CPU oracle (pure numpy; no GPU).

Used by the GPU parity tests and by the benchmark's oracle leg, which prints
the same counts in its JSON line.

Accept tests (DFlash reading notes, section 5.2, eq. 6: accept iff
u q(x) < p(x)).  The GPU decides in fp32, the oracle in double, so a decision
may differ only where the two sides are nearly equal.  Two bands are counted
for every request, over the tests that decide its accept length (positions
0 .. min(A_gpu, A_oracle)):

* the absolute band |p - u q| < 1e-5, and
* the relative band |p - u q| < 1e-5 max(p, u q).

At V = 151936 many p and u q are far below 1e-5, so the absolute band holds
most requests; a difference of accept length is therefore accepted only
inside the relative band.  Draws (eqs. 7-8, inverse CDF of the residual or of
the bonus row): a token may differ only where the oracle's threshold lies
within 1e-5 of the total mass from a CDF boundary of its token.
"""
from __future__ import annotations

import numpy as np

ABS_BAND = 1e-5   # |p - u q| for accept tests
REL_BAND = 1e-5   # |p - u q| / max(p, u q) for accept tests
DRAW_BAND = 1e-5  # distance of the draw threshold to a CDF boundary, over the total mass


def verify_counts(g: dict, r: dict, T: float, tokens: np.ndarray, verify_len: np.ndarray, k: int) -> dict:
    """Checks accept lengths and emitted tokens of the GPU (g) against the
    oracle (r) and returns the counts.  Greedy (T == 0): bit-exact.  Sampled:
    every difference must fall in the relative accept band at the first
    position where the two decisions part, or (same accept length) in the draw
    band.  Raises AssertionError otherwise, and on any structural error of the
    GPU output (accept length out of range, accepted prefix not the drafts,
    padding not -1)."""
    A_g, A_r = np.asarray(g["accept_len"]), np.asarray(r["accept_len"])
    tok_g, tok_r = np.asarray(g["out_tokens"]), np.asarray(r["out_tokens"])
    B = A_r.shape[0]
    L = np.clip(verify_len, 1, k)
    out = {"requests": int(B), "in_abs_band": 0, "in_rel_band": 0, "near_draw": 0, "flips": 0,
           "accept_flips": 0, "draw_flips": 0}
    for b in range(B):
        a = int(A_g[b])
        assert 0 <= a <= L[b], f"request {b}: accept length {a} outside [0, {L[b]}]"
        assert np.array_equal(tok_g[b, :a], tokens[b, :a]), f"request {b}: accepted prefix is not the drafts"
        assert (tok_g[b, a + 1:] == -1).all(), f"request {b}: padding after the emitted token"
        assert 0 <= tok_g[b, a], f"request {b}: no emitted token"
    if T == 0:
        assert np.array_equal(A_g, A_r), np.nonzero(A_g != A_r)[0][:10]
        assert np.array_equal(tok_g, tok_r)
        return out
    mr = r["margins"]
    pq = r["accept_pq"]
    for b in range(B):
        n = min(int(A_r[b]), int(A_g[b])) + 1
        n = min(n, int(L[b]))
        m = np.abs(mr[b, :n])
        scale = np.maximum(pq[b, :n, 0], pq[b, :n, 1])
        abs_b = m < ABS_BAND
        rel_b = m < REL_BAND * scale
        near_draw = mr[b, k] < DRAW_BAND
        out["in_abs_band"] += int(abs_b.any())
        out["in_rel_band"] += int(rel_b.any())
        out["near_draw"] += int(near_draw)
        if A_g[b] == A_r[b] and np.array_equal(tok_g[b], tok_r[b]):
            continue
        out["flips"] += 1
        if A_g[b] != A_r[b]:
            a = min(int(A_g[b]), int(A_r[b]))
            out["accept_flips"] += 1
            assert rel_b[a], (f"request {b}: accept length {A_g[b]} vs oracle {A_r[b]}; margin {mr[b, a]:.3e} "
                              f"with p = {pq[b, a, 0]:.3e}, u q = {pq[b, a, 1]:.3e} is outside the relative band")
        else:
            out["draw_flips"] += 1
            a = int(A_r[b])
            assert near_draw, (f"request {b}: token {tok_g[b, a]} vs oracle {tok_r[b, a]} "
                               f"(draw margin {mr[b, k]:.3e})")
    return out


def add_counts(total: dict, part: dict) -> dict:
    for key, v in part.items():
        total[key] = total.get(key, 0) + v
    return total


def margin_error(g_margins: np.ndarray, r_margins: np.ndarray, verify_len: np.ndarray, k: int) -> float:
    """Largest |GPU margin - oracle margin| over the accept tests i < L_b (the
    GPU writes NaN at i >= L_b, which is checked too)."""
    L = np.clip(verify_len, 1, k)
    worst = 0.0
    for b in range(g_margins.shape[0]):
        m_g = g_margins[b, :L[b]].astype(np.float64)
        worst = max(worst, float(np.abs(m_g - r_margins[b, :L[b]]).max()))
        assert np.isnan(g_margins[b, L[b]:k]).all(), f"request {b}: margins past the verify length"
    return worst


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def loss_excess(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Error beyond 1e-3 relative + 1e-6 absolute; equal infinities match."""
    g = g.astype(np.float64)
    same_inf = np.isinf(r) & (g == r)
    with np.errstate(invalid="ignore"):
        e = np.abs(g - r) - (1e-3 * np.abs(r) + 1e-6)
    e = np.where(same_inf, -1.0, e)
    return np.where(np.isnan(e), np.inf, e)


def loss_rel_error(g: np.ndarray, r: np.ndarray) -> float:
    """Largest |g - r| / max(|r|, 1e-3) over finite pairs (for reports)."""
    g = g.astype(np.float64)
    fin = np.isfinite(r) & np.isfinite(g)
    if not fin.any():
        return 0.0
    return float((np.abs(g[fin] - r[fin]) / np.maximum(np.abs(r[fin]), 1e-3)).max())


def grad_tolerance(g_ref: np.ndarray, bf16: bool = True) -> np.ndarray:
    """2e-3 absolute, or one bf16 ulp of the reference where that is larger."""
    return np.maximum(2e-3, bf16_ulp(g_ref)) if bf16 else 2e-5 + 1e-5 * np.abs(g_ref)


def grad_errors(g_gpu: np.ndarray, g_ref: np.ndarray, bf16: bool = True) -> dict:
    err = np.abs(g_gpu.astype(np.float64) - g_ref)
    tol = grad_tolerance(g_ref, bf16)
    over = ~(err <= tol)  # (an undefined entry counts as over)
    return {"max_abs": float(np.nanmax(err)) if err.size and not np.isnan(err).all() else 0.0,
            "over_tol": int(over.sum()), "undefined": int(np.isnan(err).sum()),
            "ulp_entries": int((np.abs(g_ref) >= 0.5).sum())}
