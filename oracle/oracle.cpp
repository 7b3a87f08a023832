// CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, double-precision reference for the verify-and-supervise pass.
// Only the tests, the package smoke check and the benchmark's CPU-baseline leg
// may load it.  It shares no code, header or table with the GPU library and
// never reads anything the GPU library produced.
//
// Sources (pages as titled; citations name the section or equation):
//  * "AdaFlash: Taming Variance in Diffusion Speculative Decoding" (review, EN),
//    section "Speculative Decoding: The Basic Idea", steps 3-4: accept draft x_i
//    with probability min(1, p(x_i)/q(x_i)); keep the drafts before the first
//    rejection; resample the rejected position from the renormalised residual
//    max(0, p - q).
//  * "DFlash 阅读笔记：并行起草、目标特征与精确验证" (DFlash reading notes),
//    section 5.1 (greedy mode: compare with the target argmax, stop at the first
//    mismatch and emit the target's choice, bonus token if all match) and
//    section 5.2, eqs. 6-8 (acceptance min(1, p/q), residual [p-q]_+ / Z,
//    losslessness), plus Algorithm 1 step 9 (bonus token from the target).
//  * AdaFlash review, "The Reverse-KL + Hard-Label Mixture Loss, Derived"
//    (l_hard on the target's top-1 token) and "Entry-Wise Divergence Clipping,
//    Derived" (Algorithm 2 and its closed form: each per-entry term
//    q log(q/p) is capped at the threshold before summing over the vocabulary);
//    reverse-KL temperature 1.0 from its "Reproducibility Notes".
//
// Readings where the pages leave a step open (each is listed in the design doc):
//  * Accept test is strict and division free: accept iff u * q(x) < p(x).
//  * One uniform per accept test, and one more (uniforms[b][k]) for the single
//    correction-or-bonus draw.
//  * Inverse CDF: scan token ids ascending; the token is the smallest v whose
//    running sum exceeds the threshold (strict); if rounding leaves no such v,
//    take the last v with positive mass.  The residual threshold is u * Z with
//    Z the summed residual; if Z == 0 the draw falls back to p_A.
//  * The bonus row is target row L (the request's verify length), not row k.
//  * Every argmax takes the lowest index on ties.
//  * Per-row supervision loss l = CE + lambda * R_c, with R_c the entry-wise
//    clipped reverse KL(q || p) at temperature 1 (clip threshold c) and CE the
//    hard-label cross entropy on the target's top-1 token.  The paper's mixture
//    alpha*l_hard + (1-alpha)*l_rkl^clip is alpha times this with
//    lambda = (1-alpha)/alpha.  Losses are per row; the 1/k mean is left to the
//    caller.  An entry is clipped iff its term exceeds c; clipped entries add c
//    to R_c and nothing to the gradient.  A term with q == 0 is 0; a term with
//    p == 0 < q is +inf (always clipped).
//  * Gradient with respect to the draft logits of row i (derived by the chain
//    rule; the pages print no gradient):
//      d l / d z_v = (q_v - [v == x*]) + lambda * q_v * ([v in U](lq_v - lp_v + 1) - S),
//      S = sum_{w in U} (f_w + q_w),  f_w = q_w (lq_w - lp_w),  U = {w : f_w <= c}.
//
// Nothing here is blocked, fused or reordered: every row is a plain ascending
// loop in double.  Requests (verify) and rows (supervision) are independent,
// so they are spread over std::thread workers.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

const double kInf = std::numeric_limits<double>::infinity();
const double kNaN = std::numeric_limits<double>::quiet_NaN();

// Logit element as double (bf16 and fp32 both convert exactly).
double logit(int dtype, const void* base, int64_t row, int V, int v) {
  if (dtype == 1) {
    uint16_t h = ((const uint16_t*)base)[row * (int64_t)V + v];
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
  }
  return (double)((const float*)base)[row * (int64_t)V + v];
}

void row_values(int dtype, const void* base, int64_t row, int V, std::vector<double>& z) {
  z.resize(V);
  for (int v = 0; v < V; ++v) z[v] = logit(dtype, base, row, V, v);
}

// softmax(z / T) in double: m = max(z/T), probs = exp(z/T - m) / sum.
void softmax_T(const std::vector<double>& z, double T, std::vector<double>& prob) {
  const int V = (int)z.size();
  double m = -kInf;
  for (int v = 0; v < V; ++v) m = std::max(m, z[v] / T);
  double s = 0.0;
  prob.resize(V);
  for (int v = 0; v < V; ++v) {
    prob[v] = std::exp(z[v] / T - m);
    s += prob[v];
  }
  for (int v = 0; v < V; ++v) prob[v] /= s;
}

int argmax_lowest(const std::vector<double>& z) {
  int best = 0;
  for (int v = 1; v < (int)z.size(); ++v)
    if (z[v] > z[best]) best = v;
  return best;
}

// Smallest v whose running sum of w exceeds thr; else the last v with w > 0.
// Reports the running sum just before and just after the chosen token.
int inverse_cdf(const std::vector<double>& w, double thr, double* cum_before, double* cum_at) {
  double cum = 0.0;
  int last_pos = -1;
  double last_before = 0.0;
  for (int v = 0; v < (int)w.size(); ++v) {
    double before = cum;
    cum += w[v];
    if (w[v] > 0.0) {
      last_pos = v;
      last_before = before;
    }
    if (cum > thr) {
      *cum_before = before;
      *cum_at = cum;
      return v;
    }
  }
  if (last_pos < 0) last_pos = 0;
  *cum_before = last_before;
  *cum_at = cum;
  return last_pos;
}

template <typename F>
void parallel_for(int64_t n, int nthreads, F&& fn) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  int nt = (int)std::min<int64_t>(nthreads, n);
  for (int t = 0; t < nt; ++t)
    pool.emplace_back([&] {
      for (;;) {
        int64_t i = next.fetch_add(1);
        if (i >= n) break;
        fn(i);
      }
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Negative-control variants, used only by tests that show the statistical
// checks can tell a wrong sampler from the right one.
enum {
  ORACLE_NEG_RESAMPLE_TARGET = 1,  // on rejection, draw from p_A instead of the residual
  ORACLE_NEG_ARGMAX = 2,           // on rejection, emit argmax p_A
};

// Verification of one batch.
//   target [B, k+1, V], draft [B, k, V] (dtype 0: fp32, 1: bf16 bits), tokens [B, k],
//   verify_len [B] (clamped to [1, k]), uniforms [B, k+1].
//   Outputs: accept_len [B]; out_tokens [B, k+1] (accepted drafts, then the correction
//   or bonus token, then -1); margins [B, k+1] (p(x_i) - u_i q(x_i) for i < L, NaN
//   elsewhere and in greedy mode; margins[b][k] is the sample's distance to the nearest
//   CDF boundary of the chosen token divided by the total mass; NaN in greedy mode);
//   sample_info [B, 4] = {total mass Z, threshold, running sum before token, after token};
//   accept_pq [B, k, 2] (may be NULL) = {p(x_i), u_i q(x_i)} of every accept test
//   i < L (the two sides whose difference is the margin), NaN elsewhere and in
//   greedy mode.
int oracle_verify(int dtype, const void* target, const void* draft, const int32_t* tokens,
                  const int32_t* verify_len, const float* uniforms, int B, int k, int V, double T,
                  int32_t* accept_len, int32_t* out_tokens, double* margins, double* sample_info,
                  double* accept_pq, int flags, int nthreads) {
  if (B < 0 || k < 1 || V < 1 || !(T >= 0.0)) return -1;
  parallel_for(B, nthreads, [&](int64_t b) {
    int L = verify_len ? verify_len[b] : k;
    if (L < 1) L = 1;
    if (L > k) L = k;
    const float* u = uniforms + b * (int64_t)(k + 1);
    std::vector<double> zp, zq, p, q;
    int A = L;
    for (int i = 0; i <= k; ++i) margins[b * (k + 1) + i] = kNaN;
    if (accept_pq)
      for (int i = 0; i < 2 * k; ++i) accept_pq[b * 2 * k + i] = kNaN;
    auto record = [&](int i, double px, double uqx) {
      margins[b * (k + 1) + i] = px - uqx;
      if (accept_pq) {
        accept_pq[(b * k + i) * 2 + 0] = px;
        accept_pq[(b * k + i) * 2 + 1] = uqx;
      }
    };

    // Accept tests, left to right; stop at the first rejection.
    for (int i = 0; i < L; ++i) {
      int x = tokens[b * k + i];
      if (x < 0) x = 0;
      if (x >= V) x = V - 1;
      row_values(dtype, target, b * (int64_t)(k + 1) + i, V, zp);
      bool accept;
      if (T == 0.0) {
        accept = (x == argmax_lowest(zp));
      } else {
        row_values(dtype, draft, b * (int64_t)k + i, V, zq);
        softmax_T(zp, T, p);
        softmax_T(zq, T, q);
        accept = (double)u[i] * q[x] < p[x];
        record(i, p[x], (double)u[i] * q[x]);
      }
      if (!accept) {
        A = i;
        break;
      }
    }
    // Margins of the tests after the first rejection are still defined (the
    // GPU evaluates every test in parallel); report them for near-tie checks.
    if (T > 0.0) {
      for (int i = A + 1; i < L; ++i) {
        int x = tokens[b * k + i];
        if (x < 0) x = 0;
        if (x >= V) x = V - 1;
        row_values(dtype, target, b * (int64_t)(k + 1) + i, V, zp);
        row_values(dtype, draft, b * (int64_t)k + i, V, zq);
        softmax_T(zp, T, p);
        softmax_T(zq, T, q);
        record(i, p[x], (double)u[i] * q[x]);
      }
    }

    // Correction (A < L) or bonus (A == L) token.
    const double us = (double)u[k];
    int token;
    double Z = 1.0, thr = 0.0, cb = 0.0, ca = 0.0;
    row_values(dtype, target, b * (int64_t)(k + 1) + A, V, zp);
    if (T == 0.0) {
      token = argmax_lowest(zp);
    } else if (A < L) {
      row_values(dtype, draft, b * (int64_t)k + A, V, zq);
      softmax_T(zp, T, p);
      softmax_T(zq, T, q);
      if (flags & ORACLE_NEG_ARGMAX) {
        token = argmax_lowest(zp);
      } else if (flags & ORACLE_NEG_RESAMPLE_TARGET) {
        thr = us;
        token = inverse_cdf(p, thr, &cb, &ca);
      } else {
        std::vector<double> r(V);
        Z = 0.0;
        for (int v = 0; v < V; ++v) {
          r[v] = std::max(0.0, p[v] - q[v]);
          Z += r[v];
        }
        if (Z > 0.0) {
          thr = us * Z;
          token = inverse_cdf(r, thr, &cb, &ca);
        } else {
          Z = 1.0;
          thr = us;
          token = inverse_cdf(p, thr, &cb, &ca);
        }
      }
    } else {
      softmax_T(zp, T, p);
      thr = us;
      token = inverse_cdf(p, thr, &cb, &ca);
    }
    if (T > 0.0) margins[b * (k + 1) + k] = std::min(thr - cb, ca - thr) / Z;

    accept_len[b] = A;
    for (int i = 0; i <= k; ++i) {
      int32_t t = -1;
      if (i < A) t = std::min(std::max(tokens[b * k + i], 0), V - 1);
      else if (i == A) t = token;
      out_tokens[b * (k + 1) + i] = t;
    }
    if (sample_info) {
      double* si = sample_info + 4 * b;
      si[0] = (T == 0.0) ? kNaN : Z;
      si[1] = (T == 0.0) ? kNaN : thr;
      si[2] = (T == 0.0) ? kNaN : cb;
      si[3] = (T == 0.0) ? kNaN : ca;
    }
  });
  return 0;
}

// Supervision loss and gradient for packed rows.
//   Packed row n is (b, i) with i < L_b, in request order (L_b = verify_len[b]
//   clamped to [1, k], or k when verify_len is NULL).  `rows` lists the packed
//   rows to evaluate (NULL: all of them, in order); results are written at the
//   position of each row in that list.  loss_ce and loss_rkl [nrows] are
//   required when any row is evaluated; grad [nrows, V] may be NULL.  With
//   rows non-NULL and nrows == 0 nothing is evaluated (only N is returned).
//   Returns the number of packed rows N, or a negative value on bad arguments.
int64_t oracle_opd(int dtype, const void* target, const void* draft, const int32_t* verify_len,
                   int B, int k, int V, double c, double lambda, const int64_t* rows, int64_t nrows,
                   double* loss_ce, double* loss_rkl, double* grad, int nthreads) {
  if (B < 0 || k < 1 || V < 1 || !(c > 0.0) || !(lambda >= 0.0)) return -1;
  std::vector<int64_t> row_b, row_i;
  for (int b = 0; b < B; ++b) {
    int L = verify_len ? verify_len[b] : k;
    if (L < 1) L = 1;
    if (L > k) L = k;
    for (int i = 0; i < L; ++i) {
      row_b.push_back(b);
      row_i.push_back(i);
    }
  }
  const int64_t N = (int64_t)row_b.size();
  const int64_t n_eval = rows ? nrows : N;
  if (n_eval < 0 || (n_eval > 0 && (!loss_ce || !loss_rkl))) return -1;
  for (int64_t j = 0; j < n_eval; ++j)
    if (rows && (rows[j] < 0 || rows[j] >= N)) return -2;

  parallel_for(n_eval, nthreads, [&](int64_t j) {
    const int64_t n = rows ? rows[j] : j;
    const int64_t b = row_b[n], i = row_i[n];
    std::vector<double> zp, zq;
    row_values(dtype, target, b * (k + 1) + i, V, zp);
    row_values(dtype, draft, b * k + i, V, zq);

    // Log-normalisers at temperature 1.
    double mq = -kInf, mp = -kInf;
    for (int v = 0; v < V; ++v) {
      mq = std::max(mq, zq[v]);
      mp = std::max(mp, zp[v]);
    }
    double sq = 0.0, sp = 0.0;
    for (int v = 0; v < V; ++v) {
      sq += std::exp(zq[v] - mq);
      sp += std::exp(zp[v] - mp);
    }
    const double lse_q = mq + std::log(sq), lse_p = mp + std::log(sp);
    const int xs = argmax_lowest(zp);  // target top-1 token

    // Hard-label cross entropy on the target's top-1 token.
    const double ce = lse_q - zq[xs];

    // Entry-wise clipped reverse KL and the sum S over unclipped entries.
    double R = 0.0, S = 0.0;
    std::vector<char> inU(V);
    std::vector<double> qv(V), lq(V), lp(V);
    for (int v = 0; v < V; ++v) {
      lq[v] = zq[v] - lse_q;
      lp[v] = zp[v] - lse_p;
      qv[v] = std::exp(lq[v]);
      double f;
      if (qv[v] == 0.0) f = 0.0;
      else if (lp[v] == -kInf) f = kInf;
      else f = qv[v] * (lq[v] - lp[v]);
      if (f <= c) {
        inU[v] = 1;
        R += f;
        S += f + qv[v];
      } else {
        inU[v] = 0;
        R += c;
      }
    }
    loss_ce[j] = ce;
    loss_rkl[j] = R;
    if (grad) {
      double* g = grad + j * (int64_t)V;
      for (int v = 0; v < V; ++v) {
        double hard = qv[v] - (v == xs ? 1.0 : 0.0);
        double soft;
        if (qv[v] == 0.0) soft = 0.0;
        else if (inU[v]) soft = qv[v] * ((lq[v] - lp[v] + 1.0) - S);
        else soft = qv[v] * (-S);
        g[v] = hard + lambda * soft;
      }
    }
  });
  return N;
}

}  // extern "C"
