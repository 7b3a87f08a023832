// Seeded synthetic input generator for the verify-and-supervise pass.
//
// This module only synthesises inputs: logits that stand in for a target model
// and a diffusion drafter, draft tokens drawn from the drafter's own
// distribution, per-request verify lengths and the uniforms the verifier
// consumes.  It contains none of the verifier's or the loss's arithmetic and
// is shared by the CPU oracle side and the GPU side only through the arrays it
// writes.
//
// Random numbers: Philox4x32-10, the counter-based generator of Salmon, Moraes,
// Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
// Counter layout: (element block, row id, round, stream); key: 64-bit seed.
//   stream 0: target-logit normals       stream 1: draft-logit noise
//   stream 2: draft-token Gumbel noise   stream 3: verifier uniforms
//   stream 4: verify lengths             stream 5: per-request noise level
//
// Normals: Box-Muller in double on (0,1] uniforms.  Each logit is computed in
// double, rounded once to fp32 and, for bf16 outputs, once more to bf16 (RNE).
// Draft tokens: Gumbel-max sampling from softmax(z_q / T) of the rounded
// logits (argmax, lowest index on ties, when T == 0).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <atomic>
#include <limits>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;  // Philox multipliers
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;  // Weyl key increments

inline void philox4x32_10(const uint32_t in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t a = (uint64_t)kM0 * c0;
    uint64_t b = (uint64_t)kM1 * c2;
    uint32_t n0 = (uint32_t)(b >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)b;
    uint32_t n2 = (uint32_t)(a >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)a;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += kW0; k1 += kW1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

inline void draw(uint64_t seed, uint32_t blk, uint32_t row, uint32_t round, uint32_t stream,
                 uint32_t out[4]) {
  uint32_t ctr[4] = {blk, row, round, stream};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  philox4x32_10(ctr, key, out);
}

// (0,1] uniform from 32 random bits, in double.
inline double u01_open0(uint32_t x) { return ((double)x + 1.0) * (1.0 / 4294967296.0); }
// [0,1) uniform with 24 bits, exactly representable in fp32.
inline float u24(uint32_t x) { return (float)(x >> 8) * (1.0f / 16777216.0f); }

inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Four standard normals from one Philox block (two Box-Muller pairs).
inline void normals4(uint64_t seed, uint32_t blk, uint32_t row, uint32_t round, uint32_t stream,
                     double z[4]) {
  uint32_t r[4];
  draw(seed, blk, row, round, stream, r);
  const double two_pi = 6.283185307179586476925286766559;
  for (int h = 0; h < 2; ++h) {
    double u0 = u01_open0(r[2 * h]), u1 = u01_open0(r[2 * h + 1]);
    double rad = std::sqrt(-2.0 * std::log(u0));
    z[2 * h] = rad * std::cos(two_pi * u1);
    z[2 * h + 1] = rad * std::sin(two_pi * u1);
  }
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

// Raw Philox4x32-10 block, for known-answer tests.
void wl_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  philox4x32_10(ctr, key, out);
}

// Logit models.
enum {
  WL_GAUSS = 0,      // z_p = p_scale*N0 ; z_q = q_coef*z_p + sigma*N1
  WL_ZIPF = 1,       // z_p = p_scale*N0 - zipf_s*ln(v+1) ; z_q = q_coef*z_p + sigma_b*N1
  WL_TWO_LEVEL = 2,  // z_q = 0 ; z_p = ln(1+d) on the lower half of ids, ln(1-d) on the upper half
};

struct wl_spec {
  int32_t B, k, V;      // requests, draft tokens, vocabulary
  int32_t bf16;         // 1: bf16 logits (uint16 storage), 0: fp32
  int32_t model;        // WL_*
  int32_t ragged;       // 1: verify_len ~ U{1..k} per request, 0: verify_len = k
  int32_t sigma_choice; // 1: sigma_b ~ U{sigmas[0..2]} per request, 0: sigma = sigmas[0]
  int32_t nthreads;
  uint64_t seed;
  uint32_t round;       // round for tokens, uniforms, verify lengths, sigma choice
  uint32_t logits_round;// round for the logits (equal to round unless logits are held fixed)
  double T;             // drafter sampling temperature (0: argmax)
  double p_scale, q_coef, zipf_s, two_level_d;
  double sigmas[3];
};

// Fills target [B, k+1, V], draft [B, k, V], tokens [B, k], verify_len [B],
// uniforms [B, k+1], sigma_out [B] (may be NULL).  Any output may be NULL to skip it,
// except that tokens need draft logits (they are drawn from them).
int wl_generate(const wl_spec* s, void* target, void* draft, int32_t* tokens, int32_t* verify_len,
                float* uniforms, float* sigma_out) {
  const int B = s->B, k = s->k, V = s->V;
  if (B < 0 || k < 1 || V < 1) return -1;
  if (tokens && !draft) return -1;
  const int64_t rows_t = (int64_t)B * (k + 1);
  const uint64_t seed = s->seed;

  // Per-request noise level and verify length.
  std::vector<double> sig(B > 0 ? B : 1, s->sigmas[0]);
  for (int b = 0; b < B; ++b) {
    if (s->sigma_choice) {
      uint32_t r[4];
      draw(seed, 0, (uint32_t)b, s->round, 5, r);
      int idx = (int)(((uint64_t)(r[0] >> 8) * 3) >> 24);
      sig[b] = s->sigmas[idx];
    }
    if (sigma_out) sigma_out[b] = (float)sig[b];
    if (verify_len) {
      if (s->ragged) {
        uint32_t r[4];
        draw(seed, 0, (uint32_t)b, s->round, 4, r);
        verify_len[b] = 1 + (int32_t)(((uint64_t)(r[0] >> 8) * (uint64_t)k) >> 24);
      } else {
        verify_len[b] = k;
      }
    }
    if (uniforms) {
      for (int j = 0; j <= k; j += 4) {
        uint32_t r[4];
        draw(seed, (uint32_t)(j / 4), (uint32_t)b, s->round, 3, r);
        for (int t = 0; t < 4 && j + t <= k; ++t) uniforms[(int64_t)b * (k + 1) + j + t] = u24(r[t]);
      }
    }
  }

  // Logits, one target row (and the matching draft row) per task.
  std::vector<double> ln1p_v;
  if (s->model == WL_ZIPF) {
    ln1p_v.resize(V);
    for (int v = 0; v < V; ++v) ln1p_v[v] = std::log((double)v + 1.0);
  }
  auto store = [&](void* base, int64_t row, int v, double val) {
    float f = (float)val;
    if (s->bf16)
      ((uint16_t*)base)[row * V + v] = f32_to_bf16_rne(f);
    else
      ((float*)base)[row * V + v] = f;
  };
  auto load = [&](const void* base, int64_t row, int v) -> double {
    return s->bf16 ? (double)bf16_to_f32(((const uint16_t*)base)[row * V + v])
                   : (double)((const float*)base)[row * V + v];
  };

  if (target || draft) {
    parallel_for(rows_t, s->nthreads, [&](int64_t rt) {
      const int b = (int)(rt / (k + 1)), i = (int)(rt % (k + 1));
      const uint32_t rowid = (uint32_t)rt;
      const bool has_draft = (i < k) && draft;
      const int64_t rd = (int64_t)b * k + i;
      for (int v0 = 0; v0 < V; v0 += 4) {
        double n0[4] = {0, 0, 0, 0}, n1[4] = {0, 0, 0, 0};
        if (s->model != WL_TWO_LEVEL) {
          normals4(seed, (uint32_t)(v0 / 4), rowid, s->logits_round, 0, n0);
          if (has_draft) normals4(seed, (uint32_t)(v0 / 4), rowid, s->logits_round, 1, n1);
        }
        for (int t = 0; t < 4 && v0 + t < V; ++t) {
          const int v = v0 + t;
          double zp, zq;
          if (s->model == WL_TWO_LEVEL) {
            zp = (v < V / 2) ? std::log(1.0 + s->two_level_d) : std::log(1.0 - s->two_level_d);
            zq = 0.0;
          } else {
            zp = s->p_scale * n0[t];
            if (s->model == WL_ZIPF) zp -= s->zipf_s * ln1p_v[v];
            zq = s->q_coef * zp + sig[b] * n1[t];
          }
          if (target) store(target, rt, v, zp);
          if (has_draft) store(draft, rd, v, zq);
        }
      }
    });
  }

  // Draft tokens: x_i ~ softmax(z_q[b,i,:] / T) of the stored (rounded) logits.
  if (tokens) {
    parallel_for((int64_t)B * k, s->nthreads, [&](int64_t rd) {
      const int b = (int)(rd / k), i = (int)(rd % k);
      const uint32_t rowid = (uint32_t)((int64_t)b * (k + 1) + i);
      int best = 0;
      double best_key = -std::numeric_limits<double>::infinity();
      bool any = false;
      for (int v0 = 0; v0 < V; v0 += 4) {
        uint32_t r[4] = {0, 0, 0, 0};
        if (s->T > 0) draw(seed, (uint32_t)(v0 / 4), rowid, s->round, 2, r);
        for (int t = 0; t < 4 && v0 + t < V; ++t) {
          const int v = v0 + t;
          double z = load(draft, rd, v);
          double key;
          if (s->T > 0) {
            double u = ((double)r[t] + 0.5) * (1.0 / 4294967296.0);  // (0,1)
            key = z / s->T - std::log(-std::log(u));
          } else {
            key = z;
          }
          if (!any || key > best_key) {
            best_key = key;
            best = v;
            any = true;
          }
        }
      }
      tokens[rd] = best;
    });
  }
  return 0;
}

}  // extern "C"
