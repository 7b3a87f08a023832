// Sanitizer driver for the CPU oracle (oracle/oracle.cpp) and the seeded
// input generator (workloads/gen.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer: every logit model, both dtypes, ragged and fixed
// verify lengths, greedy and sampled verification, every draw flag, supervision
// with and without selected rows and gradients, the degenerate sizes, and the
// rejected arguments.  Exits non-zero on a failed check.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

extern "C" {
// Same layout as the generator's spec (workloads/gen.cpp).
struct wl_spec {
  int32_t B, k, V;
  int32_t bf16;
  int32_t model;
  int32_t ragged;
  int32_t sigma_choice;
  int32_t nthreads;
  uint64_t seed;
  uint32_t round;
  uint32_t logits_round;
  double T;
  double p_scale, q_coef, zipf_s, two_level_d;
  double sigmas[3];
};
void wl_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
int wl_generate(const wl_spec* s, void* target, void* draft, int32_t* tokens, int32_t* verify_len, float* uniforms,
                float* sigma_out);
int oracle_verify(int dtype, const void* target, const void* draft, const int32_t* tokens,
                  const int32_t* verify_len, const float* uniforms, int B, int k, int V, double T,
                  int32_t* accept_len, int32_t* out_tokens, double* margins, double* sample_info,
                  double* accept_pq, int flags, int nthreads);
int64_t oracle_opd(int dtype, const void* target, const void* draft, const int32_t* verify_len, int B, int k,
                   int V, double c, double lambda, const int64_t* rows, int64_t nrows, double* loss_ce,
                   double* loss_rkl, double* grad, int nthreads);
}

static int failures = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

static void one_case(int B, int k, int V, int bf16, int model, int ragged, int nthreads) {
  wl_spec s{};
  s.B = B;
  s.k = k;
  s.V = V;
  s.bf16 = bf16;
  s.model = model;
  s.ragged = ragged;
  s.sigma_choice = 1;
  s.nthreads = nthreads;
  s.seed = 1234 + (uint64_t)V;
  s.round = 3;
  s.logits_round = 3;
  s.T = 1.0;
  s.p_scale = 2.0;
  s.q_coef = 0.7;
  s.zipf_s = 1.1;
  s.two_level_d = 0.3;
  s.sigmas[0] = 0.3;
  s.sigmas[1] = 1.0;
  s.sigmas[2] = 2.0;
  const size_t es = bf16 ? 2 : 4;
  std::vector<char> target((size_t)B * (k + 1) * V * es + 1), draft((size_t)B * k * V * es + 1);
  std::vector<int32_t> tokens((size_t)B * k + 1), vlen(B + 1), acc(B + 1), out((size_t)B * (k + 1) + 1);
  std::vector<float> uni((size_t)B * (k + 1) + 1), sig(B + 1);
  CHECK(wl_generate(&s, target.data(), draft.data(), tokens.data(), vlen.data(), uni.data(), sig.data()) == 0);
  CHECK(wl_generate(&s, target.data(), nullptr, nullptr, nullptr, nullptr, nullptr) == 0);
  std::vector<double> margins((size_t)B * (k + 1) + 1), info((size_t)B * 4 + 1), pq((size_t)B * k * 2 + 1);
  for (double T : {0.0, 0.7, 1.0})
    for (int flags : {0, 1, 2})
      for (const int32_t* vl : {(const int32_t*)nullptr, (const int32_t*)vlen.data()}) {
        const int rc = oracle_verify(bf16, target.data(), draft.data(), tokens.data(), vl, uni.data(), B, k, V, T,
                                     acc.data(), out.data(), margins.data(), info.data(),
                                     flags == 1 ? nullptr : pq.data(), flags, nthreads);
        CHECK(rc == 0);
        for (int b = 0; b < B; ++b) CHECK(acc[b] >= 0 && acc[b] <= k);
      }
  // Supervision: all rows, then a selection; with and without gradients.
  std::vector<int32_t> vbad(vlen);
  if (B > 0) vbad[0] = k + 5;  // clamped to k
  const int64_t none = 0;
  int64_t N = oracle_opd(bf16, target.data(), draft.data(), vbad.data(), B, k, V, 0.01, 1.0, &none, 0, nullptr,
                         nullptr, nullptr, nthreads);  // row count only
  CHECK(N >= 0);
  if (N > 0)
    CHECK(oracle_opd(bf16, target.data(), draft.data(), vbad.data(), B, k, V, 0.01, 1.0, nullptr, 0, nullptr,
                     nullptr, nullptr, nthreads) < 0);  // every row, but no loss outputs
  std::vector<double> ce(N + 1), rk(N + 1), grad((size_t)(N + 1) * V);
  CHECK(oracle_opd(bf16, target.data(), draft.data(), vbad.data(), B, k, V, 10.0, 0.5, nullptr, N, ce.data(),
                   rk.data(), grad.data(), nthreads) == N);
  std::vector<int64_t> rows;
  for (int64_t n = N - 1; n >= 0; n -= 3) rows.push_back(n);
  std::vector<double> ce2(rows.size() + 1), rk2(rows.size() + 1), g2((rows.size() + 1) * V);
  CHECK(oracle_opd(bf16, target.data(), draft.data(), vbad.data(), B, k, V, 0.01, 1.0, rows.data(),
                   (int64_t)rows.size(), ce2.data(), rk2.data(), g2.data(), nthreads) == N);
  CHECK(oracle_opd(bf16, target.data(), draft.data(), nullptr, B, k, V, 1.0, 0.0, rows.data(),
                   (int64_t)rows.size(), ce2.data(), rk2.data(), nullptr, nthreads) >= 0);
  for (size_t q = 0; q < rows.size(); ++q) CHECK(std::isfinite(ce2[q]));
}

int main() {
  uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, o[4];
  wl_philox4x32_10(ctr, key, o);
  const int models[] = {0, 1, 2};
  for (int model : models)
    for (int bf16 : {0, 1})
      for (int ragged : {0, 1}) one_case(3, 4, 37, bf16, model, ragged, 1 + ragged * 2);
  one_case(2, 16, 4096 + 8, 1, 1, 1, 4);
  one_case(1, 1, 1, 0, 0, 0, 1);   // one entry per row
  one_case(0, 3, 10, 1, 1, 1, 2);  // empty batch
  // Rejected arguments.
  wl_spec s{};
  s.B = -1;
  s.k = 1;
  s.V = 1;
  CHECK(wl_generate(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != 0);
  s.B = 1;
  s.k = 2;
  s.V = 4;
  int32_t tok[2];
  CHECK(wl_generate(&s, nullptr, nullptr, tok, nullptr, nullptr, nullptr) != 0);  // tokens need draft logits
  float z[12] = {0};
  int32_t t2[2] = {0, 1}, acc[1], out[3];
  float u[3] = {0.5f, 0.5f, 0.5f};
  double m[3], inf4[4];
  CHECK(oracle_verify(0, z, z, t2, nullptr, u, 1, 0, 4, 1.0, acc, out, m, inf4, nullptr, 0, 1) != 0);
  CHECK(oracle_verify(0, z, z, t2, nullptr, u, 1, 2, 4, -1.0, acc, out, m, inf4, nullptr, 0, 1) != 0);
  CHECK(oracle_verify(0, z, z, t2, nullptr, u, 1, 2, 4, NAN, acc, out, m, inf4, nullptr, 0, 1) != 0);
  CHECK(oracle_opd(0, z, z, nullptr, 1, 2, 4, 0.0, 1.0, nullptr, 0, nullptr, nullptr, nullptr, 1) < 0);
  CHECK(oracle_opd(0, z, z, nullptr, 1, 2, 4, 1.0, -1.0, nullptr, 0, nullptr, nullptr, nullptr, 1) < 0);
  std::printf("oracle driver: %d failed checks\n", failures);
  return failures == 0 ? 0 : 1;
}
