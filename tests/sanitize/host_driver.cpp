// Sanitizer driver for the library's host code: argument checks of every
// entry point, the workspace layouts and the admission queue, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against launch_stub.cpp.
// Host arrays stand in for device buffers (the host code never dereferences
// them).  Exits non-zero on a failed check; the sanitizers abort on any error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "../../include/adaflash.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static void error_text_ok() {
  const char* e = adaflash_last_error();
  CHECK(e != nullptr);
  CHECK(std::strlen(e) < 512);
}

// A rejected call: a negative status other than the stub's launch error.
static void rejected(int rc) {
  CHECK(rc < 0 && rc != ADAFLASH_E_HIP);
  error_text_ok();
}

struct Buffers {
  std::vector<uint16_t> target, draft;
  std::vector<int32_t> tokens, vlen, acc, out, ro, status;
  std::vector<float> uni, margins, ce, rk, grad_f;
  std::vector<char> ws;
  Buffers(int B, int k, int V)
      : target((size_t)B * (k + 1) * V + 1), draft((size_t)B * k * V + 1), tokens((size_t)B * k + 1),
        vlen(B + 1, k), acc(B + 1), out((size_t)B * (k + 1) + 1), ro(B + 2), status(1),
        uni((size_t)B * (k + 1) + 1), margins((size_t)B * (k + 1) + 1), ce((size_t)B * k + 1),
        rk((size_t)B * k + 1), grad_f((size_t)B * k * V + 1),
        ws(adaflash_workspace_bytes(B, k, V) + 1) {}
};

static void verify_calls() {
  const int B = 5, k = 4, V = 96;
  Buffers b(B, k, V);
  const size_t need = adaflash_workspace_bytes(B, k, V);
  CHECK(need > 0);
  auto call = [&](int dtype, const void* t, const void* d, const int32_t* tok, const float* u, int B_, int k_,
                  int V_, float T, float c, float lam, int32_t* ro, void* ws, size_t wsb) {
    return adaflash_verify((adaflash_dtype)dtype, t, d, tok, b.vlen.data(), u, B_, k_, V_, T, b.acc.data(),
                           b.out.data(), b.margins.data(), c, lam, ro, b.ce.data(), b.rk.data(), b.grad_f.data(),
                           b.status.data(), ws, wsb, nullptr);
  };
  const void* t = b.target.data();
  const void* d = b.draft.data();
  // Valid arguments reach the (stubbed) launch.
  for (float T : {0.f, 0.7f, 1.f})
    for (int dt : {0, 1}) {
      CHECK(call(dt, t, d, b.tokens.data(), b.uni.data(), B, k, V, T, 10.f, 1.f, b.ro.data(), b.ws.data(), need) ==
            ADAFLASH_E_HIP);
      error_text_ok();
    }
  CHECK(call(1, t, d, b.tokens.data(), b.uni.data(), 0, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need) <= 0);
  // Rejected arguments.
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();
  rejected(call(7, t, d, b.tokens.data(), b.uni.data(), B, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, nullptr, d, b.tokens.data(), b.uni.data(), B, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, nullptr, b.tokens.data(), b.uni.data(), B, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, nullptr, b.uni.data(), B, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), nullptr, B, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), -1, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, 0, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, 65, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, 0, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, (1 << 20) + 1, 1.f, 10.f, 1.f, b.ro.data(),
                b.ws.data(), need));
  for (float T : {-1.f, nan, inf})
    rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, V, T, 10.f, 1.f, b.ro.data(), b.ws.data(), need));
  for (float c : {0.f, -1.f, nan})
    rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, V, 1.f, c, 1.f, b.ro.data(), b.ws.data(), need));
  for (float lam : {-1.f, nan, inf})
    rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, V, 1.f, 10.f, lam, b.ro.data(), b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, V, 1.f, 10.f, 1.f, nullptr, b.ws.data(), need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, V, 1.f, 10.f, 1.f, b.ro.data(), nullptr, need));
  rejected(call(1, t, d, b.tokens.data(), b.uni.data(), B, k, V, 1.f, 10.f, 1.f, b.ro.data(), b.ws.data(), need - 1));
  // Packed form: same checks on the same arguments.
  CHECK(adaflash_verify_packed(ADAFLASH_BF16, t, d, b.tokens.data(), b.vlen.data(), b.uni.data(), B, k, V, 1.f,
                               b.acc.data(), b.out.data(), b.margins.data(), 10.f, 1.f, b.ro.data(), b.ce.data(),
                               b.rk.data(), b.grad_f.data(), b.status.data(), b.ws.data(), need,
                               nullptr) == ADAFLASH_E_HIP);
  rejected(adaflash_verify_packed(ADAFLASH_BF16, t, d, b.tokens.data(), b.vlen.data(), b.uni.data(), B, k, V, 1.f,
                                  b.acc.data(), b.out.data(), b.margins.data(), 10.f, 1.f, nullptr, b.ce.data(),
                                  b.rk.data(), b.grad_f.data(), b.status.data(), b.ws.data(), need, nullptr));
}

static void opd_calls() {
  const int B = 3, k = 6, V = 4097;
  Buffers b(B, k, V);
  const size_t need = adaflash_workspace_bytes(B, k, V);
  const void* t = b.target.data();
  const void* d = b.draft.data();
  for (int dt : {0, 1})
    for (const int32_t* vl : {(const int32_t*)nullptr, (const int32_t*)b.vlen.data()}) {
      CHECK(adaflash_opd_loss_fwd_bwd((adaflash_dtype)dt, t, d, vl, B, k, V, 0.01f, 1.f, b.ro.data(), b.ce.data(),
                                      b.rk.data(), b.grad_f.data(), b.status.data(), b.ws.data(), need,
                                      nullptr) == ADAFLASH_E_HIP);
      CHECK(adaflash_opd_loss_fwd_bwd_packed((adaflash_dtype)dt, t, d, vl, B, k, V, 10.f, 0.f, b.ro.data(), nullptr,
                                             nullptr, b.grad_f.data(), nullptr, b.ws.data(), need,
                                             nullptr) == ADAFLASH_E_HIP);
    }
  rejected(adaflash_opd_loss_fwd_bwd(ADAFLASH_BF16, t, nullptr, nullptr, B, k, V, 10.f, 1.f, b.ro.data(),
                                     b.ce.data(), b.rk.data(), b.grad_f.data(), nullptr, b.ws.data(), need, nullptr));
  rejected(adaflash_opd_loss_fwd_bwd(ADAFLASH_BF16, t, d, nullptr, B, k, V, 0.f, 1.f, b.ro.data(), b.ce.data(),
                                     b.rk.data(), b.grad_f.data(), nullptr, b.ws.data(), need, nullptr));
  rejected(adaflash_opd_loss_fwd_bwd(ADAFLASH_BF16, t, d, nullptr, B, k, V, 10.f, 1.f, b.ro.data(), b.ce.data(),
                                     b.rk.data(), b.grad_f.data(), nullptr, b.ws.data(), 0, nullptr));
  // Loss variants, each parameter range.
  struct Case {
    int variant;
    float p1, p2;
    bool ok;
  };
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const Case cases[] = {{ADAFLASH_LOSS_RKL, 0.f, 0.f, true},       {ADAFLASH_LOSS_RKL_CLIP, 0.05f, 0.f, true},
                        {ADAFLASH_LOSS_RKL_CLIP, 0.f, 0.f, false},  {ADAFLASH_LOSS_MIXTURE, 0.8f, 0.01f, true},
                        {ADAFLASH_LOSS_MIXTURE, 1.5f, 0.01f, false}, {ADAFLASH_LOSS_MIXTURE, 0.8f, -1.f, false},
                        {ADAFLASH_LOSS_FKL, 0.f, 0.f, true},       {ADAFLASH_LOSS_WCE, 7.f, 0.f, true},
                        {ADAFLASH_LOSS_WCE, nan, 0.f, false},       {0, 0.f, 0.f, false},
                        {6, 0.f, 0.f, false}};
  for (const Case& c : cases) {
    const int rc = adaflash_loss_variant_fwd_bwd(ADAFLASH_BF16, t, d, b.vlen.data(), B, k, V, c.variant, c.p1, c.p2,
                                                 b.ro.data(), b.ce.data(), b.grad_f.data(), b.status.data(),
                                                 b.ws.data(), need, nullptr);
    if (c.ok) CHECK(rc == ADAFLASH_E_HIP);
    else rejected(rc);
  }
}

static void workspace_sizes() {
  const int Bs[] = {-1, 0, 1, 7, 128, 4096, 1 << 23};
  const int ks[] = {0, 1, 16, 64, 65};
  const int Vs[] = {0, 1, 8, 151936, 1 << 20, (1 << 20) + 1};
  for (int B : Bs)
    for (int k : ks)
      for (int V : Vs) {
        const size_t n = adaflash_workspace_bytes(B, k, V);
        const bool bad = B < 0 || k < 1 || k > 64 || V < 1 || V > (1 << 20);
        if (bad) CHECK(n == 0);
        if (!bad && B > 0 && (long long)B * (k + 1) < (1LL << 24)) CHECK(n > 0);
      }
  const int Hs[] = {-1, 0, 8, 4096};
  for (int H : Hs)
    for (int Hp : Hs) (void)adaflash_length_head_workspace_bytes(16, 8, H, Hp);
}

static void length_head_calls() {
  const int B = 4, k = 8, H = 128, Hp = 64;
  const size_t need = adaflash_length_head_workspace_bytes(B, k, H, Hp);
  CHECK(need > 0);
  std::vector<uint16_t> h((size_t)B * k * H), W1((size_t)Hp * H);
  std::vector<float> b1(Hp), w2(Hp), a(B), loss(B), dW1((size_t)Hp * H), db1(Hp), dw2(Hp), db2(1),
      z1((size_t)B * k * Hp);
  std::vector<int32_t> kh(B), acc(B, 2), vl(B, 4);
  std::vector<char> ws(need + 1);
  CHECK(adaflash_length_head_forward(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp, 0.9f, a.data(),
                                     kh.data(), ws.data(), need, nullptr) == ADAFLASH_E_HIP);
  CHECK(adaflash_length_head_backward(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp, acc.data(),
                                      vl.data(), loss.data(), dW1.data(), db1.data(), dw2.data(), db2.data(),
                                      ws.data(), need, nullptr) == ADAFLASH_E_HIP);
  CHECK(adaflash_length_head_forward_cached(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp, 0.9f,
                                            a.data(), kh.data(), z1.data(), ws.data(), need,
                                            nullptr) == ADAFLASH_E_HIP);
  CHECK(adaflash_length_head_backward_cached(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp,
                                             acc.data(), vl.data(), loss.data(), dW1.data(), db1.data(), dw2.data(),
                                             db2.data(), z1.data(), ws.data(), need, nullptr) == ADAFLASH_E_HIP);
  const float nan = std::numeric_limits<float>::quiet_NaN();
  rejected(adaflash_length_head_forward(nullptr, W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp, 0.9f, a.data(),
                                        kh.data(), ws.data(), need, nullptr));
  rejected(adaflash_length_head_forward(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp, nan, a.data(),
                                        kh.data(), ws.data(), need, nullptr));
  rejected(adaflash_length_head_forward(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, -1, Hp, 0.9f,
                                        a.data(), kh.data(), ws.data(), need, nullptr));
  rejected(adaflash_length_head_forward(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp, 0.9f, a.data(),
                                        kh.data(), ws.data(), need - 1, nullptr));
  rejected(adaflash_length_head_backward(h.data(), W1.data(), b1.data(), w2.data(), 0.f, B, k, H, Hp, nullptr,
                                         vl.data(), loss.data(), dW1.data(), db1.data(), dw2.data(), db2.data(),
                                         ws.data(), need, nullptr));
}

static void timing_calls() {
  CHECK(adaflash_timing_enable(-1) < 0);
  error_text_ok();
  CHECK(adaflash_timing_enable((1 << 20) + 1) < 0);
  CHECK(adaflash_timing_enable(4) == 0);
  CHECK(adaflash_timing_every(0) < 0);
  CHECK(adaflash_timing_every(3) == 0);
  float ms[4];
  CHECK(adaflash_timing_read(ms, 4) >= 0);
  CHECK(adaflash_timing_enable(0) == 0);
}

// The admission queue: invalid arguments, then a long pseudo-random sequence
// of operations (a 64-bit LCG), including repeated and unknown ids.
static void admission_calls() {
  CHECK(adaflash_admission_create(0.0, 1.0, 100) == nullptr);
  CHECK(adaflash_admission_create(1.5, 1.0, 100) == nullptr);
  CHECK(adaflash_admission_create(0.5, -1.0, 100) == nullptr);
  CHECK(adaflash_admission_create(0.5, std::numeric_limits<double>::infinity(), 100) == nullptr);
  CHECK(adaflash_admission_create(0.5, 1.0, 0) == nullptr);
  CHECK(std::isnan(adaflash_admission_estimate(nullptr)));
  adaflash_admission_destroy(nullptr);
  CHECK(adaflash_admission_enqueue(nullptr, nullptr, 0) < 0);
  void* h = adaflash_admission_create(0.3, 4.0, 512);
  CHECK(h != nullptr);
  CHECK(adaflash_admission_enqueue(h, nullptr, 3) < 0);
  CHECK(adaflash_admission_enqueue(h, nullptr, -1) < 0);
  uint64_t s = 0x9E3779B97F4A7C15ull;
  auto next = [&]() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
  };
  std::vector<int64_t> ids, out(4096), inflight;
  std::vector<int32_t> khat;
  int64_t next_id = 1;
  for (int it = 0; it < 3000; ++it) {
    const uint32_t op = next() % 5;
    if (op == 0) {
      const int n = (int)(next() % 9);
      ids.assign(n, 0);
      for (int q = 0; q < n; ++q) ids[q] = (next() % 7 == 0 && next_id > 1) ? (int64_t)(next() % next_id) : next_id++;
      (void)adaflash_admission_enqueue(h, ids.data(), n);
    } else if (op == 1) {
      const int cap = (int)(next() % 40);
      const int n = adaflash_admission_propose(h, out.data(), cap);
      CHECK(n <= cap);
      if (n > 0) {
        khat.assign(n, 0);
        for (int q = 0; q < n; ++q) khat[q] = (int32_t)(next() % 20) - 2;
        std::vector<int64_t> admitted(n);
        const int m = adaflash_admission_commit(h, khat.data(), n, admitted.data());
        CHECK(m <= n);
        for (int q = 0; q < m; ++q) inflight.push_back(admitted[q]);
      }
    } else if (op == 2 && !inflight.empty()) {
      const int n = (int)(next() % (inflight.size() + 1));
      (void)adaflash_admission_finish(h, inflight.data(), n);
      inflight.erase(inflight.begin(), inflight.begin() + n);
    } else if (op == 3) {
      const int64_t bogus[2] = {-5, next_id + 1000};
      (void)adaflash_admission_finish(h, bogus, 2);
      (void)adaflash_admission_commit(h, nullptr, 0, nullptr);
    } else {
      CHECK(adaflash_admission_pending(h) >= 0);
      CHECK(!(adaflash_admission_estimate(h) < 0.0));
    }
  }
  adaflash_admission_destroy(h);
}

int main() {
  CHECK(adaflash_version() > 0);
  workspace_sizes();
  verify_calls();
  opd_calls();
  length_head_calls();
  timing_calls();
  admission_calls();
  std::printf("host driver: %d failed checks\n", failures);
  return failures == 0 ? 0 : 1;
}
