// Adaptive length head on gfx950: forward (predicted accept rate and verify
// length) and the squared-error loss with the head's parameter gradients.
//
// The head (AdaFlash review, section 2.2; AdaFlash review (EN), Algorithm 3
// and "Online Update of the Length Head, Derived"):
//   z1[b,i] = W1 h[b,i] + b1            (per position, W1: H' x H)
//   hbar[b] = mean_i SiLU(z1[b,i])
//   a[b]    = sigmoid(w2 . hbar[b] + b2)
//   k_hat   = clamp(floor(gamma a k), 1, k)
//   loss[b] = (a[b] - A_b / L_b)^2, gradients of the batch sum with respect to
//   W1, b1, w2, b2 only (the hidden states are detached).
//
// The two dense products run on the matrix cores (v_mfma_f32_32x32x16_bf16):
//   forward  Z1 [M x H'] = h [M x H] . W1^T      (M = B k), both operands with
//            the reduction dimension contiguous, one 16-byte load per lane;
//   backward dW1 [H' x H] = dZ1^T [H' x M] . h [M x H], with dZ1 split into a
//            bf16 high part and a bf16 remainder (two products, ~16 mantissa
//            bits) and h gathered along M by 2-byte loads (each load
//            instruction reads 64 contiguous bytes per row across the wave).
// Everything else (bias, SiLU, mean, second layer, loss, small reductions)
// is element-wise or a fixed-order reduction in fp32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaflash_internal.h"

namespace adaflash {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLhThreads = 256;  // four waves, one 32 x 32 output tile each
constexpr int kTile = 64;        // output tile per workgroup (rows and columns)

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

// Matrix-core fragment layout (32 x 32 x 16, bf16 in, fp32 accumulate): lane l
// supplies A[l % 32][8 (l / 32) + 0..7] and B[8 (l / 32) + 0..7][l % 32];
// accumulator register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// C[M x N] (fp32, row stride ldc) = A[M x K] . B[N x K]^T, A and B bf16 with
// row strides lda, ldb (elements), K a multiple of 16, rows 16-byte aligned.
__global__ __launch_bounds__(kLhThreads) void lh_gemm_tn(const uint16_t* __restrict__ A, int lda,
                                                          const uint16_t* __restrict__ Bm, int ldb,
                                                          float* __restrict__ C, int ldc, int M, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Row tiles along x (up to 2^24 rows), column tiles along y.
  const int m0 = blockIdx.x * kTile + 32 * (wave >> 1);
  const int n0 = blockIdx.y * kTile + 32 * (wave & 1);
  const int ra = m0 + (lane & 31), rb = n0 + (lane & 31);
  const int ko = 8 * (lane >> 5);
  const bool va = ra < M, vb = rb < N;
  const uint16_t* pa = A + (size_t)(va ? ra : 0) * lda + ko;
  const uint16_t* pb = Bm + (size_t)(vb ? rb : 0) * ldb + ko;
  f32x16_t acc = {};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 16) {
    const u32x4_t a = va ? *(const u32x4_t*)(pa + k0) : zero;
    const u32x4_t b = vb ? *(const u32x4_t*)(pb + k0) : zero;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
  }
  const int col = n0 + (lane & 31);
  if (col < N) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + acc_row(r, lane);
      if (row < M) C[(size_t)row * ldc + col] = acc[r];
    }
  }
}

// Workgroup sum (fixed order); every thread gets the result.
__device__ float lh_block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// One workgroup per request: bias, SiLU, mean over the k positions, second
// layer, sigmoid, verify length; with accept_len given also the label, the
// loss and d loss / d s, and the pooled vector kept for the weight gradient.
__global__ __launch_bounds__(kLhThreads) void lh_pool(const float* __restrict__ Z1, int Hp, int k,
                                                       const float* __restrict__ b1, const float* __restrict__ w2,
                                                       float b2, float gamma, float* __restrict__ a_hat,
                                                       int32_t* __restrict__ k_hat, const int32_t* __restrict__ accept_len,
                                                       const int32_t* __restrict__ verify_len, float* __restrict__ loss,
                                                       float* __restrict__ hbar, float* __restrict__ ds) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const float invk = 1.f / (float)k;
  float part = 0.f;
  for (int n = threadIdx.x; n < Hp; n += kLhThreads) {
    const float bias = b1[n];
    float acc = 0.f;
    for (int i = 0; i < k; ++i) {
      const float z = Z1[((size_t)b * k + i) * Hp + n] + bias;
      acc += z * sigmoidf_(z);
    }
    const float hb = acc * invk;
    if (hbar) hbar[(size_t)b * Hp + n] = hb;
    part = fmaf(hb, w2[n], part);
  }
  const float s = lh_block_sum(part, red) + b2;
  if (threadIdx.x == 0) {
    const float a = sigmoidf_(s);
    if (a_hat) a_hat[b] = a;
    if (k_hat) {
      const float x = floorf(gamma * a * (float)k);
      k_hat[b] = x < 1.f ? 1 : (x > (float)k ? k : (int)x);
    }
    if (accept_len) {
      // Label a* = A / L; L clamped to [1, k] and A to [0, L] as the verifier does.
      int L = verify_len[b];
      L = L < 1 ? 1 : (L > k ? k : L);
      int A = accept_len[b];
      A = A < 0 ? 0 : (A > L ? L : A);
      const float astar = (float)A / (float)L;
      const float d = a - astar;
      loss[b] = d * d;
      ds[b] = 2.f * d * a * (1.f - a);
    }
  }
}

// dZ1 = ds[b] w2[n] / k * SiLU'(z1) for a 64 x 64 tile of (row m, column n),
// transposed through LDS and written as dZ1^T split into a bf16 high part and
// a bf16 remainder ([H' x Mp], Mp = M rounded up to 16, zero past M).  Each
// tile also writes its partial column sums for db1 ([ceil(M/64)][H']).
__global__ __launch_bounds__(kLhThreads) void lh_dz(const float* __restrict__ Z1, int M, int Hp, int k, int Mp,
                                                     const float* __restrict__ b1, const float* __restrict__ w2,
                                                     const float* __restrict__ ds, uint16_t* __restrict__ dzh,
                                                     uint16_t* __restrict__ dzl, float* __restrict__ db1_part) {
  __shared__ float t[kTile][kTile + 1];
  const int m0 = blockIdx.x * kTile, n0 = blockIdx.y * kTile;  // row tiles along x
  const int tc = threadIdx.x & 63, tr = threadIdx.x >> 6;
  const int n = n0 + tc;
  const float invk = 1.f / (float)k;
  float colsum = 0.f;
  for (int rr = tr; rr < kTile; rr += 4) {
    const int m = m0 + rr;
    float v = 0.f;
    if (m < M && n < Hp) {
      const float z = Z1[(size_t)m * Hp + n] + b1[n];
      const float sg = sigmoidf_(z);
      v = ds[m / k] * w2[n] * invk * (sg * (1.f + z * (1.f - sg)));
    }
    t[rr][tc] = v;
    colsum += v;
  }
  __syncthreads();
  // Partial db1: the four row groups' sums, added in a fixed order.
  __shared__ float cs[4][kTile];
  cs[tr][tc] = colsum;
  __syncthreads();
  if (tr == 0 && n < Hp) db1_part[(size_t)blockIdx.x * Hp + n] = (cs[0][tc] + cs[1][tc]) + (cs[2][tc] + cs[3][tc]);
  // Transposed write: row n of dZ1^T, 64 consecutive m.
  for (int cc = tr; cc < kTile; cc += 4) {
    const int nn = n0 + cc, m = m0 + tc;
    if (nn < Hp && m < Mp) {
      const float v = t[tc][cc];
      const __bf16 hi = (__bf16)v;
      const __bf16 lo = (__bf16)(v - (float)hi);
      dzh[(size_t)nn * Mp + m] = __builtin_bit_cast(uint16_t, hi);
      dzl[(size_t)nn * Mp + m] = __builtin_bit_cast(uint16_t, lo);
    }
  }
}

// db1 = sum of the tile partials, dw2 = sum_b ds[b] hbar[b], db2 = sum_b ds[b]
// (all in a fixed order), one workgroup.
__global__ __launch_bounds__(kLhThreads) void lh_small_grads(const float* __restrict__ db1_part, int ntiles, int Hp,
                                                              int B, const float* __restrict__ ds,
                                                              const float* __restrict__ hbar, float* __restrict__ db1,
                                                              float* __restrict__ dw2, float* __restrict__ db2) {
  __shared__ float red[4];
  for (int n = threadIdx.x; n < Hp; n += kLhThreads) {
    float a = 0.f;
    for (int t = 0; t < ntiles; ++t) a += db1_part[(size_t)t * Hp + n];
    db1[n] = a;
    float w = 0.f;
    for (int b = 0; b < B; ++b) w = fmaf(ds[b], hbar[(size_t)b * Hp + n], w);
    dw2[n] = w;
  }
  float part = 0.f;
  for (int b = threadIdx.x; b < B; b += kLhThreads) part += ds[b];
  const float tot = lh_block_sum(part, red);
  if (threadIdx.x == 0) *db2 = tot;
}

// dW1 [H' x H] = (dzh + dzl) [H' x Mp] . h [M x H]: the reduction runs over
// the M rows of h; lane l gathers h[8 (l / 32) + 0..7 + m0][col] with 2-byte
// loads.
__global__ __launch_bounds__(kLhThreads) void lh_gemm_dw(const uint16_t* __restrict__ dzh,
                                                          const uint16_t* __restrict__ dzl, int Mp,
                                                          const uint16_t* __restrict__ h, int M, int H,
                                                          float* __restrict__ dW1, int Hp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.y * kTile + 32 * (wave >> 1);  // rows of dW1 (n)
  const int c0 = blockIdx.x * kTile + 32 * (wave & 1);   // columns of dW1 (h feature)
  const int ra = r0 + (lane & 31), col = c0 + (lane & 31);
  const int ko = 8 * (lane >> 5);
  const bool va = ra < Hp, vc = col < H;
  const uint16_t* pah = dzh + (size_t)(va ? ra : 0) * Mp + ko;
  const uint16_t* pal = dzl + (size_t)(va ? ra : 0) * Mp + ko;
  const uint16_t* pb = h + (vc ? col : 0);
  f32x16_t acc = {};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int k0 = 0; k0 < Mp; k0 += 16) {
    const u32x4_t ah = va ? *(const u32x4_t*)(pah + k0) : zero;
    const u32x4_t al = va ? *(const u32x4_t*)(pal + k0) : zero;
    uint32_t g[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int m = k0 + ko + t;
      g[t] = (vc && m < M) ? (uint32_t)pb[(size_t)m * H] : 0u;
    }
    const u32x4_t bv = {g[0] | (g[1] << 16), g[2] | (g[3] << 16), g[4] | (g[5] << 16), g[6] | (g[7] << 16)};
    const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, bv);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ah), bb, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, al), bb, acc, 0, 0, 0);
  }
  if (vc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + acc_row(r, lane);
      if (row < Hp) dW1[(size_t)row * H + col] = acc[r];
    }
  }
}

}  // namespace

size_t lh_workspace_layout(int B, int k, int H, int Hp, char* base, LhWorkspace* ws) {
  const size_t M = (size_t)B * k;
  const size_t Mp = (M + 15) & ~size_t(15);
  const size_t ntiles = (M + kTile - 1) / kTile;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = (off + bytes + 255) & ~size_t(255);
    return base ? base + at : nullptr;
  };
  char* z1 = take(sizeof(float) * M * Hp);
  char* hbar = take(sizeof(float) * (size_t)B * Hp);
  char* ds = take(sizeof(float) * (size_t)B);
  char* dzh = take(sizeof(uint16_t) * Mp * Hp);
  char* dzl = take(sizeof(uint16_t) * Mp * Hp);
  char* part = take(sizeof(float) * ntiles * Hp);
  if (ws) {
    ws->z1 = (float*)z1;
    ws->hbar = (float*)hbar;
    ws->ds = (float*)ds;
    ws->dzh = (uint16_t*)dzh;
    ws->dzl = (uint16_t*)dzl;
    ws->db1_part = (float*)part;
  }
  (void)H;
  return off;
}

hipError_t lh_launch(const LhArgs& a) {
  const int M = a.B * a.k;
  const int Mp = (M + 15) & ~15;
  if (M == 0) return hipSuccess;
  const dim3 g1((M + kTile - 1) / kTile, (a.Hp + kTile - 1) / kTile);
  hipLaunchKernelGGL(lh_gemm_tn, g1, dim3(kLhThreads), 0, a.stream, a.h, a.H, a.W1, a.H, a.ws.z1, a.Hp, M, a.Hp,
                     a.H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool bwd = a.accept_len != nullptr;
  hipLaunchKernelGGL(lh_pool, dim3(a.B), dim3(kLhThreads), 0, a.stream, a.ws.z1, a.Hp, a.k, a.b1, a.w2, a.b2,
                     a.gamma, a.a_hat, a.k_hat, a.accept_len, a.verify_len, a.loss, bwd ? a.ws.hbar : nullptr,
                     a.ws.ds);
  e = hipGetLastError();
  if (e != hipSuccess || !bwd) return e;
  const int ntiles = (M + kTile - 1) / kTile;
  const dim3 g2((Mp + kTile - 1) / kTile, (a.Hp + kTile - 1) / kTile);
  hipLaunchKernelGGL(lh_dz, g2, dim3(kLhThreads), 0, a.stream, a.ws.z1, M, a.Hp, a.k, Mp, a.b1, a.w2, a.ws.ds,
                     a.ws.dzh, a.ws.dzl, a.ws.db1_part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lh_small_grads, dim3(1), dim3(kLhThreads), 0, a.stream, a.ws.db1_part, ntiles, a.Hp, a.B,
                     a.ws.ds, a.ws.hbar, a.db1, a.dw2, a.db2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g3((a.H + kTile - 1) / kTile, (a.Hp + kTile - 1) / kTile);
  hipLaunchKernelGGL(lh_gemm_dw, g3, dim3(kLhThreads), 0, a.stream, a.ws.dzh, a.ws.dzl, Mp, a.h, M, a.H, a.dW1,
                     a.Hp);
  return hipGetLastError();
}

}  // namespace adaflash
