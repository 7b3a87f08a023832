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
constexpr int kTile = kLhTile;   // output tile per workgroup (rows and columns)

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

// Matrix-core fragment layout (32 x 32 x 16, bf16 in, fp32 accumulate): lane l
// supplies A[l % 32][8 (l / 32) + 0..7] and B[8 (l / 32) + 0..7][l % 32];
// accumulator register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Split-K product: slice z = blockIdx.z of the reduction, C_z[M x N] (fp32,
// row stride N, slice stride M N) = A[M x K_z] . B[N x K_z]^T with A (and,
// with TWO_A, A + A2) and B bf16, rows of stride lda / ldb elements, K a
// multiple of 16, rows 16-byte aligned.  The workgroup stages 64-wide steps
// of the reduction through LDS (each row's 128 bytes read by eight adjacent
// threads), then every wave multiplies its 32 x 32 tile from LDS.
constexpr int kKs = 64;           // reduction step staged per round
constexpr int kLdsRow = kKs + 8;  // bf16 per LDS row (16 bytes of padding)

template <bool TWO_A>
__global__ __launch_bounds__(kLhThreads) void lh_gemm_tn(const uint16_t* __restrict__ A, const uint16_t* __restrict__ A2,
                                                          int lda, const uint16_t* __restrict__ Bm, int ldb,
                                                          float* __restrict__ C, int M, int N, int K, int kslice) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[TWO_A ? 2 : 1][kTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t sb[kTile * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Row tiles along x (up to 2^24 rows), column tiles along y, slices along z.
  const int mt0 = blockIdx.x * kTile, nt0 = blockIdx.y * kTile;
  const int kb = blockIdx.z * kslice;
  const int ke = min(K, kb + kslice);
  // Staging: thread t moves 16 bytes of rows t / 8 and t / 8 + 32, chunk t % 8.
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x16_t acc = {};
  const int wr = 32 * (wave >> 1), wc = 32 * (wave & 1);
  const int ko = 8 * (lane >> 5);
  // The next round's operands are loaded into registers while the matrix
  // cores work on the current one (the loads' latency is hidden).
  u32x4_t ga[2], ga2[2], gb[2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 32 * h;
      const int kk = k0 + lc;
      const bool okk = kk < ke;
      const int ra = mt0 + r, rb = nt0 + r;
      ga[h] = (ra < M && okk) ? *(const u32x4_t*)(A + (size_t)ra * lda + kk) : zero;
      if constexpr (TWO_A) ga2[h] = (ra < M && okk) ? *(const u32x4_t*)(A2 + (size_t)ra * lda + kk) : zero;
      gb[h] = (rb < N && okk) ? *(const u32x4_t*)(Bm + (size_t)rb * ldb + kk) : zero;
    }
  };
  if (kb < ke) fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += kKs) {
    __syncthreads();  // the previous round's fragments are consumed
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 32 * h;
      *(u32x4_t*)&sa[0][r * kLdsRow + lc] = ga[h];
      if constexpr (TWO_A) *(u32x4_t*)&sa[1][r * kLdsRow + lc] = ga2[h];
      *(u32x4_t*)&sb[r * kLdsRow + lc] = gb[h];
    }
    __syncthreads();
    if (k0 + kKs < ke) fetch(k0 + kKs);
#pragma unroll
    for (int t = 0; t < kKs / 16; ++t) {
      const int kc = 16 * t + ko;
      const u32x4_t a = *(const u32x4_t*)&sa[0][(wr + (lane & 31)) * kLdsRow + kc];
      const u32x4_t b = *(const u32x4_t*)&sb[(wc + (lane & 31)) * kLdsRow + kc];
      const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, b);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), bb, acc, 0, 0, 0);
      if constexpr (TWO_A) {
        const u32x4_t a2 = *(const u32x4_t*)&sa[1][(wr + (lane & 31)) * kLdsRow + kc];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a2), bb, acc, 0, 0, 0);
      }
    }
  }
  float* Cz = C + (size_t)blockIdx.z * M * N;
  const int col = nt0 + wc + (lane & 31);
  if (col < N) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mt0 + wr + acc_row(r, lane);
      if (row < M) Cz[(size_t)row * N + col] = acc[r];
    }
  }
}

// out[i] = sum over the S slices of part[s][i], in slice order.  VEC: four
// consecutive entries per thread with 16-byte loads and stores (n a multiple
// of 4, out 16-byte aligned).
template <bool VEC>
__global__ __launch_bounds__(kLhThreads) void lh_sum_slices(const float* __restrict__ part, int S, size_t n,
                                                             float* __restrict__ out) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  if constexpr (VEC) {
    const size_t n4 = n / 4;
    for (size_t i = (size_t)blockIdx.x * kLhThreads + threadIdx.x; i < n4; i += (size_t)gridDim.x * kLhThreads) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
      for (int z = 0; z < S; ++z) a += *(const f32x4_t*)(part + (size_t)z * n + 4 * i);
      *(f32x4_t*)(out + 4 * i) = a;
    }
  } else {
    for (size_t i = (size_t)blockIdx.x * kLhThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kLhThreads) {
      float a = 0.f;
      for (int z = 0; z < S; ++z) a += part[(size_t)z * n + i];
      out[i] = a;
    }
  }
}

hipError_t sum_slices(const float* part, int S, size_t n, float* out, hipStream_t st) {
  const bool vec = n % 4 == 0 && ((uintptr_t)out & 15) == 0;
  const size_t units = vec ? n / 4 : n;
  const int blocks = (int)((units + kLhThreads - 1) / kLhThreads < 2048 ? (units + kLhThreads - 1) / kLhThreads : 2048);
  if (blocks == 0) return hipSuccess;
  if (vec) hipLaunchKernelGGL((lh_sum_slices<true>), dim3(blocks), dim3(kLhThreads), 0, st, part, S, n, out);
  else hipLaunchKernelGGL((lh_sum_slices<false>), dim3(blocks), dim3(kLhThreads), 0, st, part, S, n, out);
  return hipGetLastError();
}

// hT [H x Mp] = h^T (bf16), zero for m >= M, through a 64 x 64 LDS tile.
// Rows of h are read and rows of hT written 16 bytes (eight entries) per
// thread; H is a multiple of 8 and Mp of 16, h 16-byte aligned.  The LDS
// rows are 66 entries long (33 words), so that the column reads of eight
// rows eight apart fall in different banks.
__global__ __launch_bounds__(kLhThreads) void lh_transpose(const uint16_t* __restrict__ h, int M, int H, int Mp,
                                                            uint16_t* __restrict__ hT) {
  __shared__ __attribute__((aligned(16))) uint16_t t[kTile][kTile + 2];
  const int m0 = blockIdx.x * kTile, c0 = blockIdx.y * kTile;
  const int r8 = threadIdx.x >> 3, e8 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = r8 + 32 * hh, m = m0 + r, c = c0 + e8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (m < M && c < H) v = *(const u32x4_t*)(h + (size_t)m * H + c);
#pragma unroll
    for (int w = 0; w < 4; ++w) *(uint32_t*)&t[r][e8 + 2 * w] = v[w];
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int cc = r8 + 32 * hh, c = c0 + cc, m = m0 + e8;
    if (c < H && m < Mp) {
      u32x4_t v;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        v[w] = (uint32_t)t[e8 + 2 * w][cc] | ((uint32_t)t[e8 + 2 * w + 1][cc] << 16);
      *(u32x4_t*)(hT + (size_t)c * Mp + m) = v;
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
// loss and d loss / d s, the pooled vector kept for the weight gradient, and
// this request's rows of dZ1 = ds w2 / k SiLU'(z1), written transposed
// (dZ1^T, [H' x Mp]) as a bf16 high part and remainder, with its column sums
// for db1 ([B][H']).  The workgroup of the last request also zeroes the
// padding columns m in [M, Mp).
__global__ __launch_bounds__(kLhThreads) void lh_pool(const float* __restrict__ Z1, int Hp, int k,
                                                       const float* __restrict__ b1, const float* __restrict__ w2,
                                                       float b2, float gamma, float* __restrict__ a_hat,
                                                       int32_t* __restrict__ k_hat, const int32_t* __restrict__ accept_len,
                                                       const int32_t* __restrict__ verify_len, float* __restrict__ loss,
                                                       float* __restrict__ hbar, float* __restrict__ ds, int M, int Mp,
                                                       uint16_t* __restrict__ dzh, uint16_t* __restrict__ dzl,
                                                       float* __restrict__ db1_part) {
  __shared__ float red[4];
  __shared__ float sh_ds;
  const int b = blockIdx.x;
  const float invk = 1.f / (float)k;
  float part = 0.f;
  for (int n = threadIdx.x; n < Hp; n += kLhThreads) {
    const float bias = b1[n];
    float acc = 0.f;
#pragma unroll 8
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
      sh_ds = ds[b];
    }
  }
  if (!accept_len) return;
  __syncthreads();
  const float dsb = sh_ds;
  const size_t m0 = (size_t)b * k;
  // 16-byte stores of a row segment when it is aligned (k a multiple of 8).
  const bool vec = (k & 7) == 0;
  for (int n = threadIdx.x; n < Hp; n += kLhThreads) {
    const float bias = b1[n];
    const float wv = dsb * w2[n] * invk;
    float colsum = 0.f;
    uint16_t* rh = dzh + (size_t)n * Mp + m0;
    uint16_t* rl = dzl + (size_t)n * Mp + m0;
    for (int i0 = 0; i0 < k; i0 += 8) {
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u;
        float v = 0.f;
        if (i < k) {
          const float z = Z1[(m0 + i) * Hp + n] + bias;
          const float sg = sigmoidf_(z);
          v = wv * (sg * (1.f + z * (1.f - sg)));
        }
        colsum += v;
        const __bf16 hi = (__bf16)v;
        const __bf16 lo = (__bf16)(v - (float)hi);
        const uint32_t hb = __builtin_bit_cast(uint16_t, hi), lb = __builtin_bit_cast(uint16_t, lo);
        if (u & 1) {
          ph[u >> 1] |= hb << 16;
          pl[u >> 1] |= lb << 16;
        } else {
          ph[u >> 1] = hb;
          pl[u >> 1] = lb;
        }
        if (!vec && i < k) {
          rh[i] = (uint16_t)hb;
          rl[i] = (uint16_t)lb;
        }
      }
      if (vec) {
        const u32x4_t vh = {ph[0], ph[1], ph[2], ph[3]}, vl = {pl[0], pl[1], pl[2], pl[3]};
        *(u32x4_t*)(rh + i0) = vh;
        *(u32x4_t*)(rl + i0) = vl;
      }
    }
    db1_part[(size_t)b * Hp + n] = colsum;
    if (b == (int)gridDim.x - 1)
      for (int m = M; m < Mp; ++m) {
        dzh[(size_t)n * Mp + m] = 0;
        dzl[(size_t)n * Mp + m] = 0;
      }
  }
}

// db1 = sum of the per-request partials, dw2 = sum_b ds[b] hbar[b], db2 =
// sum_b ds[b], all in a fixed order.  Workgroup x takes 64 columns; wave w
// sums the partials and requests congruent to w mod 4, and the four partials
// are added in wave order.  Workgroup 0 also forms db2.
__global__ __launch_bounds__(kLhThreads) void lh_small_grads(const float* __restrict__ db1_part, int ntiles, int Hp,
                                                              int B, const float* __restrict__ ds,
                                                              const float* __restrict__ hbar, float* __restrict__ db1,
                                                              float* __restrict__ dw2, float* __restrict__ db2) {
  __shared__ float red[4];
  __shared__ float pa[4][64], pw[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 64 + lane;
  float a = 0.f, w = 0.f;
  if (n < Hp) {
#pragma unroll 4
    for (int t = wave; t < ntiles; t += 4) a += db1_part[(size_t)t * Hp + n];
#pragma unroll 4
    for (int b = wave; b < B; b += 4) w = fmaf(ds[b], hbar[(size_t)b * Hp + n], w);
  }
  pa[wave][lane] = a;
  pw[wave][lane] = w;
  __syncthreads();
  if (wave == 0 && n < Hp) {
    db1[n] = (pa[0][lane] + pa[1][lane]) + (pa[2][lane] + pa[3][lane]);
    dw2[n] = (pw[0][lane] + pw[1][lane]) + (pw[2][lane] + pw[3][lane]);
  }
  if (blockIdx.x == 0) {
    float part = 0.f;
    for (int b = threadIdx.x; b < B; b += kLhThreads) part += ds[b];
    const float tot = lh_block_sum(part, red);
    if (threadIdx.x == 0) *db2 = tot;
  }
}

}  // namespace

hipError_t lh_launch(const LhArgs& a) {
  const int M = a.B * a.k;
  const int Mp = (M + 15) & ~15;
  if (M == 0) return hipSuccess;
  const int mt = (M + kTile - 1) / kTile, nt = (a.Hp + kTile - 1) / kTile;
  const LhSplit sf = lh_split_k(a.H, (long long)mt * nt);
  const bool bwd = a.accept_len != nullptr;
  hipError_t e = hipSuccess;
  // The projection Z1 = h W1^T: from the caller's copy of the forward's, or
  // computed (split-K slices summed in slice order, so that the pooling
  // kernel reads one value per entry).
  const float* z1 = a.z1_in;
  if (!z1) {
    float* zdst = a.z1_out ? a.z1_out : a.ws.zsum;
    hipLaunchKernelGGL((lh_gemm_tn<false>), dim3(mt, nt, sf.S), dim3(kLhThreads), 0, a.stream, a.h,
                       (const uint16_t*)nullptr, a.H, a.W1, a.H, a.ws.z1, M, a.Hp, a.H, sf.kslice);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = sum_slices(a.ws.z1, sf.S, (size_t)M * a.Hp, zdst, a.stream);
    if (e != hipSuccess) return e;
    z1 = zdst;
  }
  hipLaunchKernelGGL(lh_pool, dim3(a.B), dim3(kLhThreads), 0, a.stream, z1, a.Hp, a.k,
                     a.b1, a.w2, a.b2, a.gamma, a.a_hat, a.k_hat, a.accept_len, a.verify_len, a.loss,
                     bwd ? a.ws.hbar : nullptr, a.ws.ds, M, Mp, a.ws.dzh, a.ws.dzl, a.ws.db1_part);
  e = hipGetLastError();
  if (e != hipSuccess || !bwd) return e;
  hipLaunchKernelGGL(lh_small_grads, dim3((a.Hp + 63) / 64), dim3(kLhThreads), 0, a.stream, a.ws.db1_part, a.B, a.Hp, a.B,
                     a.ws.ds, a.ws.hbar, a.db1, a.dw2, a.db2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lh_transpose, dim3((Mp + kTile - 1) / kTile, (a.H + kTile - 1) / kTile), dim3(kLhThreads), 0,
                     a.stream, a.h, M, a.H, Mp, a.ws.hT);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dW1 [H' x H] = (dZ1^T high + remainder) [H' x Mp] . (h^T)^T, reduction over Mp.
  const int rt = nt, ct = (a.H + kTile - 1) / kTile;
  const LhSplit sb = lh_split_k(Mp, (long long)rt * ct);
  hipLaunchKernelGGL((lh_gemm_tn<true>), dim3(rt, ct, sb.S), dim3(kLhThreads), 0, a.stream, a.ws.dzh, a.ws.dzl, Mp,
                     a.ws.hT, Mp, a.ws.dw_part, a.Hp, a.H, Mp, sb.kslice);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sum_slices(a.ws.dw_part, sb.S, (size_t)a.Hp * a.H, a.dW1, a.stream);
}

}  // namespace adaflash
