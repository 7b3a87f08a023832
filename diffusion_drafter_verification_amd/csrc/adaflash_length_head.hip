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
// The two dense products run on the matrix cores (v_mfma_f32_32x32x16_bf16),
// in 64 x 64 output tiles with split-K slices summed in slice order:
//   forward  Z1 [M x H'] = h [M x H] . W1^T      (M = B k), both operands with
//            the reduction dimension contiguous, one 16-byte load per lane;
//   backward dW1 [H' x H] = dZ1^T [H' x M] . h [M x H], with dZ1 split into a
//            bf16 high part and a bf16 remainder (two products, ~16 mantissa
//            bits); dZ1 and h are read in their natural row layout and
//            transposed in LDS.
// Everything else (bias, SiLU, mean, second layer, loss, small reductions)
// is element-wise or a fixed-order reduction in fp32.  A step is three
// launches forward (product, slice sum, pooling) and three backward
// (pooling, weight product with the small gradients, slice sum).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaflash_internal.h"

namespace adaflash {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLhThreads = 256;  // four waves

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

// Matrix-core fragment layout (32 x 32 x 16, bf16 in, fp32 accumulate): lane l
// supplies A[l % 32][8 (l / 32) + 0..7] and B[8 (l / 32) + 0..7][l % 32];
// accumulator register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

constexpr int kTile = kLhTile;     // output tile (rows and columns)
constexpr int kKs = 64;           // reduction step staged per round
constexpr int kLdsRow = kKs + 8;  // bf16 per LDS row (16 bytes of padding)

// Projection, split-K slice z = blockIdx.z: C_z [M x N] (fp32, slice stride
// M N) = A [M x K_z] . B [N x K_z]^T, A = h and B = W1, bf16 rows of K
// entries with the reduction dimension contiguous (K a multiple of 16, rows
// 16-byte aligned).  The workgroup stages 64-wide steps of the reduction
// through LDS (each row's 128 bytes read by eight adjacent threads), then
// every wave multiplies its 32 x 32 tile from LDS; the next round's operands
// are loaded into registers while the matrix cores work on the current one.
__global__ __launch_bounds__(kLhThreads) void lh_fwd_gemm(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ Bm, float* __restrict__ C,
                                                           int M, int N, int K, int kslice) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[kTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t sb[kTile * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt0 = blockIdx.x * kTile, nt0 = blockIdx.y * kTile;
  const int kb = blockIdx.z * kslice;
  const int ke = min(K, kb + kslice);
  const int lr = tid >> 3, lc = (tid & 7) * 8;  // staging: rows lr and lr + 32, 16 bytes at lc
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x16_t acc = {};
  const int wr = 32 * (wave >> 1), wc = 32 * (wave & 1);
  const int ko = 8 * (lane >> 5);
  u32x4_t ga[2], gb[2];
  auto fetch = [&](int k0) {
    const int kk = k0 + lc;
    const bool okk = kk < ke;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ra = mt0 + lr + 32 * h, rb = nt0 + lr + 32 * h;
      ga[h] = (ra < M && okk) ? *(const u32x4_t*)(A + (size_t)ra * K + kk) : zero;
      gb[h] = (rb < N && okk) ? *(const u32x4_t*)(Bm + (size_t)rb * K + kk) : zero;
    }
  };
  if (kb < ke) fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += kKs) {
    __syncthreads();  // the previous round's fragments are consumed
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *(u32x4_t*)&sa[(lr + 32 * h) * kLdsRow + lc] = ga[h];
      *(u32x4_t*)&sb[(lr + 32 * h) * kLdsRow + lc] = gb[h];
    }
    __syncthreads();
    if (k0 + kKs < ke) fetch(k0 + kKs);
#pragma unroll
    for (int t = 0; t < kKs / 16; ++t) {
      const int kc = 16 * t + ko;
      const u32x4_t a = *(const u32x4_t*)&sa[(wr + (lane & 31)) * kLdsRow + kc];
      const u32x4_t b = *(const u32x4_t*)&sb[(wc + (lane & 31)) * kLdsRow + kc];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                    acc, 0, 0, 0);
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
// layer, sigmoid, verify length; with accept_len given also
// the label, the loss and d loss / d s, the pooled vector kept for the weight
// gradient, and this request's rows of dZ1 = ds w2 / k SiLU'(z1) as a bf16
// high part and remainder (row stride Hq), with its column sums for db1
// ([B][H']).
__global__ __launch_bounds__(kLhThreads) void lh_pool(const float* __restrict__ Z1, int Hp, int k,
                                                       const float* __restrict__ b1,
                                                       const float* __restrict__ w2, float b2, float gamma,
                                                       float* __restrict__ a_hat, int32_t* __restrict__ k_hat,
                                                       const int32_t* __restrict__ accept_len,
                                                       const int32_t* __restrict__ verify_len,
                                                       float* __restrict__ loss, float* __restrict__ hbar,
                                                       float* __restrict__ ds, int Hq,
                                                       uint16_t* __restrict__ dzh, uint16_t* __restrict__ dzl,
                                                       float* __restrict__ db1_part) {
  __shared__ float red[4];
  __shared__ float sh_ds;
  const int b = blockIdx.x;
  const float invk = 1.f / (float)k;
  const size_t m0 = (size_t)b * k;
  float part = 0.f;
  for (int n = threadIdx.x; n < Hp; n += kLhThreads) {
    const float bias = b1[n];
    float acc = 0.f;
#pragma unroll 8
    for (int i = 0; i < k; ++i) {
      const float z = Z1[(m0 + i) * Hp + n] + bias;
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
  for (int n = threadIdx.x; n < Hp; n += kLhThreads) {
    const float bias = b1[n];
    const float wv = dsb * w2[n] * invk;
    float colsum = 0.f;
    for (int i = 0; i < k; ++i) {
      const float z = Z1[(m0 + i) * Hp + n] + bias;
      const float sg = sigmoidf_(z);
      const float v = wv * (sg * (1.f + z * (1.f - sg)));
      colsum += v;
      const __bf16 hi = (__bf16)v;
      const __bf16 lo = (__bf16)(v - (float)hi);
      dzh[(m0 + i) * Hq + n] = __builtin_bit_cast(uint16_t, hi);
      dzl[(m0 + i) * Hq + n] = __builtin_bit_cast(uint16_t, lo);
    }
    db1_part[(size_t)b * Hp + n] = colsum;
  }
}

// db1 = sum of the per-request partials, dw2 = sum_b ds[b] hbar[b], db2 =
// sum_b ds[b], all in a fixed order, for columns 64 tile .. 64 tile + 63: wave
// w sums the partials and requests congruent to w mod 4, and the four
// partials are added in wave order.  Tile 0 also forms db2.
__device__ void small_grads_tile(int tile, const float* __restrict__ db1_part, int Hp, int B,
                                 const float* __restrict__ ds, const float* __restrict__ hbar,
                                 float* __restrict__ db1, float* __restrict__ dw2, float* __restrict__ db2) {
  __shared__ float red[4];
  __shared__ float pa[4][64], pw[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = tile * 64 + lane;
  float a = 0.f, w = 0.f;
  if (n < Hp) {
#pragma unroll 4
    for (int t = wave; t < B; t += 4) a += db1_part[(size_t)t * Hp + n];
#pragma unroll 4
    for (int b = wave; b < B; b += 4) w = fmaf(ds[b], hbar[(size_t)b * Hp + n], w);
  }
  __syncthreads();  // (the previous tile's partials are read)
  pa[wave][lane] = a;
  pw[wave][lane] = w;
  __syncthreads();
  if (wave == 0 && n < Hp) {
    db1[n] = (pa[0][lane] + pa[1][lane]) + (pa[2][lane] + pa[3][lane]);
    dw2[n] = (pw[0][lane] + pw[1][lane]) + (pw[2][lane] + pw[3][lane]);
  }
  if (tile == 0) {
    float part = 0.f;
    for (int b = threadIdx.x; b < B; b += kLhThreads) part += ds[b];
    const float tot = lh_block_sum(part, red);
    if (threadIdx.x == 0) *db2 = tot;
  }
}

// Weight gradient, split-K slice s over the rows m: C_s [N x Cc] (fp32, slice
// stride N Cc) = sum_m (A[m][n] + A2[m][n]) B[m][c], A, A2 = dZ1 high part
// and remainder (bf16, rows of lda entries, lda a multiple of 8), B = h
// (bf16, rows of Cc entries, Cc a multiple of 16).  Both are read in their
// natural row layout: in each 64-row round, waves 0, 1 and 2 stage A, A2 and
// B, lane l taking the 8 x 8 block of rows 8 (l % 8) ... and columns
// 8 (l / 8) ... (eight 16-byte row loads), which it transposes in registers
// and stores as eight 16-byte LDS rows, one per column, so that the matrix
// cores read the reduction dimension contiguously.  Every wave then
// multiplies its 32 x 32 tile of the 64 x 64 output tile.
// The workgroups of the extra slice z = 0, dispatched first, form db1, dw2 and
// db2 instead (small_grads_tile); slice s of the product is z = s + 1.
__global__ __launch_bounds__(kLhThreads) void lh_wgrad_gemm(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ A2, int lda,
                                                             const uint16_t* __restrict__ Bm,
                                                             float* __restrict__ C, int N, int Cc, int M,
                                                             int kslice, const float* __restrict__ db1_part,
                                                             int B, const float* __restrict__ ds,
                                                             const float* __restrict__ hbar,
                                                             float* __restrict__ db1, float* __restrict__ dw2,
                                                             float* __restrict__ db2) {
  __shared__ __attribute__((aligned(16))) uint16_t sop[3][kTile * kLdsRow];  // A, A2, B transposed
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.z == 0) {
    const int nwg = (int)(gridDim.x * gridDim.y);
    for (int t = (int)(blockIdx.y * gridDim.x + blockIdx.x); t < (N + 63) / 64; t += nwg)
      small_grads_tile(t, db1_part, N, B, ds, hbar, db1, dw2, db2);
    return;
  }
  const int zs = (int)blockIdx.z - 1;  // slice of the product
  const int n0 = blockIdx.x * kTile, c0 = blockIdx.y * kTile;
  const int mb = zs * kslice;
  const int me = min(M, mb + kslice);
  // Staging (waves 0-2): operand `wave`, rows 8 rb ..., columns 8 cg ...
  const int rb = lane & 7, cg = lane >> 3;
  const uint16_t* src = wave == 0 ? A : (wave == 1 ? A2 : Bm);
  const int ld = wave == 2 ? Cc : lda;
  const int col = (wave == 2 ? c0 : n0) + 8 * cg;
  const bool colok = col < (wave == 2 ? Cc : N);
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x16_t acc = {};
  const int wn = 32 * (wave >> 1), wc = 32 * (wave & 1);
  const int ko = 8 * (lane >> 5), l32 = lane & 31;
  u32x4_t rr[8];
  auto fetch = [&](int m0) {
    if (wave < 3) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + 8 * rb + i;
        rr[i] = (m < me && colok) ? *(const u32x4_t*)(src + (size_t)m * ld + col) : zero;
      }
    }
  };
  if (mb < me) fetch(mb);
  for (int m0 = mb; m0 < me; m0 += kKs) {
    __syncthreads();  // the previous round's fragments are consumed
    if (wave < 3) {
      // Column j of the block: entries j of rows 0..7, two rows per word.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4_t t;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = rr[2 * q][j >> 1], hi = rr[2 * q + 1][j >> 1];
          t[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        *(u32x4_t*)&sop[wave][(8 * cg + j) * kLdsRow + 8 * rb] = t;
      }
    }
    __syncthreads();
    if (m0 + kKs < me) fetch(m0 + kKs);
#pragma unroll
    for (int t = 0; t < kKs / 16; ++t) {
      const int kc = 16 * t + ko;
      const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sop[0][(wn + l32) * kLdsRow + kc]);
      const bf16x8_t al = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sop[1][(wn + l32) * kLdsRow + kc]);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sop[2][(wc + l32) * kLdsRow + kc]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bv, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bv, acc, 0, 0, 0);
    }
  }
  float* Cz = C + (size_t)zs * N * Cc;
  const int oc = c0 + wc + l32;
  if (oc < Cc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = n0 + wn + acc_row(r, lane);
      if (row < N) Cz[(size_t)row * Cc + oc] = acc[r];
    }
  }
}

}  // namespace

hipError_t lh_launch(const LhArgs& a) {
  const int M = a.B * a.k;
  if (M == 0) return hipSuccess;
  const int Hq = (a.Hp + 7) & ~7;
  const bool bwd = a.accept_len != nullptr;
  hipError_t e = hipSuccess;
  // The projection Z1 = h W1^T: from the caller's copy of the forward's, or
  // computed (split-K slices summed in slice order, so that the pooling
  // kernel reads one value per entry).
  const float* z1 = a.z1_in;
  if (!z1) {
    float* zdst = a.z1_out ? a.z1_out : a.ws.zsum;
    const LhSplit sf = lh_split_k(a.H, lh_tiles(M, a.Hp));
    hipLaunchKernelGGL(lh_fwd_gemm, dim3((M + kTile - 1) / kTile, (a.Hp + kTile - 1) / kTile, sf.S),
                       dim3(kLhThreads), 0, a.stream, a.h, a.W1, a.ws.z1, M, a.Hp, a.H, sf.kslice);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = sum_slices(a.ws.z1, sf.S, (size_t)M * a.Hp, zdst, a.stream);
    if (e != hipSuccess) return e;
    z1 = zdst;
  }
  hipLaunchKernelGGL(lh_pool, dim3(a.B), dim3(kLhThreads), 0, a.stream, z1, a.Hp, a.k, a.b1, a.w2, a.b2, a.gamma,
                     a.a_hat, a.k_hat, a.accept_len, a.verify_len, a.loss, bwd ? a.ws.hbar : nullptr, a.ws.ds,
                     Hq, a.ws.dzh, a.ws.dzl, a.ws.db1_part);
  e = hipGetLastError();
  if (e != hipSuccess || !bwd) return e;
  // dW1 [H' x H] = (dZ1 high + remainder)^T . h, reduction over the M rows,
  // and (extra first slice) db1, dw2, db2.
  const LhSplit sb = lh_split_k(M, lh_tiles(a.Hp, a.H));
  hipLaunchKernelGGL(lh_wgrad_gemm, dim3((a.Hp + kTile - 1) / kTile, (a.H + kTile - 1) / kTile, sb.S + 1),
                     dim3(kLhThreads), 0, a.stream, a.ws.dzh, a.ws.dzl, Hq, a.h, a.ws.dw_part, a.Hp, a.H, M,
                     sb.kslice, a.ws.db1_part, a.B, a.ws.ds, a.ws.hbar, a.db1, a.dw2, a.db2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sum_slices(a.ws.dw_part, sb.S, (size_t)a.Hp * a.H, a.dW1, a.stream);
}

}  // namespace adaflash
