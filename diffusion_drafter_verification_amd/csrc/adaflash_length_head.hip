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
// The two dense products run on the matrix cores (v_mfma_f32_32x32x16_bf16)
// with fp32 accumulation:
//   forward  Z1 [M x H'] = h [M x H] . W1^T      (M = B k), 64 x 64 output
//            tiles with split-K slices summed in slice order; both operands
//            have the reduction dimension contiguous and are staged through
//            LDS (eight lanes read a row's 128 bytes), so that the matrix
//            instructions read them in their operand layout;
//   backward dW1 [H' x H] = dZ1^T [H' x M] . h [M x H], with dZ1 split into a
//            bf16 high part and a bf16 remainder (two products, ~16 mantissa
//            bits).  dZ1 is written in blocks of eight rows, so that each
//            lane loads its operand directly; h is read in its row layout,
//            four columns of eight rows per lane, regrouped in registers.
//            64 x 128 tiles, the four waves of a workgroup splitting the
//            reduction and summing their tiles in LDS.
// Everything else (bias, SiLU, mean, second layer, loss, small reductions)
// is element-wise or a fixed-order reduction in fp32.  A step is three
// launches forward (product, slice sum, pooling) and two or three backward
// (pooling, weight product with the small gradients, and a slice sum when
// the weight product is split).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaflash_internal.h"

namespace adaflash {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kLhThreads = 256;  // four waves

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

// Matrix-core fragment layout (32 x 32 x 16, bf16 in, fp32 accumulate): lane l
// supplies A[l % 32][8 (l / 32) + 0..7] and B[8 (l / 32) + 0..7][l % 32];
// accumulator register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

constexpr int kTile = kLhFwdTile;  // output tile of the projection (rows and columns)
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

constexpr int kRows = kLhTileR;   // output tile of a workgroup, and of each of its waves
constexpr int kCols = kLhTileC;
constexpr uint32_t kOut = 0x40000000u;  // a buffer offset past every operand range (the load returns zero)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x2_t ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

// Work item of workgroup `id` of `n`: workgroups are dealt to the eight XCDs
// in turn, so consecutive work items (the tiles that share operand rows) are
// placed on the same XCD and share its L2.
__device__ __forceinline__ int xcd_item(int id, int n) { return n % 8 ? id : (id % 8) * (n / 8) + id / 8; }

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
// layer, sigmoid, verify length; with accept_len given also the label, the
// loss and d loss / d s, the pooled vector kept for the weight gradient, and
// this request's entries of dZ1 = ds w2 / k SiLU'(z1) as a bf16 high part and
// remainder, with their column sums for db1 ([B][H']).  dZ1 is stored in
// blocks of eight rows: entry (m, n) at (m / 8, n, m % 8), so that eight
// consecutive rows of one column are 16 contiguous bytes; the entries of the
// last block past the M = B k rows are zero.
__global__ __launch_bounds__(kLhThreads) void lh_pool(const float* __restrict__ Z1, int Hp, int k,
                                                       const float* __restrict__ b1,
                                                       const float* __restrict__ w2, float b2, float gamma,
                                                       float* __restrict__ a_hat, int32_t* __restrict__ k_hat,
                                                       const int32_t* __restrict__ accept_len,
                                                       const int32_t* __restrict__ verify_len,
                                                       float* __restrict__ loss, float* __restrict__ hbar,
                                                       float* __restrict__ ds,
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
  const bool vec = (k & 7) == 0;  // whole blocks per request: 16-byte stores
  for (int n = threadIdx.x; n < Hp; n += kLhThreads) {
    const float bias = b1[n];
    const float wv = dsb * w2[n] * invk;
    float colsum = 0.f;
    auto dz = [&](int i) {
      const float z = Z1[(m0 + i) * Hp + n] + bias;
      const float sg = sigmoidf_(z);
      const float v = wv * (sg * (1.f + z * (1.f - sg)));
      colsum += v;
      return v;
    };
    if (vec) {
      for (int i0 = 0; i0 < k; i0 += 8) {
        u32x4_t hv, lv;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float v0 = dz(i0 + e), v1 = dz(i0 + e + 1);
          const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
          const __bf16 l0 = (__bf16)(v0 - (float)h0), l1 = (__bf16)(v1 - (float)h1);
          hv[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          lv[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
        const size_t at = (((m0 + i0) >> 3) * (size_t)Hp + n) * 8;
        *(u32x4_t*)(dzh + at) = hv;
        *(u32x4_t*)(dzl + at) = lv;
      }
    } else {
      for (int i = 0; i < k; ++i) {
        const float v = dz(i);
        const __bf16 hi = (__bf16)v;
        const __bf16 lo = (__bf16)(v - (float)hi);
        const size_t m = m0 + i, at = ((m >> 3) * Hp + n) * 8 + (m & 7);
        dzh[at] = __builtin_bit_cast(uint16_t, hi);
        dzl[at] = __builtin_bit_cast(uint16_t, lo);
      }
      if (b == (int)gridDim.x - 1) {  // the rest of the last block
        for (size_t m = m0 + k; m & 7; ++m) {
          const size_t at = ((m >> 3) * Hp + n) * 8 + (m & 7);
          dzh[at] = 0;
          dzl[at] = 0;
        }
      }
    }
    db1_part[(size_t)b * Hp + n] = colsum;
  }
}

// db1 = sum of the per-request partials, dw2 = sum_b ds[b] hbar[b], db2 =
// sum_b ds[b], all in a fixed order, for columns 64 tile .. 64 tile + 63 by a
// workgroup of NW waves: wave w sums the partials and requests congruent to
// w mod NW, and the NW partials are added in wave order (LDS scratch:
// 2 NW 64 + NW floats).  Tile 0 also forms db2.
template <int NW>
__device__ void small_grads_tile(int tile, const float* __restrict__ db1_part, int Hp, int B,
                                 const float* __restrict__ ds, const float* __restrict__ hbar,
                                 float* __restrict__ db1, float* __restrict__ dw2, float* __restrict__ db2,
                                 float* lds) {
  float* pa = lds;
  float* pw = lds + 64 * NW;
  float* red = lds + 128 * NW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = tile * 64 + lane;
  float a = 0.f, w = 0.f;
  if (n < Hp) {
#pragma unroll 8
    for (int t = wave; t < B; t += NW) a += db1_part[(size_t)t * Hp + n];
#pragma unroll 8
    for (int b = wave; b < B; b += NW) w = fmaf(ds[b], hbar[(size_t)b * Hp + n], w);
  }
  __syncthreads();  // (the previous tile's partials are read)
  pa[64 * wave + lane] = a;
  pw[64 * wave + lane] = w;
  __syncthreads();
  if (wave == 0 && n < Hp) {
    float sa = pa[lane], sw = pw[lane];
#pragma unroll
    for (int v = 1; v < NW; ++v) {
      sa += pa[64 * v + lane];
      sw += pw[64 * v + lane];
    }
    db1[n] = sa;
    dw2[n] = sw;
  }
  if (tile == 0) {
    float part = 0.f;
    for (int b = threadIdx.x; b < B; b += 64 * NW) part += ds[b];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
      float tot = red[0];
#pragma unroll
      for (int v = 1; v < NW; ++v) tot += red[v];
      *db2 = tot;
    }
  }
}

// Weight gradient, slice z of the reduction over the rows m: C_z [N x Cc]
// (fp32, slice stride N Cc) = sum_m (A[m][n] + A2[m][n]) B[m][c], A, A2 = dZ1
// high part and remainder in blocks of eight rows (entry (m, n) at
// (m / 8, n, m % 8), bf16), B = h (bf16, rows of Cc entries, Cc a multiple of
// 16).  A workgroup of NW waves computes a 64 x 128 tile of C_z; its waves
// take the slice's 16-row steps in turn (wave w: steps w, w + NW, ...) and
// each accumulates the whole tile.  In a step, lane (half, j) loads the 16
// bytes of rows 8 half ... of column n = 32 b + j of each dZ1 block b (the
// matrix instruction's operand as it is stored), and four entries (columns
// 4 j ... 4 j + 3) of the eight rows 8 half ... of h, which it regroups in
// registers into four operands: column 4 j + q of the eight rows for
// fragment q, so that output column jj of fragment q is c = 4 jj + q.
// Out-of-range rows and columns come back as zero from the buffer loads.  The
// high part and remainder go through the same accumulators, every fragment's
// high-part instruction before its remainder's.  The NW partial tiles are
// summed in wave order through LDS, a group of fragments at a time, and
// stored four (NW = 4) or two (NW = 8) columns at a time.
// The first kLhSmallWg workgroups form db1, dw2 and db2 instead
// (small_grads_tile).
constexpr int kLhSmallWg = 8;
// Steps of operands in flight per wave, and waves per workgroup: deeper
// rings (4, 6) and eight waves per workgroup measured slower, as did more
// workgroups (the kernel is bound by the memory system, not by one wave's
// latency).
constexpr int kWgRing = 2;
constexpr int kWgWaves = 4;

template <int NW>
__global__ __launch_bounds__(64 * NW) void lh_wgrad(const uint16_t* __restrict__ A,
                                                     const uint16_t* __restrict__ A2,
                                                     const uint16_t* __restrict__ Bm, float* __restrict__ C,
                                                     int N, int Cc, int M, int kslice, int S, int tiles_n,
                                                     const float* __restrict__ db1_part, int B,
                                                     const float* __restrict__ ds,
                                                     const float* __restrict__ hbar, float* __restrict__ db1,
                                                     float* __restrict__ dw2, float* __restrict__ db2) {
  constexpr int QP = NW == 4 ? 4 : 2;  // fragments summed per pass
  constexpr int kThreads = 64 * NW;
  __shared__ float red[NW * QP * 16 * 64];  // 64 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, j = lane & 31;
  if ((int)blockIdx.x < kLhSmallWg) {
    for (int t = blockIdx.x; t < (N + 63) / 64; t += kLhSmallWg)
      small_grads_tile<NW>(t, db1_part, N, B, ds, hbar, db1, dw2, db2, red);
    return;
  }
  int w = xcd_item((int)blockIdx.x - kLhSmallWg, (int)gridDim.x - kLhSmallWg);
  const int tn = w % tiles_n;  // row tiles fastest: the tiles that read the same columns of h
  w /= tiles_n;
  const int z = w % S, tc = w / S;
  const int n0 = tn * kRows, c0 = tc * kCols;
  const int mb = z * kslice, me = min(M, mb + kslice);
  const uint32_t rowb = (uint32_t)Cc * 2;
  const __amdgpu_buffer_rsrc_t rh = rsrc(Bm + (size_t)mb * Cc, (uint32_t)(me - mb) * rowb);
  const size_t zb = (size_t)(mb >> 3) * N * 8;  // (kslice is a multiple of 8)
  const uint32_t zbytes = (uint32_t)((me - mb + 7) >> 3) * N * 16;
  const __amdgpu_buffer_rsrc_t rz = rsrc(A + zb, zbytes), rz2 = rsrc(A2 + zb, zbytes);
  const uint32_t hcol = c0 + 4 * j < Cc ? (uint32_t)(c0 + 4 * j) * 2 : kOut;
  uint32_t zcol[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) zcol[b] = n0 + 32 * b + j < N ? (uint32_t)(n0 + 32 * b + j) * 16 : kOut;
  const int nst = (me - mb + 15) / 16;
  // steps per wave, a multiple of the ring (the missing ones load as zero)
  const int nt = ((nst + NW - 1) / NW + kWgRing - 1) / kWgRing * kWgRing;
  struct Ops {
    u32x2_t hb[8];
    u32x4_t a[2][2];  // [row block][high part, remainder]
  };
  auto load = [&](Ops& o, int t) {
    const int r0 = 16 * (wave + NW * t) + 8 * half;  // first of the lane's eight rows, from mb
#pragma unroll
    for (int r = 0; r < 8; ++r) o.hb[r] = ld64(rh, (uint32_t)(r0 + r) * rowb + hcol);
    const uint32_t zo = (uint32_t)(r0 >> 3) * N * 16;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      o.a[b][0] = ld128(rz, zo + zcol[b]);
      o.a[b][1] = ld128(rz2, zo + zcol[b]);
    }
  };
  f32x16_t acc[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[b][q] = f32x16_t{};
  auto mac = [&](const Ops& o) {
    u32x4_t bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = o.hb[2 * p][q >> 1], hi = o.hb[2 * p + 1][q >> 1];
        bq[q][p] = (q & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[b][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, o.a[b][s]),
                                                              __builtin_bit_cast(bf16x8_t, bq[q]), acc[b][q],
                                                              0, 0, 0);
  };
  // A ring of kWgRing steps' operands: step t + kWgRing is loaded into the
  // slot that step t has just used.  The scheduling barriers keep each
  // step's instructions in their place (the prologue's too), so that a step
  // waits only for its own loads.
  Ops o[kWgRing];
#pragma unroll
  for (int d = 0; d < kWgRing; ++d) {
    load(o[d], d);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int t = 0; t < nt; t += kWgRing) {
#pragma unroll
    for (int d = 0; d < kWgRing; ++d) {
      mac(o[d]);
      load(o[d], t + d + kWgRing);  // (past the slice: zeros, never used)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  typedef float f32xq_t __attribute__((ext_vector_type(QP)));
  float* Cz = C + (size_t)z * N * Cc;
#pragma unroll
  for (int p = 0; p < 8 / QP; ++p) {
    const int blk = p / (4 / QP), q0 = (p % (4 / QP)) * QP;
    if (p) __syncthreads();  // the previous group is read
#pragma unroll
    for (int qq = 0; qq < QP; ++qq)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((wave * QP + qq) * 16 + r) * 64 + lane] = acc[blk][q0 + qq][r];
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 1024 / kThreads; ++it) {
      const int idx = tid + kThreads * it, r = idx >> 6, ln = idx & 63;
      f32xq_t v;
#pragma unroll
      for (int qq = 0; qq < QP; ++qq) {
        float sum = red[(qq * 16 + r) * 64 + ln];
#pragma unroll
        for (int u = 1; u < NW; ++u) sum += red[((u * QP + qq) * 16 + r) * 64 + ln];
        v[qq] = sum;
      }
      const int n = n0 + 32 * blk + acc_row(r, ln), c = c0 + 4 * (ln & 31) + q0;
      if (n < N && c < Cc) *(f32xq_t*)(Cz + (size_t)n * Cc + c) = v;
    }
  }
}

}  // namespace

hipError_t lh_launch(const LhArgs& a) {
  const int M = a.B * a.k;
  if (M == 0) return hipSuccess;
  const bool bwd = a.accept_len != nullptr;
  hipError_t e = hipSuccess;
  // The projection Z1 = h W1^T: from the caller's copy of the forward's, or
  // computed (split-K slices summed in slice order, so that the pooling
  // kernel reads one value per entry).
  const float* z1 = a.z1_in;
  if (!z1) {
    float* zdst = a.z1_out ? a.z1_out : a.ws.zsum;
    const LhSplit sf = lh_split_fwd(M, a.H, a.Hp);
    hipLaunchKernelGGL(lh_fwd_gemm, dim3((M + kTile - 1) / kTile, (a.Hp + kTile - 1) / kTile, sf.S),
                       dim3(kLhThreads), 0, a.stream, a.h, a.W1, sf.S == 1 ? zdst : a.ws.z1, M, a.Hp, a.H,
                       sf.kslice);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (sf.S > 1) {
      e = sum_slices(a.ws.z1, sf.S, (size_t)M * a.Hp, zdst, a.stream);
      if (e != hipSuccess) return e;
    }
    z1 = zdst;
  }
  hipLaunchKernelGGL(lh_pool, dim3(a.B), dim3(kLhThreads), 0, a.stream, z1, a.Hp, a.k, a.b1, a.w2, a.b2, a.gamma,
                     a.a_hat, a.k_hat, a.accept_len, a.verify_len, a.loss, bwd ? a.ws.hbar : nullptr, a.ws.ds,
                     a.ws.dzh, a.ws.dzl, a.ws.db1_part);
  e = hipGetLastError();
  if (e != hipSuccess || !bwd) return e;
  // dW1 [H' x H] = (dZ1 high + remainder)^T . h, reduction over the M rows,
  // and (first workgroups) db1, dw2, db2.
  const LhSplit sb = lh_split_bwd(M, a.H, a.Hp);
  const int tn = (a.Hp + kRows - 1) / kRows, tc = (a.H + kCols - 1) / kCols;
  const bool direct = sb.S == 1 && ((uintptr_t)a.dW1 & 15) == 0;
  hipLaunchKernelGGL(lh_wgrad<kWgWaves>, dim3(kLhSmallWg + tn * tc * sb.S), dim3(64 * kWgWaves), 0, a.stream,
                     a.ws.dzh,
                     a.ws.dzl, a.h, direct ? a.dW1 : a.ws.dw_part, a.Hp, a.H, M, sb.kslice, sb.S, tn,
                     a.ws.db1_part, a.B, a.ws.ds, a.ws.hbar, a.db1, a.dw2, a.db2);
  e = hipGetLastError();
  if (e != hipSuccess || direct) return e;
  return sum_slices(a.ws.dw_part, sb.S, (size_t)a.Hp * a.H, a.dW1, a.stream);
}

}  // namespace adaflash
