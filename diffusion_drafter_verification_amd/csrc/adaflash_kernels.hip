// gfx950 (CDNA4) kernels for the ragged verify-and-supervise pass.
//
// Work decomposition
//   The pack kernel clamps the verify lengths, writes the packed row offsets
//   and the packed-row -> (request, position) map, and clears the arrival
//   counters.  Request b contributes its L_b verified rows plus, when
//   verifying, its bonus row L_b.
//
//   The row kernels give each (row, chunk) pair one 256-thread workgroup.  A
//   chunk is kChunk = 8192 consecutive vocabulary entries; each thread keeps
//   32 entries of the target row and 32 of the draft row in registers,
//   loaded with 16-byte coalesced, non-temporal loads.  Row-global
//   quantities (maxima, sums of exponentials, the supervision sums) are
//   exchanged between the chunks of a row through per-chunk partial records
//   and an arrival counter: every workgroup publishes its partial,
//   increments the row counter and waits for the others, then combines all
//   partials in chunk order (so every chunk derives bit-identical row
//   statistics).  The logits therefore cross HBM exactly once however many
//   logical passes the maths needs.
//
//   Each wait is bounded: past the bound the workgroup sets
//   ADAFLASH_FLAG_SYNC_TIMEOUT and leaves, so the grid always drains.  A
//   row's workgroups have consecutive ids and depend only on each other;
//   with workgroups dispatched in id order, a waiting workgroup's partners are
//   resident or next in line, so the bound is never reached in practice.
//
//   The finaliser kernel (one workgroup per request) then takes the first
//   rejection and draws the correction token from the residual max(0, p - q)
//   of row A, or the bonus token from target row L, by locating the chunk
//   whose cumulative mass crosses the threshold and scanning only that chunk.
//
// Maths (pages cited in adaflash.h):
//   p = softmax(z_p / T), q = softmax(z_q / T); accept x_i iff u_i q(x_i) < p(x_i);
//   residual r = max(0, p_A - q_A); draw = smallest v with running sum > u Z.
//   Supervision at temperature 1, per verified row:
//     lq = z_q - lse_q, lp = z_p - lse_p, q = exp(lq), f = q (lq - lp),
//     U = {v : f_v <= c}, R = sum_U f + c |V \ U|, S = sum_U (f + q),
//     CE = lse_q - z_q[x*], grad = q - e_{x*} + lambda q (1_U (lq - lp + 1) - S).
//   Exponentials use v_exp_f32 (2^x) on log2-scaled arguments.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <vector>

#include "adaflash_internal.h"

#define ADAFLASH_FLAG_BAD_VERIFY_LEN 1
#define ADAFLASH_FLAG_BAD_TOKEN 2
#define ADAFLASH_FLAG_NONFINITE 4
#define ADAFLASH_FLAG_SYNC_TIMEOUT 8

namespace adaflash {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWaves = kThreads / 64;
static_assert(kWaves == 4, "the workgroup reductions combine four waves");
constexpr int kIntMax = 0x7fffffff;
constexpr int kSpinLimit = 1 << 18;  // bound on polls (~0.2 us of s_sleep between polls)

struct KParams {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* margins;
  int32_t* row_offsets;
  float* loss_ce;
  float* loss_rkl;
  void* grad;
  int32_t* status;
  int32_t* Lc;
  const int32_t* rowmap;
  int32_t* rowcnt;
  float* part1;
  float* part2;
  float* rowrec;
  uint32_t* epoch;  // this call's epoch (advanced by the pack step)
  int B, k, V, G;
  float kT;  // log2(e) / T (0 in greedy mode)
  float clip_c, lambda;
  // Supervision loss variants: weight of the hard-label term (1 for the
  // default loss), per-position weight decay (0: none; else row i weighs
  // exp(-i / wdecay)), and the combined per-row loss output (or null).
  float a_ce, wdecay;
  float* loss_var;
  // Logit layout: 0 = padded [B, k+1, V] / [B, k, V]; 1 = packed
  // [sum (L_b + 1), V] / [sum L_b, V] (rows located through row_offsets).
  int packed;
  // Verify-only, padded layout: the first kernel's block 0 does the pack
  // kernel's work (clamped lengths, row offsets, status word), and the other
  // blocks clamp their own request's length from verify_len.
  int pack_here;
  const int32_t* verify_len;
  // Verification alone: chunks of a row per residual workgroup (the residual
  // grid is sized to be resident at once).
  int res_chunks;
};

// ---------------------------------------------------------------- primitives

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A product rounded on its own, never fused into a following addition.  The
// residual max(0, p - q) is a difference of two such products: when the target
// and draft rows are identical both round to the same value and the residual is
// exactly zero (no rejection can occur then, except on a zero-mass draft token,
// and the draw falls back to the target row).  A contracted fma(p', s, -q)
// would leave rounding noise there instead.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// Wave reduction: a butterfly inside each 16-lane row (xor 1, xor 2, mirror 8,
// mirror 16) leaves every lane of a row with the row result; two row
// broadcasts (lane 15 into rows 1 and 3, then lane 31 into rows 2 and 3)
// accumulate the four rows into lane 63, which is read as a uniform value.
// The combination order is fixed, so the result is deterministic.  Must be
// called with all lanes active.
enum { OP_SUM = 0, OP_MAX = 1, OP_MINI = 2, OP_MAXI = 3 };

template <int OP>
__device__ __forceinline__ float op2(float a, float b) {
  if constexpr (OP == OP_SUM) return a + b;
  if constexpr (OP == OP_MAX) return fmaxf(a, b);
  if constexpr (OP == OP_MAXI) return __int_as_float(max(__float_as_int(a), __float_as_int(b)));
  return __int_as_float(min(__float_as_int(a), __float_as_int(b)));
}

template <int OP>
__device__ __forceinline__ float op_identity() {
  if constexpr (OP == OP_SUM) return -0.f;  // exact identity of addition, also for -0
  if constexpr (OP == OP_MAX) return -__builtin_inff();
  if constexpr (OP == OP_MAXI) return __int_as_float((int)0x80000000);
  return __int_as_float(0x7fffffff);
}

// A value known to be the same in every lane, moved to a scalar register.
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Order-preserving map of float bit patterns to signed integers (and back:
// the map is its own inverse).  A float maximum becomes an integer maximum,
// which needs no NaN canonicalisation.  Only used where no operand is NaN.
__device__ __forceinline__ int max_key(int x) { return x ^ ((x >> 31) & 0x7fffffff); }

// DPP move restricted to the rows in ROWMASK; other rows receive `old`.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_rows(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}

template <int OP>
__device__ __forceinline__ float wave_reduce(float v) {
  if constexpr (OP == OP_MAX) {
    // Maxima of finite values or -inf: reduced as integer keys.
    const float k = __int_as_float(max_key(__float_as_int(v)));
    return __int_as_float(max_key(__float_as_int(wave_reduce<OP_MAXI>(k))));
  }
  v = op2<OP>(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op2<OP>(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op2<OP>(v, dpp_f<0x141>(v));  // row_half_mirror
  v = op2<OP>(v, dpp_f<0x140>(v));  // row_mirror
  v = op2<OP>(v, dpp_rows<0x142, 0xA>(v, op_identity<OP>()));  // row_bcast:15
  v = op2<OP>(v, dpp_rows<0x143, 0xC>(v, op_identity<OP>()));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// As wave_reduce, but the result is left in lane 63 only (no broadcast).
template <int OP>
__device__ __forceinline__ float wave_reduce_l63(float v) {
  if constexpr (OP == OP_MAX) {
    const float k = __int_as_float(max_key(__float_as_int(v)));
    return __int_as_float(max_key(__float_as_int(wave_reduce_l63<OP_MAXI>(k))));
  }
  v = op2<OP>(v, dpp_f<0xB1>(v));
  v = op2<OP>(v, dpp_f<0x4E>(v));
  v = op2<OP>(v, dpp_f<0x141>(v));
  v = op2<OP>(v, dpp_f<0x140>(v));
  v = op2<OP>(v, dpp_rows<0x142, 0xA>(v, op_identity<OP>()));
  v = op2<OP>(v, dpp_rows<0x143, 0xC>(v, op_identity<OP>()));
  return v;
}

// Workgroup reduction whose results only thread 0 needs: the same values, in
// the same combination order, as wg_reduce, valid in thread 0 only.  `red` is
// free again once every thread has passed the next barrier.
template <int N>
__device__ __forceinline__ void wg_reduce_lead(float (&v)[N], const int (&ops)[N], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float x = v[n];
    if (ops[n] == OP_SUM) x = wave_reduce_l63<OP_SUM>(x);
    else if (ops[n] == OP_MAX) x = wave_reduce_l63<OP_MAX>(x);
    else if (ops[n] == OP_MAXI) x = wave_reduce_l63<OP_MAXI>(x);
    else x = wave_reduce_l63<OP_MINI>(x);
    v[n] = x;
  }
  if (lane == 63) {
#pragma unroll
    for (int n = 0; n < N; ++n) red[wave * N + n] = v[n];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float a = red[0 * N + n], b = red[1 * N + n], c = red[2 * N + n], d = red[3 * N + n];
      if (ops[n] == OP_SUM) v[n] = (a + b) + (c + d);
      else if (ops[n] == OP_MAX) v[n] = fmaxf(fmaxf(a, b), fmaxf(c, d));
      else if (ops[n] == OP_MAXI) v[n] = op2<OP_MAXI>(op2<OP_MAXI>(a, b), op2<OP_MAXI>(c, d));
      else v[n] = op2<OP_MINI>(op2<OP_MINI>(a, b), op2<OP_MINI>(c, d));
    }
  }
}

// Workgroup reduction of N values with per-value operators; every thread gets
// the same results.  `red` is shared scratch of kWaves*N floats.
template <int N>
__device__ __forceinline__ void wg_reduce(float (&v)[N], const int (&ops)[N], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float x = v[n];
    if (ops[n] == OP_SUM) x = wave_reduce<OP_SUM>(x);
    else if (ops[n] == OP_MAX) x = wave_reduce<OP_MAX>(x);
    else if (ops[n] == OP_MAXI) x = wave_reduce<OP_MAXI>(x);
    else x = wave_reduce<OP_MINI>(x);
    v[n] = x;
  }
  if (lane == 0) {
#pragma unroll
    for (int n = 0; n < N; ++n) red[wave * N + n] = v[n];
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float a = red[0 * N + n], b = red[1 * N + n], c = red[2 * N + n], d = red[3 * N + n];
    float x;
    if (ops[n] == OP_SUM) x = (a + b) + (c + d);
    else if (ops[n] == OP_MAX) x = fmaxf(fmaxf(a, b), fmaxf(c, d));
    else if (ops[n] == OP_MAXI) x = op2<OP_MAXI>(op2<OP_MAXI>(a, b), op2<OP_MAXI>(c, d));
    else x = op2<OP_MINI>(op2<OP_MINI>(a, b), op2<OP_MINI>(c, d));
    v[n] = uniform(x);
  }
  __syncthreads();
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the
// sum of all values.  Deterministic (fixed shuffle tree).  `red` holds kWaves floats.
__device__ __forceinline__ float wg_scan_excl(float x, float* red, float* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  float ex = __shfl_up(v, 1, 64);
  if (lane == 0) ex = 0.f;
  if (lane == 63) red[wave] = v;
  __syncthreads();
  float wb = 0.f;
  for (int w = 0; w < wave; ++w) wb += red[w];
  *total = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return wb + ex;
}

// Cross-workgroup records.  Everything one workgroup publishes for another
// (chunk records, accept flags) is written and read with agent-scope relaxed
// atomics, which are coherent across the XCDs' L2 caches; a wait on every
// outstanding memory operation before the counter increment makes those
// stores complete first, and the readers issue their loads only after they
// have seen the counter.  Agent-scope release/acquire fences would also write
// back and invalidate the L2 at every barrier, which measured about 15x slower
// for this grid.
__device__ __forceinline__ void pub_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float pub_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void complete_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Arrive at a counter and wait until it reaches `target`.  Thread 0 arrives
// and polls; the rest of the workgroup waits at the barrier.  Returns false
// if the wait hit its bound (or another wait already did).
__device__ bool arrive_and_wait(int32_t* cnt, int target, int32_t* status, int* sh) {
  if (threadIdx.x == 0) {
    complete_stores();
    __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1, spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(6);
      ++spins;
      if (spins > kSpinLimit ||
          ((spins & 63) == 0 && status &&
           (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ADAFLASH_FLAG_SYNC_TIMEOUT))) {
        ok = 0;
        break;
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (!ok && status) __hip_atomic_fetch_or(status, ADAFLASH_FLAG_SYNC_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sh = ok;
  }
  __syncthreads();
  int ok = *sh;
  __syncthreads();
  return ok != 0;
}

__device__ __forceinline__ void flag(int32_t* status, int bits) {
  if (status) __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged record fields: a value and the call's epoch in one 64-bit word,
// written and read with single agent-scope atomic accesses.  A reader that
// finds the current epoch in a field holds that field's value from this call,
// whatever the order in which the writer's stores and its arrival at the row
// counter became visible: the writer counts its arrival without waiting for
// its record stores to complete, and a reader re-reads only a field that is
// not there yet.  The epoch word sits at the start of the workspace and grows
// by one per call, so no field left by an earlier call (or any constant fill)
// carries the current epoch.
__device__ __forceinline__ void tag_store(float* base, size_t field, float v, uint32_t ep) {
  __hip_atomic_store((uint64_t*)base + field, ((uint64_t)ep << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tag_load(const float* base, size_t field) {
  return __hip_atomic_load((uint64_t*)const_cast<float*>(base) + field, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tag_value(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t ep) { return (uint32_t)(w >> 32) == ep; }

// A wave waits until the counter reaches `target` (every lane reads the same
// word: one request per poll).  Returns false when the wait hit its bound
// (flagging the status word) or another wait already did.
__device__ bool wait_count(const int32_t* cnt, int target, int32_t* status) {
  int spins = 0;
  while (__builtin_amdgcn_readfirstlane(
             __hip_atomic_load(const_cast<int32_t*>(cnt), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < target) {
    __builtin_amdgcn_s_sleep(4);
    ++spins;
    if (spins > kSpinLimit ||
        ((spins & 63) == 0 && status &&
         (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ADAFLASH_FLAG_SYNC_TIMEOUT))) {
      if ((threadIdx.x & 63) == 0) flag(status, ADAFLASH_FLAG_SYNC_TIMEOUT);
      return false;
    }
  }
  return true;
}

// A wave waits until, in every lane with `want`, fields [off, off + cnt) of
// record `rec` at recs (records `stride` fields apart; cnt <= N) carry epoch
// ep, and leaves their values in v[0 .. cnt).  Lanes poll only their own
// incomplete fields.  Returns false when the wait hit its bound (flagging the
// status word) or another wait already did.  Must be called by a whole wave.
template <int N>
__device__ bool poll_fields(const float* recs, int stride, bool want, int rec, int off, int cnt, uint32_t ep,
                            float (&v)[N], int32_t* status) {
  const int lane = threadIdx.x & 63;
  bool done = !want;
  int spins = 0;
  for (;;) {
    if (!done) {
      uint64_t w[N];
#pragma unroll
      for (int n = 0; n < N; ++n) w[n] = n < cnt ? tag_load(recs, (size_t)rec * stride + off + n) : 0ull;
      done = true;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        if (n < cnt) {
          done = done && tag_is(w[n], ep);
          v[n] = tag_value(w[n]);
        }
      }
    }
    if (__ballot(!done) == 0ull) return true;
    __builtin_amdgcn_s_sleep(2);
    ++spins;
    if (spins > kSpinLimit ||
        ((spins & 63) == 0 && status &&
         (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ADAFLASH_FLAG_SYNC_TIMEOUT))) {
      if (lane == 0) flag(status, ADAFLASH_FLAG_SYNC_TIMEOUT);
      return false;
    }
  }
}

// ------------------------------------------------------------ chunk storage

// kElems entries of one row held by one thread.  Entry e sits at vocabulary
// index v0 + (e / VEC) * kThreads * VEC + tid * VEC + e % VEC, so each slot is
// one coalesced 16-byte load across the workgroup.  Entries past V read as the
// most negative finite value in both rows: they add nothing to maxima or sums
// of exponentials, and unlike -inf their difference z_q - z_p is 0, not NaN.
template <bool BF16>
struct Chunk {
  static constexpr int VEC = BF16 ? 8 : 4;
  static constexpr int NW = BF16 ? kElems / 2 : kElems;
  uint32_t w[NW];

  // Makes the packed words opaque to the optimiser so that values unpacked
  // before this point are recomputed (one shift or mask each) rather than
  // kept live across the workgroup reductions.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int q = 0; q < NW; ++q) asm volatile("" : "+v"(w[q]));
  }

  __device__ __forceinline__ float get(int e) const {
    if constexpr (BF16) {
      uint32_t x = w[e >> 1];
      return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    } else {
      return __uint_as_float(w[e]);
    }
  }
};

// Largest entry of a chunk (exact, as a float).  bf16: packed 16-bit integer
// maxima and minima of the raw words, two entries per instruction and no
// unpacking.  Patterns of non-negative values order like signed integers,
// while among negative values the largest has the smallest signed pattern:
// the maximum is the largest signed pattern if that is non-negative, else
// the smallest one.
template <bool BF16>
__device__ __forceinline__ float chunk_max(const Chunk<BF16>& c) {
  if constexpr (BF16) {
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
    s16x2_t mx = {-32768, -32768}, mn = {32767, 32767};
#pragma unroll
    for (int q = 0; q < Chunk<BF16>::NW; ++q) {
      const s16x2_t w = __builtin_bit_cast(s16x2_t, c.w[q]);
      mx = __builtin_elementwise_max(mx, w);
      mn = __builtin_elementwise_min(mn, w);
    }
    const int a = max((int)mx.x, (int)mx.y);
    const int bits = a >= 0 ? a : min((int)mn.x, (int)mn.y);
    return __uint_as_float((uint32_t)(uint16_t)bits << 16);
  } else {
    float m = neg_inf();
#pragma unroll
    for (int e = 0; e < kElems; ++e) m = fmaxf(m, c.get(e));
    return m;
  }
}

template <bool BF16>
__device__ __forceinline__ int entry_index(int v0, int e) {
  constexpr int VEC = Chunk<BF16>::VEC;
  return v0 + (e / VEC) * (kThreads * VEC) + (int)threadIdx.x * VEC + (e % VEC);
}

// Buffer resource of one row (base and byte length in scalar registers).  A
// whole-chunk access then needs one thread offset in a vector register and
// the slot offset in a scalar register: no 64-bit address arithmetic per slot.
// Cache policy of the whole-chunk logit loads and gradient stores: every
// byte is touched once, so they are marked non-temporal (the streaming
// hint); measured about 15% more HBM throughput for this access pattern.
constexpr int kStreamPolicy = 2;  // nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, bytes, 0x00020000);
}

template <bool BF16, bool ALIGNED>
__device__ __forceinline__ void load_chunk(Chunk<BF16>& c, const void* row, int v0, int V) {
  constexpr int VEC = Chunk<BF16>::VEC;
  constexpr int NV = kElems / VEC;
  constexpr int ES = BF16 ? 2 : 4;
  const uint32_t ninf = BF16 ? 0xff7fff7fu : 0xff7fffffu;  // -max finite
  if constexpr (ALIGNED) {
    if (v0 + kChunk <= V) {  // whole chunk inside the row: no per-slot guards
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, V * ES);
      const int toff = (int)threadIdx.x * 16;
#pragma unroll
      for (int s = 0; s < NV; ++s) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, toff, (v0 + s * (kThreads * VEC)) * ES, kStreamPolicy);
        c.w[s * 4 + 0] = q[0];
        c.w[s * 4 + 1] = q[1];
        c.w[s * 4 + 2] = q[2];
        c.w[s * 4 + 3] = q[3];
      }
      return;
    }
  }
#pragma unroll
  for (int s = 0; s < NV; ++s) {
    const int idx0 = v0 + s * (kThreads * VEC) + (int)threadIdx.x * VEC;
    if constexpr (ALIGNED) {
      if (idx0 < V) {
        const uint4 q = BF16 ? *(const uint4*)((const uint16_t*)row + idx0)
                             : *(const uint4*)((const float*)row + idx0);
        c.w[s * 4 + 0] = q.x;
        c.w[s * 4 + 1] = q.y;
        c.w[s * 4 + 2] = q.z;
        c.w[s * 4 + 3] = q.w;
      } else {
        c.w[s * 4 + 0] = ninf;
        c.w[s * 4 + 1] = ninf;
        c.w[s * 4 + 2] = ninf;
        c.w[s * 4 + 3] = ninf;
      }
    } else {
#pragma unroll
      for (int u = 0; u < VEC; ++u) {
        const int idx = idx0 + u;
        if constexpr (BF16) {
          uint32_t h = idx < V ? (uint32_t)((const uint16_t*)row)[idx] : 0xff7fu;
          const int wi = s * 4 + (u >> 1);
          if (u & 1) c.w[wi] |= h << 16;
          else c.w[wi] = h;
        } else {
          c.w[s * VEC + u] = idx < V ? __float_as_uint(((const float*)row)[idx]) : ninf;
        }
      }
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float load_logit(const void* row, int v) {
  if constexpr (BF16) return __uint_as_float((uint32_t)((const uint16_t*)row)[v] << 16);
  else return ((const float*)row)[v];
}

// Uniform loads of read-only data through the scalar cache (the data were
// written before the kernel started; the scalar cache is invalidated at each
// kernel launch).  The result lives in a scalar register.
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
__device__ __forceinline__ uint32_t sload_u32(const void* p) { return *(const_u32_ptr)p; }
// Logit v of a row: the aligned dword that holds it (bf16: a 4-byte aligned
// pair, never past the allocation's rounded-up end), then the right half.
template <bool BF16>
__device__ __forceinline__ float sload_logit(const void* row, int v) {
  if constexpr (BF16) {
    const uintptr_t a = (uintptr_t)((const uint16_t*)row + v);
    const uint32_t w = sload_u32((const void*)(a & ~(uintptr_t)3));
    return __uint_as_float((a & 2) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(sload_u32((const float*)row + v));
  }
}

// Logit rows of request b, position i, in either layout.  The packed row
// of target position i is row_offsets[b] + b + i (L_b + 1 rows per request),
// of draft position i row_offsets[b] + i; row_offsets is the pack kernel's
// prefix sum of the clamped verify lengths.
// (n >= 0: the caller already knows the packed draft row n = row_offsets[b] + i.)
__device__ __forceinline__ size_t target_row_index(const KParams& P, int b, int i, int n = -1) {
  if (P.packed) return n >= 0 ? (size_t)n + b : (size_t)(int)sload_u32(P.row_offsets + b) + b + i;
  return (size_t)b * (P.k + 1) + i;
}
__device__ __forceinline__ size_t draft_row_index(const KParams& P, int b, int i, int n = -1) {
  if (P.packed) return n >= 0 ? (size_t)n : (size_t)(int)sload_u32(P.row_offsets + b) + i;
  return (size_t)b * P.k + i;
}
template <bool BF16>
__device__ __forceinline__ const void* target_row_ptr(const KParams& P, int b, int i, int n = -1) {
  const size_t row = target_row_index(P, b, i, n);
  return BF16 ? (const void*)((const uint16_t*)P.target + row * P.V) : (const void*)((const float*)P.target + row * P.V);
}
template <bool BF16>
__device__ __forceinline__ const void* draft_row_ptr(const KParams& P, int b, int i, int n = -1) {
  const size_t row = draft_row_index(P, b, i, n);
  return BF16 ? (const void*)((const uint16_t*)P.draft + row * P.V) : (const void*)((const float*)P.draft + row * P.V);
}

// Workgroup row slot -> row, two orders.  Compact (row_slot): slots [0, N)
// are the N draft rows in packed order (request b and position i from the
// pack kernel's row map), slots [N, N + B) the bonus rows i = L_b when the
// pass verifies, and the slots left over (the positions beyond each
// request's verify length) are idle, at the end of the grid.  Interleaved
// (row_slot_interleaved): slot s = b (k+1) + i, idle where i is beyond the
// request's rows.  Measured: the long-lived supervision workgroups run
// faster compact (no idle workgroups between rows), the short-lived
// statistics and greedy workgroups interleaved (idle ones spread out rather
// than in one tail).
struct RowSlot {
  int b, i;  // request and position; b < 0: idle slot
  int n;     // packed draft row, or -1 for a bonus row
};
__device__ __forceinline__ RowSlot row_slot(const KParams& P, int s, bool bonus) {
  const int nk = P.B * P.k;
  // (both loads issued together; the map index is clamped into the map)
  const int N = (int)sload_u32(P.Lc + P.B);
  const int m = (int)sload_u32(P.rowmap + (s < nk ? s : nk - 1));
  RowSlot o;
  o.n = -1;
  if (s < N) {
    o.b = m >> 6;
    o.i = m & 63;
    o.n = s;
  } else if (bonus && s - N < P.B) {
    o.b = s - N;
    o.i = (int)sload_u32(P.Lc + o.b);
    if (o.i < 0) o.b = -1;  // unusable packed rows
  } else {
    o.b = -1;
    o.i = 0;
  }
  return o;
}
// L_b = verify_len[b] clamped to [1, k] (k when verify_len is NULL).
__device__ __forceinline__ int clamp_len(const KParams& P, int b) {
  const int L = P.verify_len ? (int)sload_u32(P.verify_len + b) : P.k;
  return L < 1 ? 1 : (L > P.k ? P.k : L);
}

__device__ __forceinline__ RowSlot row_slot_interleaved(const KParams& P, int s, bool bonus) {
  RowSlot o;
  o.b = s / (P.k + 1);
  o.i = s - o.b * (P.k + 1);
  // (padded rows, located by (b, i); packed rows through the row offsets)
  const int L = P.pack_here ? clamp_len(P, o.b) : (int)sload_u32(P.Lc + o.b);
  const int off = P.pack_here ? 0 : (int)sload_u32(P.row_offsets + o.b);
  o.n = o.i < L ? off + o.i : -1;
  if (L < 0 || o.i > L || (!bonus && o.i == L)) o.b = -1;
  return o;
}

// Slot s = b k + i of the draft positions alone (no bonus rows).
__device__ __forceinline__ RowSlot row_slot_draft(const KParams& P, int s) {
  RowSlot o;
  o.b = s / P.k;
  o.i = s - o.b * P.k;
  const int L = P.pack_here ? clamp_len(P, o.b) : (int)sload_u32(P.Lc + o.b);
  const int off = P.pack_here ? 0 : (int)sload_u32(P.row_offsets + o.b);
  o.n = o.i < L ? off + o.i : -1;
  if (L < 0 || o.i >= L) o.b = -1;
  return o;
}

// Two values rounded to bf16 (nearest even) and packed: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Two values rounded to fp16 (nearest even) and packed: one v_cvt_pk_f16_f32.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}
// z_q - z_p of the eight bf16 entries in four packed words of each row: a
// byte permute puts the two rows' halves side by side and a bf16 dot product
// with (1, -1) subtracts them (the products are exact).  The three-operand
// dot form with a zero addend is written out (the compiler otherwise picks
// the accumulating form plus a move).  The compiler does not see the hazards
// of an asm block: a dot result may be read by another VALU instruction only
// three wait states after it is written, hence the closing s_nop; the opening
// one keeps two wait states after the permutes.
__device__ __forceinline__ void bf16_diff8(const uint32_t* wq, const uint32_t* wp, float (&dz)[8]) {
  uint32_t pr[8];
#pragma unroll
  for (int h = 0; h < 8; ++h)
    pr[h] = __builtin_amdgcn_perm(wp[h >> 1], wq[h >> 1], (h & 1) ? 0x07060302u : 0x05040100u);
  asm volatile(
      "s_nop 1\n\t"
      "v_dot2_f32_bf16 %0, %8, %16, 0\n\t"
      "v_dot2_f32_bf16 %1, %9, %16, 0\n\t"
      "v_dot2_f32_bf16 %2, %10, %16, 0\n\t"
      "v_dot2_f32_bf16 %3, %11, %16, 0\n\t"
      "v_dot2_f32_bf16 %4, %12, %16, 0\n\t"
      "v_dot2_f32_bf16 %5, %13, %16, 0\n\t"
      "v_dot2_f32_bf16 %6, %14, %16, 0\n\t"
      "v_dot2_f32_bf16 %7, %15, %16, 0\n\t"
      "s_nop 2"
      : "=&v"(dz[0]), "=&v"(dz[1]), "=&v"(dz[2]), "=&v"(dz[3]), "=&v"(dz[4]), "=&v"(dz[5]), "=&v"(dz[6]),
        "=&v"(dz[7])
      : "v"(pr[0]), "v"(pr[1]), "v"(pr[2]), "v"(pr[3]), "v"(pr[4]), "v"(pr[5]), "v"(pr[6]), "v"(pr[7]),
        "s"(0xbf803f80u));  // bf16 pair (1, -1)
}

// Half h (0 or 1) of a packed fp16 pair times y, plus z: one v_fma_mix_f32.
__device__ __forceinline__ float fma_f16(uint32_t w, int h, float y, float z) {
  const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
  return __builtin_fmaf(h ? (float)v.y : (float)v.x, y, z);
}

// ------------------------------------------------------------ row statistics

struct RowStats {
  float Mp, Mq;      // row maxima of z_p, z_q
  float SpT, SqT;    // sum exp2((z - M) kT)
  float Sp1, Sq1;    // sum exp2((z - M) log2 e)
  int xstar;         // lowest index of the maximum of z_p
};

// Combines the G chunk records of row r in a fixed order (identical in every
// workgroup that calls it).
template <bool NEED_T, bool NEED_1>
__device__ RowStats combine_part1(const KParams& P, int r, float kT, float* red) {
  // Thread t holds the record of chunk t (G <= kThreads).
  float4 a = make_float4(neg_inf(), __int_as_float(kIntMax), 0.f, 0.f);
  float4 c = make_float4(neg_inf(), 0.f, 0.f, 0.f);
  if ((int)threadIdx.x < P.G) {
    const float* rec = P.part1 + ((size_t)r * P.G + threadIdx.x) * kRec1;
    a = make_float4(pub_load(rec + 0), pub_load(rec + 1), NEED_T ? pub_load(rec + 2) : 0.f,
                    NEED_1 ? pub_load(rec + 3) : 0.f);
    c = make_float4(pub_load(rec + 4), NEED_T ? pub_load(rec + 5) : 0.f, NEED_1 ? pub_load(rec + 6) : 0.f, 0.f);
  }
  float m[2] = {a.x, c.x};
  const int mops[2] = {OP_MAX, OP_MAX};
  wg_reduce<2>(m, mops, red);
  const float mp = m[0], mq = m[1];
  float spT = 0.f, sqT = 0.f, sp1 = 0.f, sq1 = 0.f;
  if (a.x != neg_inf()) {
    if constexpr (NEED_T) spT = a.z * fexp2((a.x - mp) * kT);
    if constexpr (NEED_1) sp1 = a.w * fexp2((a.x - mp) * kLog2e);
  }
  if (c.x != neg_inf()) {
    if constexpr (NEED_T) sqT = c.y * fexp2((c.x - mq) * kT);
    if constexpr (NEED_1) sq1 = c.z * fexp2((c.x - mq) * kLog2e);
  }
  const int xi = (a.x == mp) ? __float_as_int(a.y) : kIntMax;
  float v[5] = {spT, sqT, sp1, sq1, __int_as_float(xi)};
  const int ops[5] = {OP_SUM, OP_SUM, OP_SUM, OP_SUM, OP_MINI};
  wg_reduce<5>(v, ops, red);
  RowStats s;
  s.Mp = mp;
  s.Mq = mq;
  s.SpT = v[0];
  s.SqT = v[1];
  s.Sp1 = v[2];
  s.Sq1 = v[3];
  s.xstar = __float_as_int(v[4]);
  return s;
}

// ----------------------------------------------------------------- finaliser

struct FinShared {
  float red[kWaves * 8];
  float f[16];
  int i[8];
  float slot[kWaves][kElems / 4];   // per-wave slot totals of the in-chunk scan
  unsigned long long amax[72];      // greedy: per-row (value, index) argmax keys
};

// Shared scratch of the supervision kernel for bf16 rows: reductions and the
// row values handed between waves.
struct SupShared {
  float red[kWaves * 8];
  float f[16];
  int i[8];
};

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_scan_incl(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Order-preserving unsigned key of a float for 64-bit (value, index) maxima.
__device__ __forceinline__ unsigned int ukey(float x) {
  const unsigned int u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Draws the correction or bonus token for request b.  Runs on one workgroup.
// LOG2REC: the records of the bf16 supervision kernel (64-bit tagged fields,
// sums relative to powers of two with the exponents in fields 1 and 4, at
// T = 1); otherwise float records relative to the chunk maxima rec[0] and
// rec[4] of z / T.  (Both are complete here: the finaliser runs after the
// kernel that wrote them.)
// What the residual kernel already knows when its last workgroup of a
// request draws: the first rejection A and, for A < L, row A's statistics at
// T (natural-unit maxima, sums relative to them), and the call epoch that
// tags the residual partials.
struct KnownRow {
  int A = 0;
  uint32_t ep = 0;
  float Mp = 0.f, SpT = 0.f, Mq = 0.f, SqT = 0.f;
};

template <bool BF16, bool ALIGNED, int VMODE, bool LOG2REC = false, bool KNOWN = false>
__device__ void finalize_request(const KParams& P, int b, FinShared& fs, const KnownRow& kr = KnownRow{}) {
  static_assert(!KNOWN || (VMODE == 2 && !LOG2REC), "known rows: sampled verification, natural-unit records");
  const int k = P.k, V = P.V, G = P.G;
  const int tid = threadIdx.x;  // (k + 1 <= 65 rows: thread i holds position i)
  const int lane = tid & 63;
  const int r0 = b * (k + 1);   // row slot of position 0
  // Reads that do not depend on the verify length are issued with it: the
  // clamped draft token of position tid and (sampled) the accept flag of
  // position `lane` in every wave, and the uniform of the draw.
  int tok = 0;
  float acc_flag = 1.f, us = 0.f;
  if (tid < k) {
    const int x = P.tokens[(size_t)b * k + tid];
    tok = x < 0 ? 0 : (x >= V ? V - 1 : x);
  }
  if constexpr (VMODE != 1) {
    if (!KNOWN && lane < k) acc_flag = pub_load(P.rowrec + (size_t)(r0 + lane) * kRowRec + 1);
    us = P.uniforms[(size_t)b * (k + 1) + k];
  }
  const int L = P.Lc[b];
  if (L < 0) return;  // packed rows unusable (see pack_kernel)
  int A = L, token = 0;
  float sample_margin = __int_as_float(0x7fc00000);

  if constexpr (VMODE == 1) {
    // Greedy: the argmax of every row slot from its chunk records, all rows
    // at once (largest maximum, then lowest index, as one 64-bit key; slots
    // past row L hold stale records and are not used), then the first
    // position whose draft token differs from its row's argmax.
    const int nrows = L + 1;
    for (int i = tid; i <= k; i += kThreads) fs.amax[i] = 0ull;
    __syncthreads();
    for (int q = tid; q < (k + 1) * G; q += kThreads) {
      const int i = q / G, j = q - i * G;
      const float* rec = P.part1 + ((size_t)(r0 + i) * G + j) * kRec1;
      const float m = pub_load(rec + 0);
      const unsigned int idx = (unsigned int)__float_as_int(pub_load(rec + 1));
      const unsigned long long key = ((unsigned long long)ukey(m) << 32) | (0xffffffffu - idx);
      atomicMax(&fs.amax[i], key);
    }
    __syncthreads();
    int mism = kIntMax;
    int bad = 0;
    if (tid < nrows) {
      const int i = tid;
      int am = (int)(0xffffffffu - (unsigned int)(fs.amax[i] & 0xffffffffull));
      if (am == kIntMax || am < 0 || am >= V) {  // NaN row: no chunk holds the maximum
        am = 0;
        bad = 1;
      }
      if (i < L && tok != am) mism = min(mism, i);
      fs.amax[i] = (unsigned long long)am;  // now the row's argmax
    }
    float v[2] = {__int_as_float(mism), __int_as_float(bad)};
    const int ops[2] = {OP_MINI, OP_MAXI};
    wg_reduce<2>(v, ops, fs.red);
    if (tid == 0 && __float_as_int(v[1])) flag(P.status, ADAFLASH_FLAG_NONFINITE);
    A = __float_as_int(v[0]) < L ? __float_as_int(v[0]) : L;
    token = (int)fs.amax[A];
  } else {
    // Sampled.  Every wave finds the first rejected row, the statistics of
    // the row the draw reads and the chunk of the draw by itself, from k <= 64
    // accept flags (one per lane) and G <= 128 chunk records (up to two per
    // lane), in the same fixed order in every wave: no workgroup barrier
    // separates these steps, and all threads hold the same results.
    float res[2] = {0.f, 0.f}, pj[2] = {0.f, 0.f};
    float Mp, Mq, SpT, SqT, Zres;
    bool resid;
    if constexpr (KNOWN) {
      // The residual partials of row A (waiting for this call's tags), then
      // the known statistics; a bonus draw waits for the bonus row's chunk
      // statistics, and a zero residual reads row A's target records.
      A = kr.A;
      const int rs = r0 + A;
      bool ok = true;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v1[1] = {0.f};
        const int jj = lane + 64 * h;
        if (h == 0 || G > 64)
          ok = poll_fields<1>(P.part2, kRec2, A < L && jj < G, rs * G + jj, 2, 1, kr.ep, v1, P.status) && ok;
        res[h] = A < L && jj < G ? v1[0] : 0.f;
      }
      Zres = wave_reduce<OP_SUM>(res[0] + res[1]);
      resid = A < L && Zres > 0.f;
      Mp = kr.Mp;
      SpT = kr.SpT;
      Mq = kr.Mq;
      SqT = kr.SqT;
      if (!resid) {
        // Row A's target statistics: the bonus row's from the residual
        // kernel's tagged fields, a rejected row's (zero residual) from the
        // statistics kernel's records.
        float mp[2], spT[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jj = lane + 64 * h;
          mp[h] = neg_inf();
          spT[h] = 0.f;
          if (A == L) {
            float v2[2] = {neg_inf(), 0.f};
            if (h == 0 || G > 64)
              ok = poll_fields<2>(P.part2, kRec2, jj < G, rs * G + jj, 0, 2, kr.ep, v2, P.status) && ok;
            if (jj < G) {
              mp[h] = v2[0];
              spT[h] = v2[1];
            }
          } else if (jj < G) {
            const float* rec = P.part1 + ((size_t)rs * G + jj) * kRec1;
            mp[h] = pub_load(rec + 0);
            spT[h] = pub_load(rec + 2);
          }
        }
        Mp = wave_reduce<OP_MAX>(fmaxf(mp[0], mp[1]));
#pragma unroll
        for (int h = 0; h < 2; ++h) pj[h] = mp[h] == neg_inf() ? 0.f : spT[h] * fexp2((mp[h] - Mp) * P.kT);
        SpT = wave_reduce<OP_SUM>(pj[0] + pj[1]);
        Mq = neg_inf();
        SqT = 1.f;
      }
      (void)ok;  // (a timed-out wait has flagged the status word)
    } else {
      const unsigned long long rej = __ballot(lane < L && acc_flag == 0.f);
      A = rej ? min((int)__builtin_ctzll(rej), L) : L;

      // Row statistics at T of the row the draw reads (rejected row A or the
      // bonus row L) and, for a rejected row, its per-chunk residual masses.
      const int rs = r0 + A;
      float mp[2], spT[2], mq[2], sqT[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int jj = lane + 64 * h;
        mp[h] = neg_inf();
        mq[h] = neg_inf();
        spT[h] = sqT[h] = 0.f;
        if (jj < G) {
          if constexpr (LOG2REC) {
            const size_t f0 = ((size_t)rs * G + jj) * kRec1;
            mp[h] = tag_value(tag_load(P.part1, f0 + 1));
            spT[h] = tag_value(tag_load(P.part1, f0 + 2));
            if (A < L) {
              mq[h] = tag_value(tag_load(P.part1, f0 + 4));
              sqT[h] = tag_value(tag_load(P.part1, f0 + 5));
              res[h] = tag_value(tag_load(P.part2, ((size_t)rs * G + jj) * kRec2 + 2));
            }
          } else {
            const float* rec = P.part1 + ((size_t)rs * G + jj) * kRec1;
            mp[h] = pub_load(rec + 0);
            spT[h] = pub_load(rec + 2);
            if (A < L) {
              mq[h] = pub_load(rec + 4);
              sqT[h] = pub_load(rec + 5);
              res[h] = pub_load(P.part2 + ((size_t)rs * G + jj) * kRec2 + 2);
            }
          }
        }
      }
      Mp = wave_reduce<OP_MAX>(fmaxf(mp[0], mp[1]));
      Mq = wave_reduce<OP_MAX>(fmaxf(mq[0], mq[1]));
      float qj[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (LOG2REC) {
          pj[h] = mp[h] == neg_inf() ? 0.f : __builtin_ldexpf(spT[h], (int)fmaxf(mp[h] - Mp, -256.f));
          qj[h] = mq[h] == neg_inf() ? 0.f : __builtin_ldexpf(sqT[h], (int)fmaxf(mq[h] - Mq, -256.f));
        } else {
          pj[h] = mp[h] == neg_inf() ? 0.f : spT[h] * fexp2((mp[h] - Mp) * P.kT);
          qj[h] = mq[h] == neg_inf() ? 0.f : sqT[h] * fexp2((mq[h] - Mq) * P.kT);
        }
      }
      SpT = wave_reduce<OP_SUM>(pj[0] + pj[1]);
      SqT = wave_reduce<OP_SUM>(qj[0] + qj[1]);
      Zres = wave_reduce<OP_SUM>(res[0] + res[1]);
      resid = A < L && Zres > 0.f;
    }
    const float invSp = 1.f / SpT, invSq = 1.f / SqT;

    // Chunk-level inverse CDF over the chunk masses in chunk order: the first
    // chunk whose running mass passes u_s times the total, else the last
    // chunk with positive mass, else chunk 0.
    float mj[2], ex[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) mj[h] = lane + 64 * h < G ? (resid ? res[h] : pj[h] * invSp) : 0.f;
    const float inc0 = wave_scan_incl(mj[0]);
    const float tot0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc0), 63));
    const float inc1 = tot0 + wave_scan_incl(mj[1]);
    const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc1), 63));
    ex[0] = __shfl_up(inc0, 1, 64);
    ex[1] = __shfl_up(inc1, 1, 64);
    if (lane == 0) {
      ex[0] = 0.f;
      ex[1] = tot0;
    }
    const float thr = us * tot;
    const unsigned long long c0 = __ballot(lane < G && ex[0] + mj[0] > thr);
    const unsigned long long c1 = __ballot(lane + 64 < G && ex[1] + mj[1] > thr);
    const unsigned long long q0 = __ballot(lane < G && mj[0] > 0.f);
    const unsigned long long q1 = __ballot(lane + 64 < G && mj[1] > 0.f);
    int jc = 0;
    if (c0) jc = (int)__builtin_ctzll(c0);
    else if (c1) jc = 64 + (int)__builtin_ctzll(c1);
    else if (q1) jc = 127 - (int)__builtin_clzll(q1);
    else if (q0) jc = 63 - (int)__builtin_clzll(q0);
    const float base = __shfl(jc < 64 ? ex[0] : ex[1], jc & 63, 64);

    // Scan chunk jc in index order: per-entry masses, one prefix sum over
    // (slot, thread, entry), the lowest index with positive mass whose
    // running sum passes thr (a thread's start, taken from the prefix sum,
    // can pass thr by rounding alone: a zero-mass entry is never drawn).
    const void* trow = target_row_ptr<BF16>(P, b, A);
    const void* drow = draft_row_ptr<BF16>(P, b, A);
    const int v0 = jc * kChunk;
    Chunk<BF16> cp, cq;
    load_chunk<BF16, ALIGNED>(cp, trow, v0, V);
    if (resid) load_chunk<BF16, ALIGNED>(cq, drow, v0, V);
    const float ap = LOG2REC ? -Mp : -Mp * P.kT, aq = LOG2REC ? -Mq : -Mq * P.kT;
    constexpr int VEC = Chunk<BF16>::VEC;
    constexpr int NV = kElems / VEC;
    const int wave = tid >> 6;
    float w[kElems];
    float incl[NV], tsum[NV];
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2) {
      float ts = 0.f;
#pragma unroll
      for (int u = 0; u < VEC; ++u) {
        const int e = s2 * VEC + u;
        const float zp = cp.get(e);
        float mass;
        if (resid) {
          const float pv = mul_rn(fexp2(fmaf(zp, P.kT, ap)), invSp);
          const float qv = mul_rn(fexp2(fmaf(cq.get(e), P.kT, aq)), invSq);
          mass = fmaxf(0.f, pv - qv);
        } else {
          mass = zp == neg_inf() ? 0.f : fexp2(fmaf(zp, P.kT, ap)) * invSp;
        }
        w[e] = entry_index<BF16>(v0, e) < V ? mass : 0.f;
        ts += w[e];
      }
      tsum[s2] = ts;
      incl[s2] = wave_scan_incl(ts);
      if (lane == 63) fs.slot[wave][s2] = incl[s2];
    }
    __syncthreads();
    float run = base;  // running sum before this thread's first entry of the slot
    int found = kIntMax, last_pos = -1;
    float found_before = 0.f, found_at = 0.f, last_before = 0.f, last_at = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2) {
      float woff = 0.f, stot = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const float t = fs.slot[w2][s2];
        if (w2 < wave) woff += t;
        stot += t;
      }
      float cum = run + woff + (incl[s2] - tsum[s2]);
#pragma unroll
      for (int u = 0; u < VEC; ++u) {
        const int e = s2 * VEC + u;
        const int idx = entry_index<BF16>(v0, e);
        const float before = cum;
        cum += w[e];
        if (w[e] > 0.f) {  // (entries past V have no mass)
          last_pos = idx;
          last_before = before;
          last_at = cum;
          if (found == kIntMax && cum > thr) {
            found = idx;
            found_before = before;
            found_at = cum;
          }
        }
      }
      run += stot;
    }
    // Winner: the lowest crossing index, else the last positive-mass entry.
    float v2[2] = {__int_as_float(found), __int_as_float(last_pos < 0 ? kIntMax : -last_pos)};
    const int o2[2] = {OP_MINI, OP_MINI};
    wg_reduce<2>(v2, o2, fs.red);
    const int fmin = __float_as_int(v2[0]);
    const int lmax = __float_as_int(v2[1]) == kIntMax ? -1 : -__float_as_int(v2[1]);
    if (tid == 0) {
      fs.f[5] = base;
      fs.f[6] = base;
    }
    __syncthreads();
    if (fmin != kIntMax) {
      token = fmin;
      if (found == fmin) {
        fs.f[5] = found_before;
        fs.f[6] = found_at;
      }
    } else {
      token = lmax >= 0 ? lmax : v0;
      if (lmax >= 0 && last_pos == lmax) {
        fs.f[5] = last_before;
        fs.f[6] = last_at;
      }
    }
    __syncthreads();
    const float cb = fs.f[5], ca = fs.f[6];
    sample_margin = fminf(thr - cb, ca - thr) / tot;
    __syncthreads();
  }

  // Outputs.
  if (tid <= k) {
    const int i = tid;
    int32_t t = -1;
    if (i < A) t = tok;
    else if (i == A) t = token;
    P.out_tokens[(size_t)b * (k + 1) + i] = t;
    if (P.margins) {
      if (i == k) P.margins[(size_t)b * (k + 1) + k] = sample_margin;
      else if (VMODE == 1 || i >= L) P.margins[(size_t)b * (k + 1) + i] = __int_as_float(0x7fc00000);
    }
  }
  if (tid == 0) P.accept_len[b] = A;
}

// ---------------------------------------------------------------- row kernel

template <bool BF16, bool ALIGNED, bool OPD, int VMODE, bool T1>
__global__ __launch_bounds__(kThreads) void row_kernel(KParams P) {
  constexpr bool SAMPLED = VMODE == 2, GREEDY = VMODE == 1, VERIFY = VMODE != 0;
  constexpr int VEC = Chunk<BF16>::VEC;
  __shared__ FinShared fs;
  __shared__ int sh_ok;

  const int tid = threadIdx.x;
  const int G = P.G;
  const int k = P.k, V = P.V;
  // Workgroup -> (row slot, chunk j) -> (request b, position i); workspace
  // slot r = b*(k+1) + i.
  const int s_ = (int)blockIdx.x / G;
  const int j = (int)blockIdx.x - s_ * G;
  const RowSlot sl = row_slot_interleaved(P, s_, VERIFY);
  if (sl.b < 0) return;
  const int b = sl.b, i = sl.i;
  const int r = b * (k + 1) + i;
  const bool draft_row = sl.n >= 0;
  const bool need_q = draft_row && (OPD || SAMPLED);
  const int v0 = j * kChunk;

  const void* trow = target_row_ptr<BF16>(P, b, i, sl.n);
  const void* drow = nullptr;
  if (need_q)
    drow = draft_row_ptr<BF16>(P, b, i, sl.n);

  // ---- phase 1: load the chunk, chunk maxima, argmax, sums of exponentials.
  Chunk<BF16> cp, cq;
  load_chunk<BF16, ALIGNED>(cp, trow, v0, V);
  if (need_q) load_chunk<BF16, ALIGNED>(cq, drow, v0, V);

  float mp = chunk_max<BF16>(cp), mq = neg_inf();
  if (need_q) mq = chunk_max<BF16>(cq);
  cp.opaque();
  cq.opaque();
  {
    float v[2] = {mp, mq};
    const int ops[2] = {OP_MAX, OP_MAX};
    const float mp_t = mp;
    wg_reduce<2>(v, ops, fs.red);
    // Lowest index holding the chunk maximum of z_p (only lanes that hold it search).
    int cand = kIntMax;
    if (mp_t == v[0]) {
#pragma unroll
      for (int e = kElems - 1; e >= 0; --e)
        if (cp.get(e) == v[0]) cand = entry_index<BF16>(v0, e);
    }
    mp = v[0];
    mq = v[1];
    float spT = 0.f, sqT = 0.f, sp1 = 0.f, sq1 = 0.f;
    const float Mp = mp, Mq = mq;
    if constexpr (SAMPLED) {
      const float ap = Mp == neg_inf() ? 0.f : -Mp * P.kT;
#pragma unroll
      for (int e = 0; e < kElems; ++e) spT += fexp2(fmaf(cp.get(e), P.kT, ap));
      if (need_q) {
        const float aq = Mq == neg_inf() ? 0.f : -Mq * P.kT;
#pragma unroll
        for (int e = 0; e < kElems; ++e) sqT += fexp2(fmaf(cq.get(e), P.kT, aq));
      }
    }
    if constexpr (OPD) {
      if (draft_row) {
        if constexpr (SAMPLED && T1) {
          sp1 = spT;
          sq1 = sqT;
        } else {
          const float ap = Mp == neg_inf() ? 0.f : -Mp * kLog2e;
          const float aq = Mq == neg_inf() ? 0.f : -Mq * kLog2e;
#pragma unroll
          for (int e = 0; e < kElems; ++e) {
            sp1 += fexp2(fmaf(cp.get(e), kLog2e, ap));
            sq1 += fexp2(fmaf(cq.get(e), kLog2e, aq));
          }
        }
      }
    }
    float s[5] = {spT, sqT, sp1, sq1, __int_as_float(cand)};
    const int sops[5] = {OP_SUM, OP_SUM, OP_SUM, OP_SUM, OP_MINI};
    wg_reduce<5>(s, sops, fs.red);
    if (tid == 0) {
      float* rec = P.part1 + ((size_t)r * G + j) * kRec1;
      pub_store(rec + 0, Mp);
      pub_store(rec + 1, s[4]);
      pub_store(rec + 2, s[0]);
      pub_store(rec + 3, s[2]);
      pub_store(rec + 4, Mq);
      pub_store(rec + 5, s[1]);
      pub_store(rec + 6, s[3]);
    }
  }

  const bool do_rows = draft_row && (SAMPLED || OPD);
  bool alive = true;
  if (do_rows) {
    // ---- barrier 1: all chunks of this row have published their statistics.
    alive = arrive_and_wait(&P.rowcnt[(size_t)r * kCounterStride], G, P.status, &sh_ok);
    if (alive) {
      const RowStats st = combine_part1<SAMPLED, OPD && !(SAMPLED && T1)>(P, r, P.kT, fs.red);
      float Sp1 = st.Sp1, Sq1 = st.Sq1;
      if constexpr (SAMPLED && T1) {
        Sp1 = st.SpT;
        Sq1 = st.SqT;
      }
      if (tid == 0) {
        const bool bad = !(st.Mp < __builtin_inff()) || !(st.SpT > 0.f || !SAMPLED);
        if (bad) flag(P.status, ADAFLASH_FLAG_NONFINITE);
      }
      // Accept test for this row (sampled mode).
      bool accept = true;
      if constexpr (SAMPLED) {
        int x = P.tokens[(size_t)b * k + i];
        if (x < 0 || x >= V) {
          if (tid == 0 && j == 0) flag(P.status, ADAFLASH_FLAG_BAD_TOKEN);
          x = x < 0 ? 0 : V - 1;
        }
        const float zpx = load_logit<BF16>(trow, x), zqx = load_logit<BF16>(drow, x);
        const float px = fexp2((zpx - st.Mp) * P.kT) / st.SpT;
        const float qx = fexp2((zqx - st.Mq) * P.kT) / st.SqT;
        const float u = P.uniforms[(size_t)b * (k + 1) + i];
        accept = u * qx < px;
        if (tid == 0 && j == 0) {
          pub_store(P.rowrec + (size_t)r * kRowRec + 1, accept ? 1.f : 0.f);
          pub_store(P.rowrec + (size_t)r * kRowRec + 2, px - u * qx);
          if (P.margins) P.margins[(size_t)b * (k + 1) + i] = px - u * qx;
        }
      }

      // ---- phase 2: supervision sums and/or the residual mass of this chunk.
      cp.opaque();
      cq.opaque();
      float Spart = 0.f, Rpart = 0.f, Zpart = 0.f;
      float gc[kElems];
      float qv[kElems];
      const float lse_q2 = st.Mq * kLog2e + flog2(Sq1);  // log2-domain normalisers
      const float lse_p2 = st.Mp * kLog2e + flog2(Sp1);
      const float D = (lse_q2 - lse_p2) * kLn2;          // lse_q - lse_p
      if constexpr (OPD) {
        const float c = P.clip_c, lam = P.lambda;
        const float nq = -lse_q2;
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
          const float zq = cq.get(e), zp = cp.get(e);
          const float q = fexp2(fmaf(zq, kLog2e, nq));
          const float d = (zq - zp) - D;
          const float f = q > 0.f ? q * d : 0.f;
          const bool inU = f <= c;
          Rpart += inU ? f : c;
          const float sterm = inU ? f + q : 0.f;
          Spart += sterm;
          gc[e] = fmaf(lam, sterm, q);
          qv[e] = q;
        }
      }
      if constexpr (SAMPLED) {
        if (!accept) {
          const float invSp = 1.f / st.SpT, invSq = 1.f / st.SqT;
          const float ap = -st.Mp * P.kT, aq = -st.Mq * P.kT;
#pragma unroll
          for (int e = 0; e < kElems; ++e) {
            const float pv = mul_rn(fexp2(fmaf(cp.get(e), P.kT, ap)), invSp);
            const float qq = mul_rn(fexp2(fmaf(cq.get(e), P.kT, aq)), invSq);
            Zpart += fmaxf(0.f, pv - qq);
          }
        }
      }
      {
        float s[3] = {Spart, Rpart, Zpart};
        const int ops[3] = {OP_SUM, OP_SUM, OP_SUM};
        wg_reduce<3>(s, ops, fs.red);
        if (tid == 0) {
          float* rec = P.part2 + ((size_t)r * G + j) * kRec2;
          pub_store(rec + 0, s[0]);
          pub_store(rec + 1, s[1]);
          pub_store(rec + 2, s[2]);
        }
      }

      if constexpr (OPD) {
        // ---- barrier 2: supervision sums of every chunk are published.
        alive = arrive_and_wait(&P.rowcnt[(size_t)r * kCounterStride], 2 * G, P.status, &sh_ok);
        if (alive) {
          float sr[2] = {0.f, 0.f};
          if (tid < G) {
            const float* rec = P.part2 + ((size_t)r * G + tid) * kRec2;
            sr[0] = pub_load(rec + 0);
            sr[1] = pub_load(rec + 1);
          }
          const int srops[2] = {OP_SUM, OP_SUM};
          wg_reduce<2>(sr, srops, fs.red);
          const float S = sr[0], R = sr[1];
          const int n = sl.n;  // packed row
          const float lamS = P.lambda * S;
          // x* correction: only the thread holding x* takes this branch.
          const int xs = st.xstar;
          const int xo = xs - v0;
          const bool xs_here = xo >= 0 && xo < kChunk && ((xo % (kThreads * VEC)) / VEC) == tid;
          if (xs_here) {
            const int es = (xo / (kThreads * VEC)) * VEC + (xo % VEC);
#pragma unroll
            for (int e = 0; e < kElems; ++e)
              if (e == es) gc[e] -= 1.f;
          }
          if (P.grad) {
            constexpr int NV = kElems / VEC;
#pragma unroll
            for (int s2 = 0; s2 < NV; ++s2) {
              const int idx0 = v0 + s2 * (kThreads * VEC) + tid * VEC;
              float g[VEC];
#pragma unroll
              for (int u = 0; u < VEC; ++u) g[u] = fmaf(-lamS, qv[s2 * VEC + u], gc[s2 * VEC + u]);
              if constexpr (BF16) {
                uint16_t* gr = (uint16_t*)P.grad + (size_t)n * V;
                if constexpr (ALIGNED) {
                  if (idx0 < V) {
                    uint4 o;
                    o.x = pack_bf16x2(g[0], g[1]);
                    o.y = pack_bf16x2(g[2], g[3]);
                    o.z = pack_bf16x2(g[4], g[5]);
                    o.w = pack_bf16x2(g[6], g[7]);
                    *(uint4*)(gr + idx0) = o;
                  }
                } else {
#pragma unroll
                  for (int u = 0; u < VEC; ++u)
                    if (idx0 + u < V) gr[idx0 + u] = __builtin_bit_cast(uint16_t, (__bf16)g[u]);
                }
              } else {
                float* gr = (float*)P.grad + (size_t)n * V;
                if constexpr (ALIGNED) {
                  if (idx0 < V) *(float4*)(gr + idx0) = make_float4(g[0], g[1], g[2], g[3]);
                } else {
#pragma unroll
                  for (int u = 0; u < VEC; ++u)
                    if (idx0 + u < V) gr[idx0 + u] = g[u];
                }
              }
            }
          }
          // Losses: written by the chunk that holds x*.
          if (tid == 0 && xs >= v0 && xs < v0 + kChunk) {
            const float zqx = load_logit<BF16>(drow, xs);
            if (P.loss_ce) P.loss_ce[n] = (lse_q2 * kLn2) - zqx;
            if (P.loss_rkl) P.loss_rkl[n] = R;
          }
        }
      }
    }
  }

  (void)alive;
  (void)GREEDY;
}

// ----------------------------------------------- supervision kernel (T = 1)
//
// Supervision at temperature 1, alone or fused with greedy verification or
// with sampled verification at T = 1.  Pass 1 publishes per chunk the maxima,
// the sums of exponentials, W = sum e dz and A = max e dz, where
// e = exp(z_q - m) (m: this chunk's maximum of z_q) and dz = z_q - z_p.  After
// the row barrier every chunk derives lse_q, lse_p, D = lse_q - lse_p, the
// unclipped KL = sum_v q_v dz_v - D, and a bound on every entry's term
// f_v = q_v (dz_v - D):
//   f_v <= exp(m_j - lse_q) (A_j + max(0, -D)) <= (max_j e^{m_j - M} A_j + max(0, -D)) / S_q,
// using e_v <= 1 (M: row maximum of z_q, S_q = sum_v exp(z_q - M)).
// When the bound is below c no entry is clipped, so R = KL and S = KL + 1,
// and each chunk writes its gradient at once:
//   g_v = q_v (1 + lambda (d_v - KL)) - [v == x*],  d_v = dz_v - D.
// Otherwise (or when a row holds -inf or non-finite logits) the exact path
// accumulates R and S per chunk and meets the row at a second barrier.
// Only the packed logits stay in registers between passes; q and dz are
// recomputed (the kernel is bound by bytes in flight, so registers are worth
// more than the extra arithmetic).

struct SupStats {
  float Mp, Mq, Sp, Sq, Wsum, BA;
  int xstar;     // lowest index of the row maximum of z_p, or (chunk-level
                 // records) the lowest chunk holding it
  int nonfinite;
  float margin;  // p(x) - u q(x) of the accept test (sampled verification)
  // Derived row values: log2 normalisers of q and p, D = lse_q - lse_p, the
  // unclipped reverse KL, and the bound on the largest per-entry term.
  float lse_q2, lse_p2, D, KL, bound;
  float fkl;  // forward KL(p || q) of the row (forward-KL variant only)
  int alive;  // the row's records arrived (bf16 supervision kernel; 0: the wait hit its bound)
};

__device__ __forceinline__ void derive_sup(float Mp, float Mq, float Sp, float Sq, float Wsum, float BA,
                                           float (&d)[5]) {
  const float lq = Mq * kLog2e + flog2(Sq);
  const float lp = Mp * kLog2e + flog2(Sp);
  const float D = (lq - lp) * kLn2;
  d[0] = lq;
  d[1] = lp;
  d[2] = D;
  d[3] = Wsum / Sq - D;
  d[4] = (BA + fmaxf(0.f, -D)) / Sq;
}

// Accept test of sampled verification at T = 1: u q(x) < p(x).
__device__ __forceinline__ float accept_margin(float zpx, float zqx, float u, float Mp, float Mq, float Sp,
                                              float Sq) {
  const float px = fexp2((zpx - Mp) * kLog2e) * __builtin_amdgcn_rcpf(Sp);
  const float qx = fexp2((zqx - Mq) * kLog2e) * __builtin_amdgcn_rcpf(Sq);
  return px - u * qx;
}

// Combines the G chunk records of row r (identical in every workgroup of the
// row).  With G <= 64 wave 0 alone reduces them (lane j holds chunk j) and
// hands the results to the other waves through fs.f; otherwise every wave
// takes part.  CHUNK_X: the records carry no argmax; xstar is then the lowest
// chunk whose maximum is the row maximum.
template <bool SAMPLED, bool CHUNK_X, bool FKL, typename SH>
__device__ SupStats combine_sup(const KParams& P, int r, SH& fs, float zpx, float zqx, float u) {
  const int tid = threadIdx.x;
  const int G = P.G;
  auto reduce = [&](float mp, float mq, float sp, float sq, float w, float a, int idx, bool valid,
                    float (&m)[2], float (&v)[6], bool whole_group) {
    if (whole_group) {
      m[0] = mp;
      m[1] = mq;
      const int mops[2] = {OP_MAX, OP_MAX};
      wg_reduce<2>(m, mops, fs.red);
    } else {
      m[0] = wave_reduce<OP_MAX>(mp);
      m[1] = wave_reduce<OP_MAX>(mq);
    }
    const float fp = mp == neg_inf() ? 0.f : fexp2((mp - m[0]) * kLog2e);
    const float fq = mq == neg_inf() ? 0.f : fexp2((mq - m[1]) * kLog2e);
    const bool fin = !valid || (__builtin_isfinite(w) && !__builtin_isnan(a) && a < __builtin_inff());
    v[0] = sp * fp;
    v[1] = sq * fq;
    v[2] = fq > 0.f ? w * fq : 0.f;
    v[3] = fq > 0.f ? fq * a : neg_inf();
    v[4] = __int_as_float(mp == m[0] ? idx : kIntMax);
    v[5] = __int_as_float(fin ? 0 : 1);
    if (whole_group) {
      const int ops[6] = {OP_SUM, OP_SUM, OP_SUM, OP_MAX, OP_MINI, OP_MAXI};
      wg_reduce<6>(v, ops, fs.red);
    } else {
      v[0] = wave_reduce<OP_SUM>(v[0]);
      v[1] = wave_reduce<OP_SUM>(v[1]);
      v[2] = wave_reduce<OP_SUM>(v[2]);
      v[3] = wave_reduce<OP_MAX>(v[3]);
      v[4] = wave_reduce<OP_MINI>(v[4]);
      v[5] = wave_reduce<OP_MAXI>(v[5]);
    }
  };
  auto load = [&](int c, float& mp, float& mq, float& sp, float& sq, float& w, float& a, int& idx) {
    const float* rec = P.part1 + ((size_t)r * G + c) * kRec1;
    mp = pub_load(rec + 0);
    idx = CHUNK_X ? c : __float_as_int(pub_load(rec + 1));
    sp = pub_load(rec + 2);
    w = pub_load(rec + 3);
    mq = pub_load(rec + 4);
    sq = pub_load(rec + 5);
    a = pub_load(rec + 6);
  };
  float m[2], v[6], dv[5], wpr = 0.f;
  if (G <= 64) {
    if (tid < 64) {
      float mp = neg_inf(), mq = neg_inf(), sp = 0.f, sq = 0.f, w = 0.f, a = neg_inf();
      int idx = kIntMax;
      if (tid < G) load(tid, mp, mq, sp, sq, w, a, idx);
      reduce(mp, mq, sp, sq, w, a, idx, tid < G, m, v, false);
      float wp = 0.f;
      if constexpr (FKL) {
        if (tid < G && mp != neg_inf())
          wp = pub_load(P.part1 + ((size_t)r * G + tid) * kRec1 + 7) * fexp2((mp - m[0]) * kLog2e);
        wp = wave_reduce<OP_SUM>(wp);
      }
      if (tid == 0) {
        fs.f[14] = wp;
        fs.f[0] = m[0];
        fs.f[1] = m[1];
#pragma unroll
        for (int q = 0; q < 6; ++q) fs.f[2 + q] = v[q];
        if (SAMPLED) fs.f[8] = accept_margin(zpx, zqx, u, m[0], m[1], v[0], v[1]);
        // The derived values once here rather than in every wave.
        float d[5];
        derive_sup(m[0], m[1], v[0], v[1], v[2], v[3], d);
#pragma unroll
        for (int q = 0; q < 5; ++q) fs.f[9 + q] = d[q];
      }
    }
    __syncthreads();
    m[0] = fs.f[0];
    m[1] = fs.f[1];
#pragma unroll
    for (int q = 0; q < 6; ++q) v[q] = fs.f[2 + q];
#pragma unroll
    for (int q = 0; q < 5; ++q) dv[q] = fs.f[9 + q];
    wpr = fs.f[14];
  } else {
    float mp = neg_inf(), mq = neg_inf(), sp = 0.f, sq = 0.f, w = 0.f, a = neg_inf();
    int idx = kIntMax;
    if (tid < G) load(tid, mp, mq, sp, sq, w, a, idx);
    reduce(mp, mq, sp, sq, w, a, idx, tid < G, m, v, true);
    if (SAMPLED && tid == 0) fs.f[8] = accept_margin(zpx, zqx, u, m[0], m[1], v[0], v[1]);
    derive_sup(m[0], m[1], v[0], v[1], v[2], v[3], dv);
    if constexpr (FKL) {
      float w1[1] = {0.f};
      if (tid < G && mp != neg_inf())
        w1[0] = pub_load(P.part1 + ((size_t)r * G + tid) * kRec1 + 7) * fexp2((mp - m[0]) * kLog2e);
      const int o1[1] = {OP_SUM};
      wg_reduce<1>(w1, o1, fs.red);
      wpr = w1[0];
    }
    __syncthreads();
  }
  SupStats s;
  s.Mp = uniform(m[0]);
  s.Mq = uniform(m[1]);
  s.Sp = uniform(v[0]);
  s.Sq = uniform(v[1]);
  s.Wsum = uniform(v[2]);
  s.BA = uniform(v[3]);
  s.xstar = __float_as_int(uniform(v[4]));
  s.nonfinite = __float_as_int(uniform(v[5])) != 0;
  s.margin = SAMPLED ? uniform(fs.f[8]) : 0.f;
  s.lse_q2 = uniform(dv[0]);
  s.lse_p2 = uniform(dv[1]);
  s.D = uniform(dv[2]);
  s.KL = uniform(dv[3]);
  s.bound = uniform(dv[4]);
  // Forward KL = sum p (log p - log q) = -E_p[z_q - z_p] + D.
  s.fkl = FKL ? uniform(-wpr / s.Sp + s.D) : 0.f;
  return s;
}

// Power-of-two scale exponent of a block of logits with maximum m:
// ceil(m log2 e), clamped to [-2^20, 2^20] (-inf and NaN give -2^20).  Every
// exp(z - ...) of the block is taken as 2^(z log2 e - a) <= 1 (up to one
// rounding), and partial sums at different exponents merge by exact scaling
// with ldexp.  Monotone in m: the exponent of a maximum is the maximum of the
// exponents.
__device__ __forceinline__ int shift_of(float m) {
  return (int)fminf(fmaxf(__builtin_ceilf(m * kLog2e), -1048576.f), 1048576.f);
}

// Row statistics from the chunk records of the bf16 supervision kernel, whose
// sums are relative to powers of two: rec[1] = a_p and rec[4] = a_q (the
// chunk's scale exponents), rec[2] = sum 2^(z_p log2 e - a_p), rec[5] the same
// for z_q, rec[3] = W and rec[6] = A on the z_q scale, rec[7] = sum p' (z_q -
// z_p) on the z_p scale (forward KL), rec[0] = the chunk's exact maximum of
// z_p (x*: the lowest chunk holding the row maximum); every field is tagged
// with the call's epoch.  Wave 0 waits for the row's G arrivals and for the
// records (the row barrier), reduces them, chunk j in lane j (G <= 32), and
// hands the results to the other waves through fs.f; lse_q2 and lse_p2 are
// in log2 units.  EARLY: the counter wait ends with one chunk still to
// arrive, and that chunk's record is polled for with the others' loaded
// (measured faster where most rows take the exact path, slower otherwise).
template <bool SAMPLED, bool FKL, typename SH, bool EARLY = false>
__device__ SupStats combine_sup_pow2(const KParams& P, int r, SH& fs, float zpx, float zqx, float u, uint32_t ep) {
  const int tid = threadIdx.x;
  const int G = P.G;  // <= 32 (the host dispatches larger rows elsewhere)
  if (tid < 64) {
    // Lane c holds fields 0-3 of record c, lane 32 + c fields 4-7; the two
    // halves then swap, and the reductions run over lanes c < G.
    const int c = tid & 31, half = tid >> 5;
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    const float* recs = (const float*)((const uint64_t*)P.part1 + (size_t)r * G * kRec1);
    const bool ok = wait_count(P.rowcnt + (size_t)r * kCounterStride, EARLY ? G - 1 : G, P.status) &&
                    poll_fields<4>(recs, kRec1, c < G, c, 4 * half, half && !FKL ? 3 : 4, ep, h, P.status);
    float o[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) o[n] = __shfl_xor(h[n], 32, 64);
    const bool valid = half == 0 && c < G;
    const float mx = valid ? h[0] : neg_inf(), ap = h[1], sp = valid ? h[2] : 0.f, w = valid ? h[3] : 0.f;
    const float aq = o[0], sq = valid ? o[1] : 0.f, a = valid ? o[2] : neg_inf();
    const float wp = FKL && valid ? o[3] : 0.f;
    // Scale exponents are integers in [-2^20, 2^20] (float in the record).
    const int api = valid ? (int)ap : -(1 << 21), aqi = valid ? (int)aq : -(1 << 21);
    const float Mx = wave_reduce<OP_MAX>(mx);
    const int Api = __float_as_int(wave_reduce<OP_MAXI>(__int_as_float(api)));
    const int Aqi = __float_as_int(wave_reduce<OP_MAXI>(__int_as_float(aqi)));
    const float Ap = (float)Api, Aq = (float)Aqi;
    const int dp = max(api - Api, -256), dq = max(aqi - Aqi, -256);
    float v[7];
    v[0] = wave_reduce<OP_SUM>(__builtin_ldexpf(sp, dp));
    v[1] = wave_reduce<OP_SUM>(__builtin_ldexpf(sq, dq));
    v[2] = wave_reduce<OP_SUM>(__builtin_ldexpf(w, dq));
    v[3] = wave_reduce<OP_MAX>(__builtin_ldexpf(a, dq));
    v[4] = wave_reduce<OP_MINI>(__int_as_float(valid && mx == Mx ? tid : kIntMax));
    v[5] = wave_reduce<OP_MAXI>(
        __int_as_float(!valid || (__builtin_isfinite(w) && !__builtin_isnan(a) && a < __builtin_inff()) ? 0 : 1));
    v[6] = FKL ? wave_reduce<OP_SUM>(__builtin_ldexpf(wp, dp)) : 0.f;
    if (tid == 0) {
      fs.i[2] = ok;
      const float rSp = __builtin_amdgcn_rcpf(v[0]), rSq = __builtin_amdgcn_rcpf(v[1]);
      const float lq = Aq + flog2(v[1]);
      const float lp = Ap + flog2(v[0]);
      const float D = (lq - lp) * kLn2;
      fs.f[0] = Mx;
      fs.f[1] = Aq;
#pragma unroll
      for (int q = 0; q < 6; ++q) fs.f[2 + q] = v[q];
      if (SAMPLED) {
        const float px = fexp2(fmaf(zpx, kLog2e, -Ap)) * rSp;
        const float qx = fexp2(fmaf(zqx, kLog2e, -Aq)) * rSq;
        fs.f[8] = px - u * qx;
      }
      fs.f[9] = lq;
      fs.f[10] = lp;
      fs.f[11] = D;
      fs.f[12] = v[2] * rSq - D;
      fs.f[13] = (v[3] + fmaxf(0.f, -D)) * rSq;
      fs.f[14] = v[6];
    }
  }
  __syncthreads();
  SupStats s;
  s.Mp = uniform(fs.f[0]);
  s.Mq = uniform(fs.f[1]);
  s.Sp = uniform(fs.f[2]);
  s.Sq = uniform(fs.f[3]);
  s.Wsum = uniform(fs.f[4]);
  s.BA = uniform(fs.f[5]);
  s.xstar = __float_as_int(uniform(fs.f[6]));
  s.nonfinite = __float_as_int(uniform(fs.f[7])) != 0;
  s.margin = SAMPLED ? uniform(fs.f[8]) : 0.f;
  s.lse_q2 = uniform(fs.f[9]);
  s.lse_p2 = uniform(fs.f[10]);
  s.D = uniform(fs.f[11]);
  s.KL = uniform(fs.f[12]);
  s.bound = uniform(fs.f[13]);
  // Forward KL = sum p (log p - log q) = -E_p[z_q - z_p] + D.
  s.fkl = FKL ? uniform(-fs.f[14] / s.Sp + s.D) : 0.f;
  s.alive = __builtin_amdgcn_readfirstlane(fs.i[2]);
  return s;
}

// Gradient value of the exact path (q recomputed in fp32: clip decisions).
__device__ __forceinline__ float grad_exact(float zq, float zp, float lse_q2, float D, float lam, float lamS,
                                            float c, float ace) {
  const float q = fexp2(fmaf(zq, kLog2e, -lse_q2));
  const float dd = (zq - zp) - D;
  const float f = q > 0.f ? q * dd : 0.f;
  const float sterm = f <= c ? f + q : 0.f;
  return fmaf(-lamS, q, fmaf(lam, sterm, ace * q));
}

// Workgroups per CU: aligned bf16 chunks fit 64 VGPRs without spills (eight
// per CU; the exact path reads its chunk again rather than holding it across
// its second barrier, and a rejected row's residual mass has a loop of its
// own), measured 5% faster than seven for supervision alone and 1-2% fused
// with verification; fp32 chunks take twice the registers and the
// element-wise loads of unaligned rows more.
template <bool BF16, bool ALIGNED, int VMODE, bool FKL>
constexpr int sup_min_waves() {
  return BF16 && ALIGNED ? (FKL ? 4 : (kElems <= 32 ? 8 : 4)) : 1;
}

// FKL: the forward-KL variant (supervision only): pass 1 also sums
// e^{z_p - m} (z_q - z_p) per chunk, the gradient adds q - p.
template <bool BF16, bool ALIGNED, int VMODE, bool FKL = false>
__global__ __launch_bounds__(kThreads, (sup_min_waves<BF16, ALIGNED, VMODE, FKL>())) void sup_kernel(KParams P) {
  constexpr bool SAMPLED = VMODE == 2, VERIFY = VMODE != 0;
  constexpr bool DEFER_X = VMODE != 1;  // argmax searched after the row barrier
  constexpr int VEC = Chunk<BF16>::VEC;
  constexpr int NV = kElems / VEC;
  __shared__ FinShared fs;
  __shared__ int sh_ok;
  // bf16 logits: exp(z_q - m) of this thread's draft entries from pass 1, as
  // fp16 pairs (slot-major, 16 KB); the fast-path gradient reads q back
  // instead of recomputing an exponential (fp16 keeps q to 2^-11, well inside
  // the bf16 output's rounding).  fp32 logits recompute q.  Each thread reads
  // only what it wrote.
  constexpr bool ECACHE = BF16;
  __shared__ uint32_t ecache[ECACHE ? kElems / 2 * kThreads : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int G = P.G;
  const int k = P.k, V = P.V;
  // Workgroup -> (row slot, chunk j) -> (request b, position i); workspace
  // slot r = b*(k+1) + i.  The draft rows come first; the bonus rows of
  // verification (one per request, i = L_b) follow them, so that the short
  // workgroups that never wait at a barrier run last.
  const int s_ = (int)blockIdx.x / G;
  const int j = (int)blockIdx.x - s_ * G;
  const RowSlot sl = row_slot(P, s_, VERIFY);
  if (sl.b < 0) return;
  const int b = sl.b, i = sl.i;
  const int r = b * (k + 1) + i;
  const bool draft_row = sl.n >= 0;
  const int v0 = j * kChunk;

  const void* trow = target_row_ptr<BF16>(P, b, i, sl.n);
  const void* drow = nullptr;
  if (draft_row)
    drow = draft_row_ptr<BF16>(P, b, i, sl.n);

  // ---- pass 1
  Chunk<BF16> cp, cq;
  load_chunk<BF16, ALIGNED>(cp, trow, v0, V);
  if (draft_row) load_chunk<BF16, ALIGNED>(cq, drow, v0, V);
  // Per-row scalars needed after the barrier, fetched now so that their
  // latency overlaps the chunk loads.
  int xtok = 0, n = 0;
  float u_acc = 0.f, zpx = 0.f, zqx = 0.f;
  if (draft_row) {
    n = sl.n;  // packed row
    if constexpr (SAMPLED) {
      xtok = (int)sload_u32(P.tokens + (size_t)b * k + i);
      if (xtok < 0 || xtok >= V) {
        if (tid == 0 && j == 0) flag(P.status, ADAFLASH_FLAG_BAD_TOKEN);
        xtok = xtok < 0 ? 0 : V - 1;
      }
      u_acc = __uint_as_float(sload_u32(P.uniforms + (size_t)b * (k + 1) + i));
      zpx = sload_logit<BF16>(trow, xtok);
      zqx = sload_logit<BF16>(drow, xtok);
    }
  }
  float mp = chunk_max<BF16>(cp), mq = neg_inf();
  if (draft_row) mq = chunk_max<BF16>(cq);
  cp.opaque();
  cq.opaque();
  float Mw[2] = {mp, mq};
  {
    const int ops[2] = {OP_MAX, OP_MAX};
    wg_reduce<2>(Mw, ops, fs.red);
  }
  // Greedy verification needs every row's argmax in the finaliser: the lowest
  // index of this chunk holding the chunk maximum of z_p goes into the record
  // (only threads that hold it search).  Otherwise only the chunk that holds
  // the row maximum looks for it, after the row barrier.
  int cand = kIntMax;
  if (!DEFER_X && mp == Mw[0]) {
    int ce = 0;
#pragma unroll
    for (int e = kElems - 1; e >= 0; --e)
      if (cp.get(e) == Mw[0]) ce = e;
    cand = entry_index<BF16>(v0, ce);
    if (cand >= V) cand = kIntMax;  // padding (a row of -inf only)
  }
  float sp = 0.f, sq = 0.f, W = 0.f, Amax = neg_inf(), Wp = 0.f;
  const float ap = uniform(Mw[0] == neg_inf() ? 0.f : -Mw[0] * kLog2e);
  const float aq = uniform(Mw[1] == neg_inf() ? 0.f : -Mw[1] * kLog2e);
  if (draft_row) {
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2) {
      uint32_t hw[VEC / 2];
#pragma unroll
      for (int u = 0; u < VEC; u += 2) {
        float ee2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int e = s2 * VEC + u + t;
          const float zq = cq.get(e), zp = cp.get(e);
          const float ee = fexp2(fmaf(zq, kLog2e, aq));
          const float ep = fexp2(fmaf(zp, kLog2e, ap));
          sp += ep;
          if constexpr (FKL) Wp = fmaf(ep, zq - zp, Wp);
          sq += ee;
          const float pr = ee * (zq - zp);
          W += pr;
          Amax = fmaxf(Amax, pr);
          ee2[t] = ee;
        }
        if constexpr (ECACHE) hw[u / 2] = pack_f16x2(ee2[0], ee2[1]);
      }
      if constexpr (ECACHE)
        *(uint4*)(ecache + ((size_t)s2 * kThreads + tid) * 4) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
  } else if (SAMPLED) {
#pragma unroll
    for (int e = 0; e < kElems; ++e) sp += fexp2(fmaf(cp.get(e), kLog2e, ap));
  }
  {
    // Only thread 0 publishes the record; fs.red is next written after the
    // row barrier.
    static_assert(!FKL || DEFER_X, "the forward-KL sum takes the argmax slot");
    constexpr int NR = DEFER_X && !FKL ? 4 : 5;
    float v[5] = {sp, sq, W, Amax, FKL ? Wp : __int_as_float(cand)};
    const int ops[5] = {OP_SUM, OP_SUM, OP_SUM, OP_MAX, FKL ? OP_SUM : OP_MINI};
    wg_reduce_lead<NR>(reinterpret_cast<float(&)[NR]>(v), reinterpret_cast<const int(&)[NR]>(ops), fs.red);
    if (tid == 0) {
      float* rec = P.part1 + ((size_t)r * G + j) * kRec1;
      pub_store(rec + 0, Mw[0]);
      if (!DEFER_X) pub_store(rec + 1, v[4]);
      pub_store(rec + 2, v[0]);
      pub_store(rec + 3, v[2]);
      pub_store(rec + 4, Mw[1]);
      pub_store(rec + 5, v[1]);
      pub_store(rec + 6, v[3]);
      if (FKL) pub_store(rec + 7, v[4]);
    }
  }
  if (!draft_row) return;

  bool alive = arrive_and_wait(&P.rowcnt[(size_t)r * kCounterStride], G, P.status, &sh_ok);
  if (!alive) return;
  // Sampled verification: the finaliser draws from the residual of the first
  // rejected row only, so a row behind a row already known to be rejected
  // skips the residual.  Wave 1 reads the earlier rows' accept flags (reset
  // to "unknown" by the pack kernel) while wave 0 combines the records.
  if (SAMPLED && wave == 1) {
    const int l = tid - 64;
    const bool rej = l < i && pub_load(P.rowrec + (size_t)(r - i + l) * kRowRec + 1) == 0.f;
    const unsigned long long any = __ballot(rej);
    if (l == 0) fs.i[0] = any != 0ull;
  }
  const SupStats st = combine_sup<SAMPLED, DEFER_X, FKL>(P, r, fs, zpx, zqx, u_acc);
  const bool earlier_rejected = SAMPLED && fs.i[0] != 0;
  const float lse_q2 = st.lse_q2, lse_p2 = st.lse_p2, D = st.D, KL = st.KL;
  // Loss weights of this row: hard-label term ace, clipped reverse KL lam,
  // forward KL afk, all scaled by the position weight (1 unless decaying).
  const float wi = P.wdecay > 0.f ? uniform(fexp2(-(float)i * kLog2e / P.wdecay)) : 1.f;
  const float c = P.clip_c, lam = uniform(wi * P.lambda), ace = uniform(wi * P.a_ce);
  const float afk = FKL ? wi : 0.f;
  const bool fast = !st.nonfinite && st.bound <= 0.999f * c;
  // (A row maximum at the padding value means a row of -inf only.)
  const float pad = __uint_as_float(BF16 ? 0xff7f0000u : 0xff7fffffu);
  if (tid == 0 && j == 0 && !(st.Mp < __builtin_inff() && st.Mp > pad && st.Sp > 0.f && st.Sq > 0.f))
    flag(P.status, ADAFLASH_FLAG_NONFINITE);

  bool accept = true;
  if constexpr (SAMPLED) {
    accept = st.margin > 0.f;
    if (tid == 0 && j == 0) {
      pub_store(P.rowrec + (size_t)r * kRowRec + 1, accept ? 1.f : 0.f);
      pub_store(P.rowrec + (size_t)r * kRowRec + 2, st.margin);
      if (P.margins) P.margins[(size_t)b * (k + 1) + i] = st.margin;
    }
  }

  int xs = st.xstar;
  if constexpr (DEFER_X) {
    // st.xstar is the lowest chunk whose maximum is the row maximum; that
    // chunk finds the lowest index holding it.
    xs = kIntMax;
    if (j == st.xstar) {
      int ce = kIntMax;
#pragma unroll
      for (int e = kElems - 1; e >= 0; --e)
        if (cp.get(e) == st.Mp) ce = e;
      int cidx = ce == kIntMax ? kIntMax : entry_index<BF16>(v0, ce);
      if (cidx >= V) cidx = kIntMax;  // padding (a row of -inf only)
      float x1[1] = {__int_as_float(cidx)};
      const int o1[1] = {OP_MINI};
      wg_reduce<1>(x1, o1, fs.red);
      xs = __float_as_int(x1[0]);
    }
  }
  cp.opaque();
  cq.opaque();
  const int xo = xs - v0;
  const bool xs_here = xs < V && xo >= 0 && xo < kChunk && ((xo % (kThreads * VEC)) / VEC) == tid;
  // z_q[x*] (one value for the workgroup; z_p[x*] is the row maximum).  The
  // thread holding x* rewrites its gradient entry after the sweep with the
  // one-hot term.
  const float zqs = xs >= 0 && xs < V ? sload_logit<BF16>(drow, xs) : 0.f;

  // Residual mass max(0, p - q) of a rejected row.
  const bool need_res = SAMPLED && !accept && !earlier_rejected;
  float Zpart = 0.f;

  const bool whole = v0 + kChunk <= V;
  auto store_slot = [&](int s2, const float (&g)[VEC]) {
    const int idx0 = v0 + s2 * (kThreads * VEC) + tid * VEC;
    if constexpr (BF16 && ALIGNED) {
      if (whole) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc((const uint16_t*)P.grad + (size_t)n * V, V * 2);
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t o = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                           pack_bf16x2(g[6], g[7])};
        __builtin_amdgcn_raw_buffer_store_b128(o, rs, tid * 16, (v0 + s2 * (kThreads * VEC)) * 2, kStreamPolicy);
        return;
      }
    }
    if constexpr (BF16) {
      uint16_t* gr = (uint16_t*)P.grad + (size_t)n * V;
      if constexpr (ALIGNED) {
        if (idx0 < V) {
          uint4 o;
          o.x = pack_bf16x2(g[0], g[1]);
          o.y = pack_bf16x2(g[2], g[3]);
          o.z = pack_bf16x2(g[4], g[5]);
          o.w = pack_bf16x2(g[6], g[7]);
          *(uint4*)(gr + idx0) = o;
        }
      } else {
#pragma unroll
        for (int u = 0; u < VEC; ++u)
          if (idx0 + u < V) gr[idx0 + u] = __builtin_bit_cast(uint16_t, (__bf16)g[u]);
      }
    } else {
      float* gr = (float*)P.grad + (size_t)n * V;
      if constexpr (ALIGNED) {
        if (idx0 < V) *(float4*)(gr + idx0) = make_float4(g[0], g[1], g[2], g[3]);
      } else {
#pragma unroll
        for (int u = 0; u < VEC; ++u)
          if (idx0 + u < V) gr[idx0 + u] = g[u];
      }
    }
  };
  auto store_one = [&](int v, float g) {
    if constexpr (BF16) ((uint16_t*)P.grad)[(size_t)n * V + v] = __builtin_bit_cast(uint16_t, (__bf16)g);
    else ((float*)P.grad)[(size_t)n * V + v] = g;
  };

  float Rrow = KL;
  float gstar = 0.f;
  if (fast) {
    // g = q (1 + lambda (dz - D - KL)) = q (lambda dz + c1), with q = e s the
    // cached pass-1 exponential e = exp(z_q - m) scaled by s = exp(m - lse_q).
    // (plus, for the forward KL, afk (q - p): afk joins c1 and afk p is subtracted)
    const float c1 = FKL ? fmaf(-lam, D, ace - lam * KL) + afk : fmaf(-lam, D, ace - lam * KL);
    const float sc = uniform(fexp2(-aq - lse_q2));
    const float lsc = uniform(lam * sc), csc = uniform(c1 * sc);
    // The residual sweep shares the gradient's unpacked logits; its q is
    // recomputed in fp32 (p - q cancels).
    auto sweep = [&](auto with_res) {
#pragma unroll
      for (int s2 = 0; s2 < NV; ++s2) {
        uint32_t hw[VEC / 2];
        if constexpr (ECACHE) {
          const uint4 h4 = *(const uint4*)(ecache + ((size_t)s2 * kThreads + tid) * 4);
          hw[0] = h4.x;
          hw[1] = h4.y;
          hw[2] = h4.z;
          hw[3] = h4.w;
        }
        float g[VEC];
        float dz8[8];
        if constexpr (ECACHE && !decltype(with_res)::value) bf16_diff8(&cq.w[s2 * 4], &cp.w[s2 * 4], dz8);
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
          const int e = s2 * VEC + u;
          const float zq = cq.get(e), zp = cp.get(e);
          float q = 0.f;
          if (!ECACHE || decltype(with_res)::value) q = fexp2(fmaf(zq, kLog2e, -lse_q2));
          const float pterm = FKL ? -afk * fexp2(fmaf(zp, kLog2e, -lse_p2)) : 0.f;
          if constexpr (ECACHE) {
            const float dz = decltype(with_res)::value ? zq - zp : dz8[u];
            g[u] = fma_f16(hw[u / 2], u & 1, fmaf(lsc, dz, csc), pterm);
          } else {
            g[u] = fmaf(q, fmaf(lam, zq - zp, c1), pterm);
          }
          if constexpr (decltype(with_res)::value)
            Zpart += fmaxf(0.f, fexp2(fmaf(zp, kLog2e, -lse_p2)) - q);
        }
        if (P.grad) store_slot(s2, g);
      }
    };
    if (P.grad) sweep(std::false_type{});
    if (need_res) {
      // The residual mass of a rejected row, in a loop of its own (fewer
      // live registers than folding it into the gradient sweep).
#pragma unroll
      for (int e = 0; e < kElems; ++e) {
        const float q = fexp2(fmaf(cq.get(e), kLog2e, -lse_q2));
        Zpart += fmaxf(0.f, fexp2(fmaf(cp.get(e), kLog2e, -lse_p2)) - q);
      }
    }
    if (xs_here) {
      // (z_p at x* is the row maximum)
      const float pstar = FKL ? -afk * fexp2(st.Mp * kLog2e - lse_p2) : 0.f;
      if constexpr (ECACHE) {
        const int xs_slot = xo / (kThreads * VEC), xs_u = xo % VEC;
        const uint32_t w = ecache[((size_t)xs_slot * kThreads + tid) * 4 + xs_u / 2];
        gstar = fma_f16(w, xs_u & 1, fmaf(lsc, zqs - st.Mp, csc), pstar) - ace;
      } else {
        gstar = fmaf(fexp2(fmaf(zqs, kLog2e, -lse_q2)), fmaf(lam, zqs - st.Mp, c1), pstar) - ace;
      }
    }
  } else {
    // Exact path: clipped sums, second barrier, then the gradient (the
    // per-entry terms are recomputed from the packed logits).
    float Spart = 0.f, Rpart = 0.f;
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
      const float zq = cq.get(e), zp = cp.get(e);
      const float q = fexp2(fmaf(zq, kLog2e, -lse_q2));
      if (need_res) Zpart += fmaxf(0.f, fexp2(fmaf(zp, kLog2e, -lse_p2)) - q);
      const float dd = (zq - zp) - D;
      const float f = q > 0.f ? q * dd : 0.f;
      const bool inU = f <= c;
      Rpart += inU ? f : c;
      Spart += inU ? f + q : 0.f;
    }
    float s3[3] = {Spart, Rpart, Zpart};
    const int ops3[3] = {OP_SUM, OP_SUM, OP_SUM};
    wg_reduce<3>(s3, ops3, fs.red);
    if (tid == 0) {
      float* rec = P.part2 + ((size_t)r * G + j) * kRec2;
      pub_store(rec + 0, s3[0]);
      pub_store(rec + 1, s3[1]);
      if (SAMPLED) pub_store(rec + 2, s3[2]);
    }
    alive = arrive_and_wait(&P.rowcnt[(size_t)r * kCounterStride], 2 * G, P.status, &sh_ok);
    if (!alive) return;
    float sr[2] = {0.f, 0.f};
    if (tid < G) {
      const float* rec = P.part2 + ((size_t)r * G + tid) * kRec2;
      sr[0] = pub_load(rec + 0);
      sr[1] = pub_load(rec + 1);
    }
    const int srops[2] = {OP_SUM, OP_SUM};
    wg_reduce<2>(sr, srops, fs.red);
    Rrow = sr[1];
    const float lamS = uniform(lam * sr[0]);
    cp.opaque();
    cq.opaque();
    if (P.grad) {
#pragma unroll
      for (int s2 = 0; s2 < NV; ++s2) {
        float g[VEC];
        if constexpr (BF16 && ALIGNED) {
          // The chunk's words are read again slot by slot (this path is
          // rare), so that no chunk is held in registers across the second
          // barrier: the kernel then fits 64 registers without spills.
          const int idx0 = v0 + s2 * (kThreads * VEC) + tid * VEC;
          const uint4 pad4 = make_uint4(0xff7fff7fu, 0xff7fff7fu, 0xff7fff7fu, 0xff7fff7fu);
          const uint4 wp = idx0 < V ? *(const uint4*)((const uint16_t*)trow + idx0) : pad4;
          const uint4 wq = idx0 < V ? *(const uint4*)((const uint16_t*)drow + idx0) : pad4;
          cp.w[s2 * 4 + 0] = wp.x;
          cp.w[s2 * 4 + 1] = wp.y;
          cp.w[s2 * 4 + 2] = wp.z;
          cp.w[s2 * 4 + 3] = wp.w;
          cq.w[s2 * 4 + 0] = wq.x;
          cq.w[s2 * 4 + 1] = wq.y;
          cq.w[s2 * 4 + 2] = wq.z;
          cq.w[s2 * 4 + 3] = wq.w;
        }
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
          const int e = s2 * VEC + u;
          g[u] = grad_exact(cq.get(e), cp.get(e), lse_q2, D, lam, lamS, c, ace);
          if constexpr (FKL) g[u] -= afk * fexp2(fmaf(cp.get(e), kLog2e, -lse_p2));
          // Rarely taken path: limit the interleaving (and registers) here.
          if (u & 1) __builtin_amdgcn_sched_barrier(0);
        }
        store_slot(s2, g);
      }
    }
    gstar = grad_exact(zqs, st.Mp, lse_q2, D, lam, lamS, c, ace) - ace;
    if constexpr (FKL) gstar -= afk * fexp2(st.Mp * kLog2e - lse_p2);
  }
  if (fast && need_res) {
    // The residual mass of this chunk goes to the finaliser.
    float z1[1] = {Zpart};
    const int o1[1] = {OP_SUM};
    wg_reduce<1>(z1, o1, fs.red);
    if (tid == 0) pub_store(P.part2 + ((size_t)r * G + j) * kRec2 + 2, z1[0]);
  }
  if (xs_here) {
    // One-hot term of the hard-label cross entropy and the losses, by the
    // thread that holds x* (its slot store above is overwritten).
    if (P.grad) store_one(xs, gstar);
    if (P.loss_ce) P.loss_ce[n] = lse_q2 * kLn2 - zqs;
    if (P.loss_rkl) P.loss_rkl[n] = Rrow;
    if (P.loss_var) P.loss_var[n] = wi * (P.a_ce * (lse_q2 * kLn2 - zqs) + P.lambda * Rrow + (FKL ? st.fkl : 0.f));
  }
}

// -------------------------------- supervision kernel for bf16 rows (V % 8 == 0)
//
// The passes of sup_kernel with less work per entry, for bf16 rows whose
// length is a multiple of eight and whose base pointers are 16-byte aligned:
//  * each thread shifts its exponentials by its own maxima, so pass 1 needs no
//    workgroup reduction before it starts; the thread partials are rescaled
//    once, when the waves merge them;
//  * the thread maxima come from packed f16 maxima of the raw bf16 patterns,
//    three words per instruction (a bf16 pattern read as f16 orders like the
//    bf16 value unless the f16 reading is a NaN, which only -inf, +inf and
//    |z| >= 2^121 produce; threads holding such an entry take the exact
//    integer method);
//  * the padding past V is -2^120, a bf16 pattern that is finite as f16;
//  * a bonus row whose request already has a rejected draft is not loaded
//    (the finaliser reads row L only when every draft is accepted);
//  * the exact path writes its gradient from the pass-1 cache as well, with
//    each entry's clip decision kept as one bit;
//  * for large c the per-thread clip bound skips a multiplication per entry
//    (kLooseClip).

constexpr uint32_t kPadBf16x2 = 0xFB80FB80u;  // -2^120 in both halves

// Clip thresholds from which the bf16 supervision kernel takes the looser
// per-thread clip bound.  A thread's bound is then s max(0, max dz) with s its
// largest q, against s max(e dz) (plus s max(0, -D) in both): on the c128
// workload every row stays on the fast path at c = 10 with either, while at
// c = 0.01 the tighter bound lets 84% of the exact path's waves skip their
// recomputation, and the looser one far fewer (measured 5% slower there).
constexpr float kLooseClip = 4.f;

// Chunk of a bf16 row with V % 8 == 0: whole slots of eight entries are inside
// or past the row; slots past it hold the padding value.
__device__ __forceinline__ void load_chunk_bf16(Chunk<true>& c, const void* row, int v0, int V) {
  constexpr int NV = kElems / 8;
  if (v0 + kChunk <= V) {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, V * 2);
    const int toff = (int)threadIdx.x * 16;
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, toff, (v0 + s * (kThreads * 8)) * 2, kStreamPolicy);
      c.w[s * 4 + 0] = q[0];
      c.w[s * 4 + 1] = q[1];
      c.w[s * 4 + 2] = q[2];
      c.w[s * 4 + 3] = q[3];
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < NV; ++s) {
    const int idx0 = v0 + s * (kThreads * 8) + (int)threadIdx.x * 8;
    uint4 q = make_uint4(kPadBf16x2, kPadBf16x2, kPadBf16x2, kPadBf16x2);
    if (idx0 < V) q = *(const uint4*)((const uint16_t*)row + idx0);
    c.w[s * 4 + 0] = q.x;
    c.w[s * 4 + 1] = q.y;
    c.w[s * 4 + 2] = q.z;
    c.w[s * 4 + 3] = q.w;
  }
}

// Largest of the thread's 32 entries (exact).  Packed f16 maxima of the raw
// patterns; a NaN result means some pattern is an f16 NaN, and the signed
// 16-bit integer method (chunk_max) decides instead.
__device__ __forceinline__ float thread_max_bf16(const Chunk<true>& c) {
  f16x2_t m = __builtin_bit_cast(f16x2_t, c.w[0]);
#pragma unroll
  for (int q = 1; q < Chunk<true>::NW; ++q) m = __builtin_elementwise_maximum(m, __builtin_bit_cast(f16x2_t, c.w[q]));
  const _Float16 h = __builtin_elementwise_maximum(m.x, m.y);
  if (__builtin_isnan(h)) return chunk_max<true>(c);
  return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// LOOSE: the per-thread clip bound A_t is max(0, max dz) instead of max e dz
// (e <= 1 makes either bound every e dz): one multiplication per entry less
// in pass 1, at the cost of a looser bound, taken for large c only (see
// kLooseClip).
template <int VMODE, bool FKL = false, bool LOOSE = false>
__global__ __launch_bounds__(kThreads, 8) void fsup_kernel(KParams P) {
  static_assert(VMODE == 0 || VMODE == 2, "opd only, or fused with sampled verification at T = 1");
  constexpr bool SAMPLED = VMODE == 2, VERIFY = VMODE != 0;
  constexpr int VEC = 8;
  constexpr int NV = kElems / VEC;
  __shared__ SupShared fs;
  // exp(z_q - m) of this thread's draft entries from pass 1 (m: the thread's
  // maximum), as fp16 pairs, slot-major; each thread reads only what it wrote.
  __shared__ uint32_t ecache[kElems / 2 * kThreads];
  __shared__ float wpart[kWaves][8];
  // This thread's pass-1 sums e, W and max e dz for the exact path (kept in
  // LDS rather than in registers across the row barrier).
  __shared__ float tpart[3][kThreads];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int G = P.G;
  const int k = P.k, V = P.V;
  const int s_ = (int)blockIdx.x / G;
  const int j = (int)blockIdx.x - s_ * G;
  const uint32_t call_epoch = sload_u32(P.epoch);
  const RowSlot sl = row_slot(P, s_, VERIFY);
  if (sl.b < 0) return;
  const int b = sl.b, i = sl.i;
  const int r = b * (k + 1) + i;
  const bool draft_row = sl.n >= 0;
  const int v0 = j * kChunk;

  if (VERIFY && !draft_row) {
    // Bonus row: skip it when a draft of the request is already known to be
    // rejected (flags of rows still undecided read "unknown", 2).
    if (wave == 0) {
      const bool rej = lane < i && pub_load(P.rowrec + (size_t)(r - i + lane) * kRowRec + 1) == 0.f;
      const unsigned long long any = __ballot(rej);
      if (lane == 0) fs.i[1] = any != 0ull;
    }
    __syncthreads();
    if (fs.i[1]) return;
  }

  const void* trow = target_row_ptr<true>(P, b, i, sl.n);
  const void* drow = nullptr;
  if (draft_row) drow = draft_row_ptr<true>(P, b, i, sl.n);

  // ---- pass 1
  Chunk<true> cp, cq;
  load_chunk_bf16(cp, trow, v0, V);
  if (draft_row) load_chunk_bf16(cq, drow, v0, V);
  int xtok = 0, n = 0;
  float u_acc = 0.f, zpx = 0.f, zqx = 0.f;
  if (draft_row) {
    n = sl.n;
    if constexpr (SAMPLED) {
      xtok = (int)sload_u32(P.tokens + (size_t)b * k + i);
      if (xtok < 0 || xtok >= V) {
        if (tid == 0 && j == 0) flag(P.status, ADAFLASH_FLAG_BAD_TOKEN);
        xtok = xtok < 0 ? 0 : V - 1;
      }
      u_acc = __uint_as_float(sload_u32(P.uniforms + (size_t)b * (k + 1) + i));
      zpx = sload_logit<true>(trow, xtok);
      zqx = sload_logit<true>(drow, xtok);
    }
  }
  const float mp = thread_max_bf16(cp);
  const float mq = draft_row ? thread_max_bf16(cq) : neg_inf();
  cp.opaque();
  cq.opaque();
  // Each thread's exponentials relative to 2^(its scale exponent).
  const int Ap = shift_of(mp), Aq = shift_of(mq);
  const float ap = -(float)Ap, aq = -(float)Aq;
  float sp = 0.f, sq = 0.f, W = 0.f, Amax = LOOSE ? 0.f : neg_inf(), Wp = 0.f;
  if (draft_row) {
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2) {
      uint32_t hw[VEC / 2];
#pragma unroll
      for (int u = 0; u < VEC; u += 2) {
        float ee2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int e = s2 * VEC + u + t;
          const float zq = cq.get(e), zp = cp.get(e);
          const float ee = fexp2(fmaf(zq, kLog2e, aq));
          const float ep = fexp2(fmaf(zp, kLog2e, ap));
          sp += ep;
          if constexpr (FKL) Wp = fmaf(ep, zq - zp, Wp);
          sq += ee;
          if constexpr (LOOSE) {
            const float dz = zq - zp;
            W = fmaf(ee, dz, W);
            Amax = fmaxf(Amax, dz);
          } else {
            const float pr = ee * (zq - zp);
            W += pr;
            Amax = fmaxf(Amax, pr);
          }
          ee2[t] = ee;
        }
        hw[u / 2] = pack_f16x2(ee2[0], ee2[1]);
      }
      *(uint4*)(ecache + ((size_t)s2 * kThreads + tid) * 4) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
  } else if (SAMPLED) {
#pragma unroll
    for (int e = 0; e < kElems; ++e) sp += fexp2(fmaf(cp.get(e), kLog2e, ap));
  }
  tpart[0][tid] = sq;
  tpart[1][tid] = W;
  tpart[2][tid] = Amax;
  {
    // Thread partials to the wave's scale exponents (exact ldexp), reduced
    // inside each wave; thread 0 merges the four waves the same way and
    // publishes the chunk record.  Padding entries (and whole padded threads
    // or waves) are exact zeros or vanish in the scaling, since the chunk
    // holds at least one entry of the row.
    const int Apw = __float_as_int(wave_reduce<OP_MAXI>(__int_as_float(Ap)));
    const int Aqw = __float_as_int(wave_reduce<OP_MAXI>(__int_as_float(Aq)));
    const float Mpw = wave_reduce_l63<OP_MAX>(mp);
    const int dp = Ap - Apw, dq = Aq - Aqw;
    const float v0s = wave_reduce_l63<OP_SUM>(__builtin_ldexpf(sp, dp));
    const float v1s = wave_reduce_l63<OP_SUM>(__builtin_ldexpf(sq, dq));
    const float v2s = wave_reduce_l63<OP_SUM>(__builtin_ldexpf(W, dq));
    const float v3s = wave_reduce_l63<OP_MAX>(__builtin_ldexpf(Amax, dq));
    const float v4s = FKL ? wave_reduce_l63<OP_SUM>(__builtin_ldexpf(Wp, dp)) : 0.f;
    if (lane == 63) {
      wpart[wave][0] = Mpw;
      wpart[wave][1] = __int_as_float(Apw);
      wpart[wave][2] = v0s;
      wpart[wave][3] = __int_as_float(Aqw);
      wpart[wave][4] = v1s;
      wpart[wave][5] = v2s;
      wpart[wave][6] = v3s;
      wpart[wave][7] = v4s;
    }
    __syncthreads();
    if (wave == 0) {
      // Lane w < 4 holds wave w's partials; two quad steps merge them, in the
      // order (w0 + w1) + (w2 + w3), into lane 0.
      const bool hw = lane < kWaves;
      const int wl = hw ? lane : 0;
      float Mp = hw ? wpart[wl][0] : neg_inf();
      int Apc = hw ? __float_as_int(wpart[wl][1]) : -1048576;
      int Aqc = hw ? __float_as_int(wpart[wl][3]) : -1048576;
      const int ap_l = Apc, aq_l = Aqc;
      Mp = fmaxf(Mp, dpp_f<0xB1>(Mp));
      Mp = fmaxf(Mp, dpp_f<0x4E>(Mp));
      Apc = max(Apc, dpp_i<0xB1>(Apc));
      Apc = max(Apc, dpp_i<0x4E>(Apc));
      Aqc = max(Aqc, dpp_i<0xB1>(Aqc));
      Aqc = max(Aqc, dpp_i<0x4E>(Aqc));
      const int sp_e = ap_l - Apc, sq_e = aq_l - Aqc;
      float Sp = hw ? __builtin_ldexpf(wpart[wl][2], sp_e) : 0.f;
      float Sq = hw ? __builtin_ldexpf(wpart[wl][4], sq_e) : 0.f;
      float Ws = hw ? __builtin_ldexpf(wpart[wl][5], sq_e) : 0.f;
      float As = hw ? __builtin_ldexpf(wpart[wl][6], sq_e) : neg_inf();
      float Wps = FKL && hw ? __builtin_ldexpf(wpart[wl][7], sp_e) : 0.f;
      Sp += dpp_f<0xB1>(Sp);
      Sp += dpp_f<0x4E>(Sp);
      Sq += dpp_f<0xB1>(Sq);
      Sq += dpp_f<0x4E>(Sq);
      Ws += dpp_f<0xB1>(Ws);
      Ws += dpp_f<0x4E>(Ws);
      As = fmaxf(As, dpp_f<0xB1>(As));
      As = fmaxf(As, dpp_f<0x4E>(As));
      if (FKL) {
        Wps += dpp_f<0xB1>(Wps);
        Wps += dpp_f<0x4E>(Wps);
      }
      if (lane == 0) {
        const size_t f0 = ((size_t)r * G + j) * kRec1;
        tag_store(P.part1, f0 + 0, Mp, call_epoch);
        tag_store(P.part1, f0 + 1, (float)Apc, call_epoch);
        tag_store(P.part1, f0 + 2, Sp, call_epoch);
        tag_store(P.part1, f0 + 3, Ws, call_epoch);
        tag_store(P.part1, f0 + 4, (float)Aqc, call_epoch);
        tag_store(P.part1, f0 + 5, Sq, call_epoch);
        tag_store(P.part1, f0 + 6, As, call_epoch);
        if (FKL) tag_store(P.part1, f0 + 7, Wps, call_epoch);
        if (draft_row)
          __hip_atomic_fetch_add(P.rowcnt + (size_t)r * kCounterStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (!draft_row) return;

  const SupStats st = combine_sup_pow2<SAMPLED, FKL, SupShared, !LOOSE>(P, r, fs, zpx, zqx, u_acc, call_epoch);
  if (!st.alive) return;
  const float lse_q2 = st.lse_q2, lse_p2 = st.lse_p2, D = st.D, KL = st.KL;
  const float wi = P.wdecay > 0.f ? uniform(fexp2(-(float)i * kLog2e / P.wdecay)) : 1.f;
  const float c = P.clip_c, lam = uniform(wi * P.lambda), ace = uniform(wi * P.a_ce);
  const float afk = FKL ? wi : 0.f;
  const bool fast = !st.nonfinite && st.bound <= 0.999f * c;
  const float pad = __uint_as_float(kPadBf16x2 & 0xffff0000u);
  if (tid == 0 && j == 0 && !(st.Mp < __builtin_inff() && st.Mp > pad && st.Sp > 0.f && st.Sq > 0.f))
    flag(P.status, ADAFLASH_FLAG_NONFINITE);

  bool accept = true;
  if constexpr (SAMPLED) {
    accept = st.margin > 0.f;
    if (tid == 0 && j == 0) {
      pub_store(P.rowrec + (size_t)r * kRowRec + 1, accept ? 1.f : 0.f);
      pub_store(P.rowrec + (size_t)r * kRowRec + 2, st.margin);
      if (P.margins) P.margins[(size_t)b * (k + 1) + i] = st.margin;
    }
  }
  // Only the first rejected row of a request needs its residual mass.  A
  // rejected row reads the accept flags of the request's earlier rows here,
  // after its own barrier, and decides after its gradient: by then most
  // earlier rows have published theirs (a flag still "unknown" counts as not
  // rejected, and the row computes a residual that may go unused).
  const bool ask = SAMPLED && !accept && i > 0;  // (uniform)
  float flag_l = 1.f;
  if (ask && wave == 1 && lane < i) flag_l = pub_load(P.rowrec + (size_t)(r - i + lane) * kRowRec + 1);

  // st.xstar is the lowest chunk whose maximum is the row maximum; that chunk
  // finds the lowest index holding it.
  int xs = kIntMax;
  if (j == st.xstar) {
    int ce = kIntMax;
#pragma unroll
    for (int e = kElems - 1; e >= 0; --e)
      if (cp.get(e) == st.Mp) ce = e;
    int cidx = ce == kIntMax ? kIntMax : entry_index<true>(v0, ce);
    if (cidx >= V) cidx = kIntMax;
    float x1[1] = {__int_as_float(cidx)};
    const int o1[1] = {OP_MINI};
    wg_reduce<1>(x1, o1, fs.red);
    xs = __float_as_int(x1[0]);
  }
  cp.opaque();
  cq.opaque();
  const int xo = xs - v0;
  const bool xs_here = xs < V && xo >= 0 && xo < kChunk && ((xo % (kThreads * VEC)) / VEC) == tid;
  const float zqs = xs >= 0 && xs < V ? sload_logit<true>(drow, xs) : 0.f;

  float Zpart = 0.f;
  const bool whole = v0 + kChunk <= V;
  auto store_slot = [&](int s2, const float (&g)[VEC]) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t o = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                       pack_bf16x2(g[6], g[7])};
    if (whole) {
      const __amdgpu_buffer_rsrc_t rs = row_rsrc((const uint16_t*)P.grad + (size_t)n * V, V * 2);
      __builtin_amdgcn_raw_buffer_store_b128(o, rs, tid * 16, (v0 + s2 * (kThreads * VEC)) * 2, kStreamPolicy);
    } else {
      const int idx0 = v0 + s2 * (kThreads * VEC) + tid * VEC;
      if (idx0 < V) *(u32x4_t*)((uint16_t*)P.grad + (size_t)n * V + idx0) = o;
    }
  };

  float Rrow = KL;
  float gstar = 0.f;
  if (fast) {
    // g = q (lambda dz + c1), q = e s: e from the cache (this thread's shift),
    // s = exp(m - lse_q) with m this thread's maximum.
    const float c1 = FKL ? fmaf(-lam, D, ace - lam * KL) + afk : fmaf(-lam, D, ace - lam * KL);
    const float sc = fexp2(-aq - lse_q2);
    const float lsc = lam * sc, csc = c1 * sc;
    if (P.grad) {
#pragma unroll
      for (int s2 = 0; s2 < NV; ++s2) {
        const uint4 h4 = *(const uint4*)(ecache + ((size_t)s2 * kThreads + tid) * 4);
        const uint32_t hw[4] = {h4.x, h4.y, h4.z, h4.w};
        float dz8[8];
        bf16_diff8(&cq.w[s2 * 4], &cp.w[s2 * 4], dz8);
        float g[VEC];
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
          const float pterm = FKL ? -afk * fexp2(fmaf(cp.get(s2 * VEC + u), kLog2e, -lse_p2)) : 0.f;
          g[u] = fma_f16(hw[u / 2], u & 1, fmaf(lsc, dz8[u], csc), pterm);
        }
        store_slot(s2, g);
      }
    }
    if (xs_here) {
      const float pstar = FKL ? -afk * fexp2(st.Mp * kLog2e - lse_p2) : 0.f;
      const int xs_slot = xo / (kThreads * VEC), xs_u = xo % VEC;
      const uint32_t w = ecache[((size_t)xs_slot * kThreads + tid) * 4 + xs_u / 2];
      gstar = fma_f16(w, xs_u & 1, fmaf(lsc, zqs - st.Mp, csc), pstar) - ace;
    }
  } else {
    // Exact path: clipped sums, second barrier, then the gradient.  A wave
    // whose entries cannot be clipped (the fast path's bound, taken per
    // thread: f_v <= s (A_t + max(0, -D)), with A_t the thread's bound on
    // e dz from pass 1 and s = exp(m - lse_q)) takes its sums from the pass-1
    // partials, sum_U f = s (W_t - D e_t) and sum_U q = s e_t, and writes the
    // gradient with the fast path's formula; the other waves recompute their sums'
    // terms in fp32 from the packed logits, which stay in registers, and keep
    // each entry's clip decision for the gradient.  So does a wave with a
    // non-finite pass-1 sum: a -inf logit makes an infinite or undefined term
    // (0 * inf) there, while recomputed terms with q = 0 are taken as 0.
    const float sc = fexp2(-aq - lse_q2);
    const float tb = sc * (tpart[2][tid] + fmaxf(0.f, -D));
    const float e_t = tpart[0][tid];
    const float F = sc * fmaf(-D, e_t, tpart[1][tid]);
    const bool wskip = __ballot(!(tb <= 0.999f * c) || !__builtin_isfinite(F)) == 0ull;  // (uniform in the wave)
    float Spart = 0.f, Rpart = 0.f;
    uint32_t ubits = 0u;  // (other waves) this thread's entries in U with q > 0
    static_assert(kElems <= 32, "one bit per entry");
    if (wskip) {
      Rpart = F;
      Spart = fmaf(sc, e_t, F);
    } else {
#pragma unroll
      for (int e = 0; e < kElems; ++e) {
        const float zq = cq.get(e), zp = cp.get(e);
        const float q = fexp2(fmaf(zq, kLog2e, -lse_q2));
        const float dd = (zq - zp) - D;
        const float f = q > 0.f ? q * dd : 0.f;
        const bool inU = f <= c;
        Rpart += inU ? f : c;
        Spart += inU ? f + q : 0.f;
        ubits |= (inU && q > 0.f ? 1u : 0u) << e;
      }
    }
    float s2v[2] = {Spart, Rpart};
    const int ops2[2] = {OP_SUM, OP_SUM};
    wg_reduce_lead<2>(s2v, ops2, fs.red);  // (fs.red is next written after the barrier below)
    if (tid == 0) {
      const size_t f0 = ((size_t)r * G + j) * kRec2;
      tag_store(P.part2, f0 + 0, s2v[0], call_epoch);
      tag_store(P.part2, f0 + 1, s2v[1], call_epoch);
    }
    // Second row barrier: wave 0 polls the G partial sums S and R until each
    // carries this call's epoch (two fields per chunk: no arrival counter).
    if (wave == 0) {
      float f2[2] = {0.f, 0.f};
      const float* recs2 = (const float*)((const uint64_t*)P.part2 + (size_t)r * G * kRec2);
      const bool ok = poll_fields<2>(recs2, kRec2, lane < G, lane, 0, 2, call_epoch, f2, P.status);
      const float S = wave_reduce<OP_SUM>(lane < G ? f2[0] : 0.f);
      const float R = wave_reduce<OP_SUM>(lane < G ? f2[1] : 0.f);
      if (lane == 0) {
        fs.f[0] = S;
        fs.f[1] = R;
        fs.i[3] = ok;
      }
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(fs.i[3])) return;
    Rrow = uniform(fs.f[1]);
    const float lamS = uniform(lam * fs.f[0]);
    // Unclipped entries: g = q (ace - lambda S + lambda (dz - D + 1)); clipped
    // entries (and those with q = 0, whose gradient is 0): g = q (ace -
    // lambda S).  q = e s with e from the pass-1 cache, as on the fast path;
    // the other waves' clip decisions are the ones their sums S and R took.
    const float c1x = fmaf(lam, 1.f - D, ace) - lamS + afk;
    const float lsc = lam * sc, csc = c1x * sc;
    const float Dm1 = uniform(D - 1.f);  // (lsc (D - 1) + csc = sc (ace - lambda S))
    if (P.grad) {
#pragma unroll
      for (int s2 = 0; s2 < NV; ++s2) {
        float g[VEC];
        const uint4 h4 = *(const uint4*)(ecache + ((size_t)s2 * kThreads + tid) * 4);
        const uint32_t hw[4] = {h4.x, h4.y, h4.z, h4.w};
        float dz8[8];
        bf16_diff8(&cq.w[s2 * 4], &cp.w[s2 * 4], dz8);
        if (wskip) {  // (no entry of the wave is clipped)
#pragma unroll
          for (int u = 0; u < VEC; ++u) {
            const float pterm = FKL ? -afk * fexp2(fmaf(cp.get(s2 * VEC + u), kLog2e, -lse_p2)) : 0.f;
            g[u] = fma_f16(hw[u / 2], u & 1, fmaf(lsc, dz8[u], csc), pterm);
          }
        } else {
#pragma unroll
          for (int u = 0; u < VEC; ++u) {
            const float pterm = FKL ? -afk * fexp2(fmaf(cp.get(s2 * VEC + u), kLog2e, -lse_p2)) : 0.f;
            const bool un = ((ubits >> (s2 * VEC + u)) & 1u) != 0u;
            g[u] = fma_f16(hw[u / 2], u & 1, fmaf(lsc, un ? dz8[u] : Dm1, csc), pterm);
          }
        }
        store_slot(s2, g);
      }
    }
    gstar = grad_exact(zqs, st.Mp, lse_q2, D, lam, lamS, c, ace) - ace;
    if constexpr (FKL) gstar += afk * (fexp2(fmaf(zqs, kLog2e, -lse_q2)) - fexp2(st.Mp * kLog2e - lse_p2));
  }
  // Residual mass max(0, p - q) of this chunk, for the finaliser's draw, if
  // no earlier row of the request has been seen rejected (both paths).
  if (SAMPLED && !accept) {  // (uniform)
    bool need_res = true;
    if (ask) {
      if (wave == 1) {
        const unsigned long long any = __ballot(flag_l == 0.f);
        if (lane == 0) fs.i[0] = any != 0ull;
      }
      __syncthreads();
      need_res = fs.i[0] == 0;
    }
    if (need_res) {
#pragma unroll
      for (int e = 0; e < kElems; ++e) {
        const float q = fexp2(fmaf(cq.get(e), kLog2e, -lse_q2));
        Zpart += fmaxf(0.f, fexp2(fmaf(cp.get(e), kLog2e, -lse_p2)) - q);
      }
      float z1[1] = {Zpart};
      const int o1[1] = {OP_SUM};
      wg_reduce<1>(z1, o1, fs.red);
      if (tid == 0) tag_store(P.part2, ((size_t)r * G + j) * kRec2 + 2, z1[0], call_epoch);
    }
  }
  if (xs_here) {
    if (P.grad) ((uint16_t*)P.grad)[(size_t)n * V + xs] = __builtin_bit_cast(uint16_t, (__bf16)gstar);
    if (P.loss_ce) P.loss_ce[n] = lse_q2 * kLn2 - zqs;
    if (P.loss_rkl) P.loss_rkl[n] = Rrow;
    if (P.loss_var) P.loss_var[n] = wi * (P.a_ce * (lse_q2 * kLn2 - zqs) + P.lambda * Rrow + (FKL ? st.fkl : 0.f));
  }
}

// ------------------------------------- verify-only: the pack step in block 0

// The pack kernel's work for the verify-only paths on padded logits, by one
// whole block: Lc, row_offsets (a scan in each wave, then across the waves,
// kThreads requests at a time), Lc[B] = N, the status word (nothing else of
// the first kernel writes it), the request counters of the residual kernel
// and the call epoch (which only the next kernel reads).
__device__ void pack_rows_block(const KParams& P) {
  __shared__ int s_wave[kWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < P.B; base += kThreads) {
    const int b = base + tid;
    int L = 0;
    if (b < P.B) {
      L = P.verify_len ? P.verify_len[b] : P.k;
      if (L < 1 || L > P.k) {
        atomicOr(&s_bad, ADAFLASH_FLAG_BAD_VERIFY_LEN);
        L = L < 1 ? 1 : P.k;
      }
      P.Lc[b] = L;
      P.rowcnt[((size_t)b * (P.k + 1) + P.k) * kCounterStride] = 0;  // the request's arrivals (vres_kernel)
    }
    int x = L;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(x, off, 64);
      if (lane >= off) x += t;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = s_wave[w];
      if (w < wave) woff += t;
      tot += t;
    }
    if (b < P.B) P.row_offsets[b] = carry + woff + x - L;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) {
    P.row_offsets[P.B] = carry;
    P.Lc[P.B] = carry;
    if (P.status) *P.status = s_bad;
    P.epoch[0] += 1u;  // read by the next kernel of the call
  }
}

// ------------------------------------------ greedy verification (no OPD)

// Greedy verification needs only every target row's maximum and its lowest
// index.  One workgroup takes chunk j of kGRows consecutive rows of a request
// (all their loads in flight together) and publishes one (max, argmax)
// record per row, with two workgroup reductions for all its rows.  Rows
// beyond the request's bonus row are skipped.  One row per workgroup:
// measured faster than two or four (c128: 56.9 against 58.5 and 59.9 us;
// more rows hold more registers, five workgroups per CU at four rows against
// eight at one, and leave the rows of partly used groups idle).
constexpr int kGRows = 1;

template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void gstat_kernel(KParams P) {
  __shared__ float red[kWaves * 2 * kGRows];
  const int tid = threadIdx.x;
  const int G = P.G, k = P.k, V = P.V;
  const int NG = (k + kGRows) / kGRows;  // row groups per request (k + 1 rows)
  const int q = (int)blockIdx.x / G;
  const int j = (int)blockIdx.x - q * G;
  const int b = q / NG, g = q - b * NG;
  if (P.pack_here && blockIdx.x == 0) pack_rows_block(P);
  const int L = P.pack_here ? clamp_len(P, b) : P.Lc[b];
  if (L < 0) return;
  const int i0 = g * kGRows;
  if (i0 > L) return;
  const int nr = min(kGRows, L + 1 - i0);  // rows i0 .. i0 + nr - 1 (uniform)
  const int v0 = j * kChunk;
  Chunk<BF16> c[kGRows];
#pragma unroll
  for (int t = 0; t < kGRows; ++t)
    if (t < nr) load_chunk<BF16, ALIGNED>(c[t], target_row_ptr<BF16>(P, b, i0 + t), v0, V);
  float m[kGRows];
  int ops[kGRows];
#pragma unroll
  for (int t = 0; t < kGRows; ++t) {
    m[t] = t < nr ? chunk_max<BF16>(c[t]) : neg_inf();
    ops[t] = OP_MAX;
  }
  float M[kGRows];
#pragma unroll
  for (int t = 0; t < kGRows; ++t) M[t] = m[t];
  wg_reduce<kGRows>(M, ops, red);
  // Lowest index holding each row's chunk maximum (only lanes that hold it search).
  float cand[kGRows];
#pragma unroll
  for (int t = 0; t < kGRows; ++t) {
    int ci = kIntMax;
    if (t < nr && m[t] == M[t]) {
#pragma unroll
      for (int e = kElems - 1; e >= 0; --e)
        if (c[t].get(e) == M[t]) ci = entry_index<BF16>(v0, e);
      if (ci >= V) ci = kIntMax;  // padding (a row of -inf only)
    }
    cand[t] = __int_as_float(ci);
    ops[t] = OP_MINI;
  }
  wg_reduce_lead<kGRows>(cand, ops, red + kWaves * kGRows);
  if (tid == 0) {
#pragma unroll
    for (int t = 0; t < kGRows; ++t) {
      if (t >= nr) break;
      float* rec = P.part1 + ((size_t)(b * (k + 1) + i0 + t) * G + j) * kRec1;
      pub_store(rec + 0, M[t]);
      pub_store(rec + 1, cand[t]);
    }
  }
}

// -------------------------------------------- sampled verification (no OPD)

// Sampled verification without supervision needs the row statistics in one
// place only (the accept test), and the residual of one row per request, so
// it runs without any barrier between workgroups: vstat_kernel publishes the
// chunk statistics of every draft row in use and exits; vres_kernel (one
// workgroup per request and pair of chunks) combines them, runs the accept
// tests, finds the first rejection and, for a rejected request, computes the
// residual mass of its chunks of that row (the one row read a second time),
// or, for a request that accepts every draft, the statistics of its chunks
// of the bonus row (read only then); the last of the request's workgroups
// draws.

// Pass 1 of one (draft row, chunk): chunk maxima of z_p and z_q and sums of
// exp((z - m) / T), published as a part1 record.
template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void vstat_kernel(KParams P) {
  __shared__ float red[kWaves * 8];
  const int tid = threadIdx.x;
  const int G = P.G, k = P.k, V = P.V;
  const int s_ = (int)blockIdx.x / G;
  const int j = (int)blockIdx.x - s_ * G;
  if (P.pack_here && blockIdx.x == 0) pack_rows_block(P);
  // Draft positions only (slot s = b k + i): the bonus row of a request is
  // read by the residual kernel, and only when every draft is accepted.
  const RowSlot sl = row_slot_draft(P, s_);
  if (sl.b < 0) return;
  const int b = sl.b, i = sl.i;
  const int r = b * (k + 1) + i;
  const int v0 = j * kChunk;
  const void* trow = target_row_ptr<BF16>(P, b, i, sl.n);
  const void* drow = draft_row_ptr<BF16>(P, b, i, sl.n);
  // The chunk holding the draft token (clamped as the accept test clamps it)
  // also publishes both logits there, for the accept test.
  int x = (int)sload_u32(P.tokens + (size_t)b * k + i);
  x = x < 0 ? 0 : (x >= V ? V - 1 : x);
  const bool xhere = x / kChunk == j;
  float zpx = 0.f, zqx = 0.f;
  if (xhere) {
    zpx = sload_logit<BF16>(trow, x);
    zqx = sload_logit<BF16>(drow, x);
  }
  Chunk<BF16> cp, cq;
  load_chunk<BF16, ALIGNED>(cp, trow, v0, V);
  load_chunk<BF16, ALIGNED>(cq, drow, v0, V);
  float m[2] = {chunk_max<BF16>(cp), chunk_max<BF16>(cq)};
  cp.opaque();
  cq.opaque();
  {
    const int ops[2] = {OP_MAX, OP_MAX};
    wg_reduce<2>(m, ops, red);
  }
  const float ap = uniform(m[0] == neg_inf() ? 0.f : -m[0] * P.kT);
  const float aq = uniform(m[1] == neg_inf() ? 0.f : -m[1] * P.kT);
  float sv[2] = {0.f, 0.f};
#pragma unroll
  for (int e = 0; e < kElems; ++e) sv[0] += fexp2(fmaf(cp.get(e), P.kT, ap));
#pragma unroll
  for (int e = 0; e < kElems; ++e) sv[1] += fexp2(fmaf(cq.get(e), P.kT, aq));
  const int ops[2] = {OP_SUM, OP_SUM};
  wg_reduce_lead<2>(sv, ops, red);
  if (tid == 0) {
    float* rec = P.part1 + ((size_t)r * G + j) * kRec1;
    pub_store(rec + 0, m[0]);
    pub_store(rec + 2, sv[0]);
    pub_store(rec + 4, m[1]);
    pub_store(rec + 5, sv[1]);
    if (xhere) {
      pub_store(rec + 6, zpx);
      pub_store(rec + 7, zqx);
    }
  }
}

// Folds a chunk record (m, s) into a running (M, S) at scale kT.
__device__ __forceinline__ void fold_ms(float& M, float& S, float m, float s, float kT) {
  if (m == neg_inf()) return;
  if (M == neg_inf()) {
    M = m;
    S = s;
  } else if (m > M) {
    S = S * fexp2((M - m) * kT) + s;
    M = m;
  } else {
    S += s * fexp2((m - M) * kT);
  }
}

// Chunks of a row loaded together by a residual workgroup (one round; a
// workgroup takes P.res_chunks chunks in rounds of this many).
constexpr int kResChunks = 2;

// Reduction inside each 16-lane row of a wave (every lane of the row gets
// the row's result); the first four steps of wave_reduce.
template <int OP>
__device__ __forceinline__ float row16_reduce(float v) {
  if constexpr (OP == OP_MAX) {
    const float k = __int_as_float(max_key(__float_as_int(v)));
    return __int_as_float(max_key(__float_as_int(row16_reduce<OP_MAXI>(k))));
  }
  v = op2<OP>(v, dpp_f<0xB1>(v));
  v = op2<OP>(v, dpp_f<0x4E>(v));
  v = op2<OP>(v, dpp_f<0x141>(v));
  v = op2<OP>(v, dpp_f<0x140>(v));
  return v;
}

// Residual masses sum max(0, p - q) of chunks jb, jb + 1, ... (kResChunks of
// them, up to je) of the rejected row A of request b, for the draw (s_row:
// that row's statistics).
template <bool BF16, bool ALIGNED>
__device__ void residual_of_chunks(const KParams& P, int b, int A, int jb, int je, const float (*s_row)[4],
                                   float* red, uint32_t ep) {
  const int tid = threadIdx.x;
  const int G = P.G, k = P.k, V = P.V;
  const int r0 = b * (k + 1);
  const int rA = r0 + A;
  const void* trow = target_row_ptr<BF16>(P, b, A);
  const void* drow = draft_row_ptr<BF16>(P, b, A);
  // All chunks' loads first, then the arithmetic.
  Chunk<BF16> cp[kResChunks], cq[kResChunks];
#pragma unroll
  for (int t = 0; t < kResChunks; ++t) {
    const int jt = jb + t;
    if (jt < je) {
      load_chunk<BF16, ALIGNED>(cp[t], trow, jt * kChunk, V);
      load_chunk<BF16, ALIGNED>(cq[t], drow, jt * kChunk, V);
    }
  }
  const float invSp = 1.f / s_row[A][1], invSq = 1.f / s_row[A][3];
  const float ap = -s_row[A][0] * P.kT, aq = -s_row[A][2] * P.kT;
  float z[kResChunks];
  int o[kResChunks];
#pragma unroll
  for (int t = 0; t < kResChunks; ++t) {
    z[t] = 0.f;
    o[t] = OP_SUM;
    if (jb + t < je) {
#pragma unroll
      for (int e = 0; e < kElems; ++e) {
        const float pv = mul_rn(fexp2(fmaf(cp[t].get(e), P.kT, ap)), invSp);
        const float qq = mul_rn(fexp2(fmaf(cq[t].get(e), P.kT, aq)), invSq);
        z[t] += fmaxf(0.f, pv - qq);
      }
    }
  }
  wg_reduce_lead<kResChunks>(z, o, red);
  if (tid == 0) {
#pragma unroll
    for (int t = 0; t < kResChunks; ++t) {
      const int jt = jb + t;
      if (jt < je) tag_store(P.part2, ((size_t)rA * G + jt) * kRec2 + 2, z[t], ep);
    }
  }
}

// Statistics at T of chunks jb, jb + 1, ... (kResChunks of them, up to je) of
// the bonus row L of request b (a request that accepts every draft), as the
// statistics kernel computes them for draft rows: the chunk maximum m of z_p
// and sum exp((z - m) / T), published as epoch-tagged fields 0 and 1 of the
// row's part2 records.
template <bool BF16, bool ALIGNED>
__device__ void bonus_of_chunks(const KParams& P, int b, int L, int jb, int je, float* red, uint32_t ep) {
  const int tid = threadIdx.x;
  const int G = P.G, k = P.k, V = P.V;
  const int rL = b * (k + 1) + L;
  const void* trow = target_row_ptr<BF16>(P, b, L);
  Chunk<BF16> cp[kResChunks];
#pragma unroll
  for (int t = 0; t < kResChunks; ++t) {
    const int jt = jb + t;
    if (jt < je) load_chunk<BF16, ALIGNED>(cp[t], trow, jt * kChunk, V);
  }
  float m[kResChunks], sv[kResChunks];
  int o[kResChunks];
#pragma unroll
  for (int t = 0; t < kResChunks; ++t) {
    m[t] = jb + t < je ? chunk_max<BF16>(cp[t]) : neg_inf();
    o[t] = OP_MAX;
  }
  wg_reduce<kResChunks>(m, o, red);
#pragma unroll
  for (int t = 0; t < kResChunks; ++t) {
    sv[t] = 0.f;
    o[t] = OP_SUM;
    if (jb + t < je) {
      const float a = uniform(m[t] == neg_inf() ? 0.f : -m[t] * P.kT);
#pragma unroll
      for (int e = 0; e < kElems; ++e) sv[t] += fexp2(fmaf(cp[t].get(e), P.kT, a));
    }
  }
  wg_reduce_lead<kResChunks>(sv, o, red);
  if (tid == 0) {
#pragma unroll
    for (int t = 0; t < kResChunks; ++t) {
      const int jt = jb + t;
      if (jt < je) {
        tag_store(P.part2, ((size_t)rL * G + jt) * kRec2 + 0, m[t], ep);
        tag_store(P.part2, ((size_t)rL * G + jt) * kRec2 + 1, sv[t], ep);
      }
    }
  }
}

// One workgroup per (request b, chunk j).  Each 16-lane row of the workgroup
// takes one draft row (16 at a time): lane c folds the records of chunks c,
// c + 16, ..., the lanes reduce them, the first lane runs the accept test
// with the logits at the draft token that the statistics kernel put in the
// record of the chunk holding it.  Every workgroup of the request does the
// same and finds the same first rejection A; for A < L it computes the
// residual mass sum max(0, p - q) of its chunks of row A and publishes it
// tagged with the call epoch.  The last workgroup of the request to arrive
// draws (no kernel of its own on this path), with A and row A's statistics
// at hand.
template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void vres_kernel(KParams P) {
  __shared__ float red[kWaves * 8];
  __shared__ float s_row[64][4];  // Mp, SpT, Mq, SqT of every draft row
  __shared__ int s_acc[64];
  __shared__ int s_first;
  __shared__ int s_last;
  __shared__ FinShared fs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = P.G, k = P.k, V = P.V;
  const int RC = P.res_chunks;
  const int GH = (G + RC - 1) / RC;
  const int b = (int)blockIdx.x / GH;
  const int h = (int)blockIdx.x - b * GH;  // chunks RC h ... RC h + RC - 1
  const int j = h;                         // (workgroup h == 0 writes the row flags)
  const int L = P.Lc[b];
  if (L < 0) return;
  const uint32_t ep = sload_u32(P.epoch);
  const int r0 = b * (k + 1);
  const int grp = tid >> 4, l16 = tid & 15;  // 16 groups of 16 lanes
  for (int i0 = 0; i0 < L; i0 += kThreads / 16) {
    const int i = i0 + grp;
    const bool live = i < L;  // uniform within the group
    const int r = r0 + i;
    // Every lane of the group reads the token (one address) and folds its
    // chunk records; the record of the chunk holding the token also carries
    // both logits there (from the statistics kernel).
    int x = 0;
    float u = 0.f;
    if (live) {
      x = P.tokens[(size_t)b * k + i];
      u = P.uniforms[(size_t)b * (k + 1) + i];
    }
    const int xc = x < 0 ? 0 : (x >= V ? V - 1 : x);
    const int jx = xc / kChunk;
    float Mp = neg_inf(), Sp = 0.f, Mq = neg_inf(), Sq = 0.f, zpx = 0.f, zqx = 0.f;
    if (live) {
      // Two records per lane per round, all their loads issued before either
      // is folded (one round trip for up to 32 chunks).
      for (int c = l16; c < G; c += 32) {
        const bool two = c + 16 < G;
        const float* rec = P.part1 + ((size_t)r * G + c) * kRec1;
        const float* rec2 = rec + 16 * kRec1;
        float f[8];
        f[0] = pub_load(rec + 0);
        f[1] = pub_load(rec + 2);
        f[2] = pub_load(rec + 4);
        f[3] = pub_load(rec + 5);
        f[4] = two ? pub_load(rec2 + 0) : neg_inf();
        f[5] = two ? pub_load(rec2 + 2) : 0.f;
        f[6] = two ? pub_load(rec2 + 4) : neg_inf();
        f[7] = two ? pub_load(rec2 + 5) : 0.f;
        if (c == jx) {
          zpx = pub_load(rec + 6);
          zqx = pub_load(rec + 7);
        } else if (c + 16 == jx) {
          zpx = pub_load(rec2 + 6);
          zqx = pub_load(rec2 + 7);
        }
        fold_ms(Mp, Sp, f[0], f[1], P.kT);
        fold_ms(Mq, Sq, f[2], f[3], P.kT);
        fold_ms(Mp, Sp, f[4], f[5], P.kT);
        fold_ms(Mq, Sq, f[6], f[7], P.kT);
      }
    }
    const float RMp = row16_reduce<OP_MAX>(Mp), RMq = row16_reduce<OP_MAX>(Mq);
    const float SpT = row16_reduce<OP_SUM>(Mp == neg_inf() ? 0.f : Sp * fexp2((Mp - RMp) * P.kT));
    const float SqT = row16_reduce<OP_SUM>(Mq == neg_inf() ? 0.f : Sq * fexp2((Mq - RMq) * P.kT));
    const int src = (lane & ~15) | (jx & 15);  // the lane that folded chunk jx
    zpx = __shfl(zpx, src, 64);
    zqx = __shfl(zqx, src, 64);
    if (live && l16 == 0) {
      if ((x < 0 || x >= V) && j == 0) flag(P.status, ADAFLASH_FLAG_BAD_TOKEN);
      const float px = fexp2((zpx - RMp) * P.kT) / SpT;
      const float qx = fexp2((zqx - RMq) * P.kT) / SqT;
      const bool accept = u * qx < px;
      s_acc[i] = accept ? 1 : 0;
      s_row[i][0] = RMp;
      s_row[i][1] = SpT;
      s_row[i][2] = RMq;
      s_row[i][3] = SqT;
      if (j == 0) {
        if (!(RMp < __builtin_inff()) || !(SpT > 0.f)) flag(P.status, ADAFLASH_FLAG_NONFINITE);
        pub_store(P.rowrec + (size_t)r * kRowRec + 1, accept ? 1.f : 0.f);
        pub_store(P.rowrec + (size_t)r * kRowRec + 2, px - u * qx);
        if (P.margins) P.margins[(size_t)b * (k + 1) + i] = px - u * qx;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const unsigned long long rej = __ballot(lane < L && s_acc[lane] == 0);
    if (lane == 0) s_first = rej ? __builtin_ctzll(rej) : L;
  }
  __syncthreads();
  const int A = s_first;
  const int je = min(G, RC * h + RC);
  for (int jb = RC * h; jb < je; jb += kResChunks) {
    if (jb > RC * h) __syncthreads();  // (red is read by thread 0 after the previous round)
    if (A < L) residual_of_chunks<BF16, ALIGNED>(P, b, A, jb, je, s_row, red, ep);
    else bonus_of_chunks<BF16, ALIGNED>(P, b, L, jb, je, red, ep);
  }
  // The last of the request's GH workgroups to arrive draws the correction or
  // bonus token, with the first rejection and its row's statistics already
  // known; it waits for each residual partial's epoch tag (the others count
  // their arrival without waiting for those stores).
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(P.rowcnt + (size_t)(r0 + k) * kCounterStride, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == GH - 1;
  }
  __syncthreads();
  if (s_last) {
    KnownRow kr;
    kr.A = A;
    kr.ep = ep;
    if (A < L) {
      kr.Mp = s_row[A][0];
      kr.SpT = s_row[A][1];
      kr.Mq = s_row[A][2];
      kr.SqT = s_row[A][3];
    }
    finalize_request<BF16, ALIGNED, 2, false, true>(P, b, fs, kr);
  }
}

// ----------------------------------------------------------- finalise kernel

// One workgroup per request, after the row kernel: first rejection, then the
// correction or bonus draw.
template <bool BF16, bool ALIGNED, int VMODE, bool LOG2REC = false>
__global__ __launch_bounds__(kThreads) void final_kernel(KParams P) {
  __shared__ FinShared fs;
  finalize_request<BF16, ALIGNED, VMODE, LOG2REC>(P, (int)blockIdx.x, fs);
}

// --------------------------------------------------------------- pack kernel

// One workgroup of 1024 threads: clamps the verify lengths, writes the packed
// row offsets (prefix sum: a scan inside each wave, then across the 16
// waves), clears the arrival counters and marks the accept flags as not yet
// known for the draft rows in use (the only rows that wait at a row barrier
// or whose flags are read), advances the workspace's call epoch and
// initialises the status word.
__global__ __launch_bounds__(1024) void pack_kernel(const int32_t* verify_len, int B, int k, int packed,
                                                     int32_t* row_offsets, Workspace ws, int32_t* status) {
  __shared__ int s_wave[16];
  __shared__ int s_flags;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_flags = 0;
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    int L = 0;
    if (b < B) {
      L = verify_len ? verify_len[b] : k;
      if (L < 1 || L > k) {
        atomicOr(&s_flags, ADAFLASH_FLAG_BAD_VERIFY_LEN);
        L = L < 1 ? 1 : k;
      }
      ws.Lc[b] = L;
    }
    int x = L;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(x, off, 64);
      if (lane >= off) x += t;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int t = s_wave[w];
      if (w < wave) woff += t;
      tot += t;
    }
    if (b < B) {
      const int off = carry + woff + x - L;
      row_offsets[b] = off;
      // Draft rows i < L: packed row map, arrival counter, accept flag (not
      // yet known).  Rows past L are never waited on or read.
      const size_t r0 = (size_t)b * (k + 1);
      ws.rowcnt[(r0 + k) * kCounterStride] = 0;  // the request's arrivals (verification alone)
      for (int q = 0; q < L; ++q) {
        ws.rowmap[off + q] = b * 64 + q;  // (k <= 64)
        ws.rowcnt[(r0 + q) * kCounterStride] = 0;
        ws.rowrec[(r0 + q) * kRowRec + 1] = 2.f;
      }
    }
    carry += tot;
    __syncthreads();
  }
  // Packed logits are located through the caller's own lengths: with one of
  // them out of range the rows cannot be found, so every request is marked
  // unusable (Lc = -1) and the row kernels read nothing.
  if (packed && s_flags)
    for (int b = tid; b < B; b += 1024) ws.Lc[b] = -1;
  if (tid == 0) {
    ws.epoch[0] += 1u;
    row_offsets[B] = carry;
    ws.Lc[B] = packed && s_flags ? 0 : carry;  // rows the row kernels run on
    if (status) *status = s_flags;
  }
}

// Measurement hook: while enabled on the calling thread, each call launches
// its dominant kernel (the first row kernel) with a pair of events attached
// to that dispatch, which take the kernel's own start and end times, so that
// a benchmark can time that kernel alone.
struct Timing {
  std::vector<hipEvent_t> ev;  // two per record
  int cap = 0, used = 0;
  int every = 1;  // events on every `every`-th dominant launch
  long long seen = 0;
};
thread_local Timing t_timing;

template <typename K>
hipError_t launch_dominant(K kernel, int grid, hipStream_t st, const KParams& p) {
  Timing& t = t_timing;
  if (t.used < t.cap && t.seen++ % t.every == 0) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, st, t.ev[2 * t.used], t.ev[2 * t.used + 1], 0, p);
    ++t.used;
  } else {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

template <bool BF16, bool ALIGNED, bool OPD, int VMODE, bool T1>
hipError_t launch_rows(const KParams& p, int grid, hipStream_t st) {
  return launch_dominant(row_kernel<BF16, ALIGNED, OPD, VMODE, T1>, grid, st, p);
}

template <bool BF16, bool ALIGNED, int VMODE, bool FKL = false>
hipError_t launch_sup(const KParams& p, int grid, hipStream_t st) {
  return launch_dominant(sup_kernel<BF16, ALIGNED, VMODE, FKL>, grid, st, p);
}

template <bool BF16, bool ALIGNED, int VMODE, bool LOG2REC = false>
hipError_t launch_final(const KParams& p, hipStream_t st) {
  hipLaunchKernelGGL((final_kernel<BF16, ALIGNED, VMODE, LOG2REC>), dim3(p.B), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <bool BF16, bool ALIGNED>
hipError_t dispatch_mode(const KParams& p, int grid, int opd, int vmode, bool t1, bool fkl, hipStream_t st) {
  hipError_t e;
  if constexpr (BF16 && ALIGNED) {
    // bf16 rows of a multiple of eight entries: the lighter supervision kernel.
    if (opd && (vmode == 0 || (vmode == 2 && t1)) && p.G <= 32) {
      const bool loose = p.clip_c >= kLooseClip;
      if (vmode == 0 && fkl) e = loose ? launch_dominant(fsup_kernel<0, true, true>, grid, st, p)
                                       : launch_dominant(fsup_kernel<0, true>, grid, st, p);
      else if (vmode == 0) e = loose ? launch_dominant(fsup_kernel<0, false, true>, grid, st, p)
                                     : launch_dominant(fsup_kernel<0>, grid, st, p);
      else e = loose ? launch_dominant(fsup_kernel<2, false, true>, grid, st, p)
                     : launch_dominant(fsup_kernel<2>, grid, st, p);
      if (e != hipSuccess || vmode == 0) return e;
      return launch_final<BF16, ALIGNED, 2, true>(p, st);
    }
  }
  if (opd && vmode == 0 && fkl) e = launch_sup<BF16, ALIGNED, 0, true>(p, grid, st);
  else if (opd && vmode == 0) e = launch_sup<BF16, ALIGNED, 0>(p, grid, st);
  else if (opd && vmode == 1) e = launch_sup<BF16, ALIGNED, 1>(p, grid, st);
  else if (opd && vmode == 2 && t1) e = launch_sup<BF16, ALIGNED, 2>(p, grid, st);
  else if (opd) e = launch_rows<BF16, ALIGNED, true, 2, false>(p, grid, st);
  else if (vmode == 1) {
    const int ng = (p.k + kGRows) / kGRows;
    e = launch_dominant(gstat_kernel<BF16, ALIGNED>, p.B * ng * p.G, st, p);
  }
  else if (vmode == 2) {
    // (draft positions only: B k slots)
    e = launch_dominant(vstat_kernel<BF16, ALIGNED>, p.B * p.k * p.G, st, p);
    if (e != hipSuccess) return e;
    // (vres_kernel draws as well)
    const int gh = (p.G + p.res_chunks - 1) / p.res_chunks;
    hipLaunchKernelGGL((vres_kernel<BF16, ALIGNED>), dim3(p.B * gh), dim3(kThreads), 0, st, p);
    return hipGetLastError();
  }
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  if (vmode == 1) return launch_final<BF16, ALIGNED, 1>(p, st);
  if (vmode == 2) return launch_final<BF16, ALIGNED, 2>(p, st);
  return hipSuccess;
}

}  // namespace

int timing_enable(int cap) {
  Timing& t = t_timing;
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.clear();
  t.cap = t.used = 0;
  t.every = 1;
  t.seen = 0;
  if (cap <= 0) return 0;
  t.ev.resize(2 * (size_t)cap, nullptr);
  for (auto& e : t.ev)
    if (hipEventCreate(&e) != hipSuccess) {
      timing_enable(0);
      return -1;
    }
  t.cap = cap;
  return 0;
}

int timing_every(int n) {
  if (n < 1) return -1;
  t_timing.every = n;
  t_timing.seen = 0;
  return 0;
}

int timing_read(float* ms, int cap) {
  Timing& t = t_timing;
  const int n = t.used < cap ? t.used : cap;
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms[i], t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess)
      return -1;
  }
  t.used = 0;
  return n;
}

hipError_t launch(const LaunchArgs& a) {
  const int bonus = a.verify ? 1 : 0;
  // Verification alone on padded logits needs none of the pack kernel's row
  // map, counters or flags: its first kernel does the rest of that work.
  const bool pack_here = a.verify && !a.opd && !a.packed && a.B > 0;
  if (!pack_here) {
    hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(1024), 0, a.stream, a.verify_len, a.B, a.k, a.packed,
                       a.row_offsets, a.ws, a.status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.B == 0) return e;
  }

  KParams p;
  p.target = a.target;
  p.draft = a.draft;
  p.tokens = a.tokens;
  p.uniforms = a.uniforms;
  p.accept_len = a.accept_len;
  p.out_tokens = a.out_tokens;
  p.margins = a.margins;
  p.row_offsets = a.row_offsets;
  p.loss_ce = a.loss_ce;
  p.loss_rkl = a.loss_rkl;
  p.grad = a.grad;
  p.status = a.status;
  p.Lc = a.ws.Lc;
  p.rowmap = a.ws.rowmap;
  p.rowcnt = a.ws.rowcnt;
  p.part1 = a.ws.part1;
  p.part2 = a.ws.part2;
  p.rowrec = a.ws.rowrec;
  p.epoch = a.ws.epoch;
  p.B = a.B;
  p.k = a.k;
  p.V = a.V;
  p.G = num_chunks(a.V);
  p.kT = a.T > 0.f ? kLog2e / a.T : 0.f;
  p.clip_c = a.clip_c;
  p.lambda = a.lambda;
  p.a_ce = a.a_ce;
  p.wdecay = a.wdecay;
  p.loss_var = a.loss_var;
  p.packed = a.packed;
  p.pack_here = pack_here;
  p.verify_len = a.verify_len;
  {
    // Residual workgroups of verification alone: enough chunks each that the
    // B requests' workgroups take two slots per CU (512), at least one
    // round.  At B = 128, V = 151936 that is four workgroups of five chunks
    // per request (129 us per verification call, against 132 with seven
    // workgroups of three, 132 with five of four, 131 with four of six and
    // 133 with two of ten).
    const long long want = ((long long)a.B * p.G + 511) / 512;
    p.res_chunks = (int)(want < kResChunks ? kResChunks : (want > p.G ? p.G : want));
  }

  const int vmode = a.verify ? (a.T > 0.f ? 2 : 1) : 0;
  const int rows_max = a.B * (a.k + bonus);
  const long long grid = (long long)rows_max * p.G;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int vec = a.bf16 ? 8 : 4;
  const bool aligned = (a.V % vec == 0) && (((uintptr_t)a.target & 15) == 0) &&
                       (a.draft == nullptr || ((uintptr_t)a.draft & 15) == 0) &&
                       (a.grad == nullptr || ((uintptr_t)a.grad & 15) == 0);
  const bool t1 = a.T == 1.0f;
  if (a.bf16) {
    if (aligned) return dispatch_mode<true, true>(p, (int)grid, a.opd, vmode, t1, a.fkl != 0, a.stream);
    return dispatch_mode<true, false>(p, (int)grid, a.opd, vmode, t1, a.fkl != 0, a.stream);
  }
  if (aligned) return dispatch_mode<false, true>(p, (int)grid, a.opd, vmode, t1, a.fkl != 0, a.stream);
  return dispatch_mode<false, false>(p, (int)grid, a.opd, vmode, t1, a.fkl != 0, a.stream);
}

}  // namespace adaflash
