// Internal interface between the C-ABI entry points (adaflash_api.cpp) and
// the gfx950 kernels (adaflash_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace adaflash {

// Workgroup size and elements of each logit row a thread keeps in registers.
constexpr int kThreads = 256;
#ifndef ADAFLASH_ELEMS
#define ADAFLASH_ELEMS 32  // entries of a row per thread (tuning: 32 or 64)
#endif
constexpr int kElems = ADAFLASH_ELEMS;
constexpr int kChunk = kThreads * kElems;  // elements of one row per workgroup

inline int num_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// Largest vocabulary and draft length the verify and supervision entry
// points accept.  The finaliser's per-wave steps hold one draft position and
// at most two chunk records of a row per lane.
constexpr int kMaxV = 1 << 20, kMaxK = 64;
static_assert((kMaxV + kChunk - 1) / kChunk <= 128, "at most two chunk records per lane");
static_assert(kMaxK <= 64, "one draft position per lane");

// Arrival counters sit 256 bytes apart so that no two share a cache line.
constexpr int kCounterStride = 64;
// Floats per published chunk record.
constexpr int kRec1 = 8, kRec2 = 4, kRowRec = 4;

// Device scratch carved out of the caller's workspace.  The record arrays
// have room for 64-bit fields (the bf16 supervision kernel tags every field
// with the call's epoch).
struct Workspace {
  uint32_t* epoch;   // [1] at offset 0: call counter, advanced once per call on the device
  int32_t* Lc;       // [B+1]  clamped verify lengths; Lc[B] = rows in use N (0: none usable)
  int32_t* rowmap;   // [B*k]  packed draft row n -> 64 b + i (request b, position i)
  int32_t* rowcnt;   // [B*(k+1)*kCounterStride] per-row arrival counters (zeroed per call)
  float* part1;      // [B*(k+1)*G*kRec1] per-chunk row statistics (64-bit fields: twice that)
  float* part2;      // [B*(k+1)*G*kRec2] per-chunk supervision / residual partials (likewise)
  float* rowrec;     // [B*(k+1)*kRowRec] per-row accept flag and margin
};

// Layout of the workspace for (B, k, V); returns the bytes needed.  With
// base == nullptr only the size is computed.
size_t workspace_layout(int B, int k, int V, char* base, Workspace* ws);

struct LaunchArgs {
  int bf16;               // 1: bf16 logits, 0: fp32
  const void* target;     // [B, k+1, V] (packed: [sum(L_b+1), V])
  const void* draft;      // [B, k, V] (packed: [sum L_b, V]; may be null for greedy verify without supervision)
  const int32_t* tokens;  // [B, k] (verify only)
  const int32_t* verify_len;  // [B] or null (= k)
  const float* uniforms;  // [B, k+1] (sampled verify only)
  int B, k, V;
  float T;                // verify temperature (0: greedy)
  int verify;             // 1: verify the batch
  int opd;                // 1: supervision outputs requested
  float clip_c, lambda;
  float a_ce = 1.f;       // weight of the hard-label term (loss variants)
  float wdecay = 0.f;     // per-position weight exp(-i / wdecay); 0 = none
  int fkl = 0;            // 1: forward KL(p || q) instead of the reverse KL
  float* loss_var = nullptr;  // [N] combined per-row loss of a variant, or null
  int packed = 0;         // 1: target [sum(L_b+1), V], draft [sum L_b, V] (rows in request order)
  int32_t* accept_len;
  int32_t* out_tokens;
  float* margins;
  int32_t* row_offsets;
  float* loss_ce;
  float* loss_rkl;
  void* grad;
  int32_t* status;
  Workspace ws;
  hipStream_t stream;
};

// Enqueues the pack kernel and the row kernel.  Returns hipSuccess or the
// launch error.
hipError_t launch(const LaunchArgs& a);

// Argument checks and launch of adaflash_verify (packed = 0) and
// adaflash_verify_packed (packed = 1) with a given workspace; returns an
// adaflash_status.  fail_with records the message adaflash_last_error returns.
int verify_impl(int packed, int dtype, const void* target_logits, const void* draft_logits,
                const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms, int B, int k, int V,
                float T, int32_t* accept_len, int32_t* out_tokens, float* margins, float clip_c, float lambda,
                int32_t* row_offsets, float* loss_ce, float* loss_rkl, void* grad_draft, int32_t* status_flags,
                void* workspace, size_t workspace_bytes, void* stream);
int fail_with(int code, const char* msg);

// Measurement hook (adaflash_timing_enable / adaflash_timing_read).
int timing_enable(int cap);
int timing_read(float* ms, int cap);
int timing_every(int n);

// Adaptive length head (adaflash_length_head.hip).
struct LhWorkspace {
  float* z1;         // [Sf, B*k, Hp] split-K slices of the projection h W1^T
  float* zsum;       // [B*k, Hp] their sum (when the caller keeps no copy)
  float* hbar;       // [B, Hp] pooled vectors (backward)
  float* ds;         // [B] d loss / d logit (backward)
  uint16_t* dzh;     // [ceil(B*k / 8), Hp, 8] dZ1 in blocks of eight rows, bf16 high part (backward)
  uint16_t* dzl;     // the same, bf16 remainder (backward)
  float* db1_part;   // [B, Hp] per-request column sums of dZ1 (for db1)
  float* dw_part;    // [Sb, Hp, H] split-K partial sums of dW1 (backward)
};

size_t lh_workspace_layout(int B, int k, int H, int Hp, char* base, LhWorkspace* ws);

// Output tiles of the length head's products: 64 x 64 for the projection
// (about 1024 workgroups), 64 x 128 for the weight gradient (about 128
// workgroups of four waves).  A reduction of length K is split over slices
// for `tiles` tiles and `wgs` workgroups wanted: slices a multiple of 64, at
// least 256 long and at most max_slice long.
constexpr int kLhFwdTile = 64;
constexpr int kLhTileR = 64, kLhTileC = 128;
struct LhSplit {
  int S, kslice;
};
LhSplit lh_split_k(int K, long long tiles, long long wgs, long long max_slice);
// The projection h W1^T (reduction over H, tiles of [B k x H']) and the
// weight gradient dZ1^T h (reduction over the B k rows, tiles of [H' x H],
// slices short enough for 32-bit buffer offsets).
LhSplit lh_split_fwd(int M, int H, int Hp);
LhSplit lh_split_bwd(int M, int H, int Hp);

struct LhArgs {
  const uint16_t* h;   // [B, k, H] bf16
  const uint16_t* W1;  // [Hp, H] bf16
  const float* b1;     // [Hp]
  const float* w2;     // [Hp]
  float b2, gamma;
  int B, k, H, Hp;
  float* a_hat;        // [B] or null
  int32_t* k_hat;      // [B] or null
  const int32_t* accept_len;  // [B]: backward when non-null
  const int32_t* verify_len;  // [B]
  float* loss;         // [B]
  float* dW1;          // [Hp, H]
  float* db1;          // [Hp]
  float* dw2;          // [Hp]
  float* db2;          // [1]
  float* z1_out = nullptr;        // forward: [B*k, Hp] projection h W1^T kept for the backward
  const float* z1_in = nullptr;   // backward: that projection, instead of recomputing it
  LhWorkspace ws;
  hipStream_t stream;
};

hipError_t lh_launch(const LhArgs& a);

}  // namespace adaflash
