// Workspace layouts of the entry points (host code): where each device
// scratch array sits in the caller's workspace, and how many bytes it takes.
#include <stddef.h>
#include <stdint.h>

#include "adaflash_internal.h"

namespace adaflash {
namespace {

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t workspace_layout(int B, int k, int V, char* base, Workspace* ws) {
  const size_t rows = (size_t)B * (k + 1);
  const size_t G = (size_t)num_chunks(V);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return base ? base + at : nullptr;
  };
  char* epoch = take(sizeof(uint32_t));  // first: at the same place for every (B, k, V)
  char* Lc = take(sizeof(int32_t) * (size_t)(B + 1));
  char* rowmap = take(sizeof(int32_t) * (rows > 0 ? (size_t)B * k : 1));
  char* rowcnt = take(sizeof(int32_t) * kCounterStride * (rows > 0 ? rows : 1));
  char* part1 = take(sizeof(uint64_t) * kRec1 * (rows > 0 ? rows : 1) * G);
  char* part2 = take(sizeof(uint64_t) * kRec2 * (rows > 0 ? rows : 1) * G);
  char* rowrec = take(sizeof(float) * kRowRec * (rows > 0 ? rows : 1));
  if (ws) {
    ws->epoch = (uint32_t*)epoch;
    ws->Lc = (int32_t*)Lc;
    ws->rowmap = (int32_t*)rowmap;
    ws->rowcnt = (int32_t*)rowcnt;
    ws->part1 = (float*)part1;
    ws->part2 = (float*)part2;
    ws->rowrec = (float*)rowrec;
  }
  return off;
}

LhSplit lh_split_k(int K, long long tiles, long long wgs, long long max_slice) {
  if (tiles < 1) tiles = 1;  // (an empty product)
  const long long want = (wgs + tiles - 1) / tiles;
  const long long maxs = K / 256 > 0 ? K / 256 : 1;
  int S = (int)(want < 1 ? 1 : (want > maxs ? maxs : want));
  long long ks = ((long long)K + S - 1) / S;
  ks = (ks + 63) & ~63LL;  // whole 64-deep blocks
  const long long cap = max_slice & ~63LL;
  if (ks > cap) ks = cap > 64 ? cap : 64;
  S = K > 0 ? (int)((K + ks - 1) / ks) : 1;
  return {S, (int)ks};
}

static long long lh_tiles(long long rows, long long cols, int tr, int tc) {
  return ((rows + tr - 1) / tr) * ((cols + tc - 1) / tc);
}

LhSplit lh_split_fwd(int M, int H, int Hp) {
  return lh_split_k(H, lh_tiles(M, Hp, kLhFwdTile, kLhFwdTile), 1024, H);
}

LhSplit lh_split_bwd(int M, int H, int Hp) {
  // A slice of h is kslice rows of 2 H bytes, of dZ1 kslice / 8 blocks of 16 Hp bytes: at most 2^30 bytes each.
  const long long wide = H > Hp ? H : Hp;
  // About 128 workgroups: at B k = 2048, H' = 256, H = 4096 a single slice,
  // written straight to dW1 (no slice sum); two or more slices measured
  // slower per step.
  return lh_split_k(M, lh_tiles(Hp, H, kLhTileR, kLhTileC), 128, (1LL << 29) / wide);
}

size_t lh_workspace_layout(int B, int k, int H, int Hp, char* base, LhWorkspace* ws) {
  const size_t M = (size_t)B * k;
  const size_t M8 = (M + 7) & ~size_t(7);
  const LhSplit sf = lh_split_fwd((int)M, H, Hp);
  const LhSplit sb = lh_split_bwd((int)M, H, Hp);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return base ? base + at : nullptr;
  };
  char* z1 = take(sizeof(float) * sf.S * M * Hp);
  char* zsum = take(sizeof(float) * M * Hp);
  char* hbar = take(sizeof(float) * (size_t)B * Hp);
  char* ds = take(sizeof(float) * (size_t)B);
  char* dzh = take(sizeof(uint16_t) * M8 * Hp);
  char* dzl = take(sizeof(uint16_t) * M8 * Hp);
  char* part = take(sizeof(float) * (size_t)B * Hp);
  char* dwp = take(sizeof(float) * sb.S * (size_t)Hp * H);
  if (ws) {
    ws->z1 = (float*)z1;
    ws->zsum = (float*)zsum;
    ws->hbar = (float*)hbar;
    ws->ds = (float*)ds;
    ws->dzh = (uint16_t*)dzh;
    ws->dzl = (uint16_t*)dzl;
    ws->db1_part = (float*)part;
    ws->dw_part = (float*)dwp;
  }
  return off;
}

}  // namespace adaflash
