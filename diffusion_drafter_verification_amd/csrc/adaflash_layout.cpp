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

LhSplit lh_split_k(int K, long long tiles) {
  if (tiles < 1) tiles = 1;  // (an empty product)
  const long long want = (1024 + tiles - 1) / tiles;
  const long long maxs = K / 256 > 0 ? K / 256 : 1;
  int S = (int)(want < 1 ? 1 : (want > maxs ? maxs : want));
  int ks = (K + S - 1) / S;
  ks = (ks + 63) & ~63;  // whole 64-wide rounds of the products
  S = K > 0 ? (K + ks - 1) / ks : 1;
  return {S, ks};
}

size_t lh_workspace_layout(int B, int k, int H, int Hp, char* base, LhWorkspace* ws) {
  const size_t M = (size_t)B * k;
  const size_t Hq = ((size_t)Hp + 7) & ~size_t(7);
  const LhSplit sf = lh_split_k(H, lh_tiles((long long)M, Hp));
  const LhSplit sb = lh_split_k((int)M, lh_tiles(Hp, H));
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
  char* dzh = take(sizeof(uint16_t) * M * Hq);
  char* dzl = take(sizeof(uint16_t) * M * Hq);
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
