// Pieces shared by the gfx950 forward kernels (fa_fwd.hip, fa_fwd8.hip):
// the work item of a workgroup and the boundary-block mask.  Internal to the
// library.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_kernels.h"
#include "tile_class.h"

namespace {

// Work item of this workgroup: (batch*head, first query row).
template <int ROWS_WG>
__device__ __forceinline__ void work_item(const FaFwdParams& p, int& bh, int& q0) {
  const int T = p.n_row_tiles;
  const int b = blockIdx.x;
  int rank;
  if (p.xcd_split) {
    const int hpx = p.BH >> 3;  // heads per XCD
    const int s = b >> 3;
    bh = (b & 7) * hpx + s % hpx;
    rank = s / hpx;
  } else {
    bh = b % p.BH;
    rank = b / p.BH;
  }
  const int qt = p.heavy_first ? (T - 1 - rank) : rank;
  q0 = qt * ROWS_WG;
}

// Tile k of a persistent workgroup: false when it has no k-th tile.  Within
// its group (blockIdx mod n_groups: the XCD when every XCD owns BH / 8
// heads) the tiles are numbered s = 0 .. tiles_per_group-1 as the plain
// launch orders its workgroups (longest first under a mask, heads fastest),
// and the group's J workgroups take them in a snake: round r covers s = rJ
// .. rJ+J-1, forwards on even rounds and backwards on odd ones, so a
// workgroup that drew a long tile next draws a short one.  Once a
// workgroup's s passes the end, every later one does too.
__device__ __forceinline__ bool persist_tile(const FaFwdParams& p, int k, int& bh, int& q0,
                                             int rows_wg) {
  const int g = blockIdx.x;
  const int x = g % p.n_groups, j = g / p.n_groups;
  const int J = p.wg_per_group;
  const int s = (k & 1) ? (k + 1) * J - 1 - j : k * J + j;
  if (s >= p.tiles_per_group) return false;
  const int T = p.n_row_tiles;
  int rank;
  if (p.n_groups > 1) {
    const int hpx = p.BH / p.n_groups;  // heads per group
    bh = x * hpx + s % hpx;
    rank = s / hpx;
  } else {
    bh = s % p.BH;
    rank = s / p.BH;
  }
  const int qt = p.heavy_first ? (T - 1 - rank) : rank;
  q0 = qt * rows_wg;
  return true;
}

// Boundary blocks: scores of invisible keys become -inf, which the
// exponential maps to exactly 0 (scale_log2 > 0).  s[kb][r] is the score of
// key k0 + 32kb + 8(r/4) + 4half + r%4 for query qi.
template <int NKB>
__device__ __forceinline__ void apply_mask(fa_f32x16 (&s)[NKB], int k0, int qi, int half, int N,
                                           int mask_kind, int window) {
  // row qi sees keys jlo..jhi; key j is visible iff 0 <= j - jlo <= span
  const int jhi = mask_kind == FA_MASKK_NONE ? N - 1 : min(qi, N - 1);
  const int jlo = mask_kind == FA_MASKK_SLIDING ? max(qi - window + 1, 0) : 0;
  const int base = k0 + 4 * half - jlo;
  const unsigned int span = (unsigned int)(jhi - jlo);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
      s[kb][r] = (unsigned int)(base + off) <= span ? s[kb][r] : FA_NEG_INF;
    }
}

}  // namespace
