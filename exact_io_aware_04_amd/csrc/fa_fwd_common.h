// Pieces shared by the gfx950 forward kernels (fa_fwd.hip, fa_fwd8.hip):
// the work item of a workgroup and the boundary-block mask.  Internal to the
// library.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_kernels.h"
#include "tile_class.h"

namespace {

// Work item of this workgroup in the plain launch: (batch*head, first row).
template <int ROWS_WG>
__device__ __forceinline__ void work_item(const FaFwdParams& p, int& bh, int& q0) {
  int qt;
  fa_plain_tile_of(p, blockIdx.x, &bh, &qt);
  q0 = qt * ROWS_WG;
}

// Tile k of this persistent workgroup (order: fa_persist_tile_of).
__device__ __forceinline__ bool persist_tile(const FaFwdParams& p, int k, int& bh, int& q0,
                                             int rows_wg) {
  int qt;
  if (!fa_persist_tile_of(p, blockIdx.x, k, &bh, &qt)) return false;
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
