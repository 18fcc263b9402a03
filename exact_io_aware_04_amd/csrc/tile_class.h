// Integer tile classification for the fused attention forward pass.
//
// The tiled method of "FlashAttention (NL)", section "Tiling en blokgewijze
// verwerking", walks Q in row blocks and K/V in key blocks; masking happens
// inside the fused kernel (section "Samensmelting van bewerkingen in één
// CUDA-kernel").  A (row block, key block) pair is then in one of three
// states, decided here with integer range tests only:
//   FA_TILE_SKIP    no (query, key) pair in the block is visible: never visited
//   FA_TILE_FULL    every pair is visible: computed with no per-element mask
//   FA_TILE_PARTIAL some pairs are visible: per-element mask applied
// Visibility of key j to query i: none -> j < N; causal -> j <= i; sliding ->
// i - window < j <= i (the local window of the "Sparse Attention" glossary
// page, "Abgrenzung & Vergleiche").  Keys at or beyond N never exist.
//
// Used by the host (tile map export, argument checks) and by the kernels.
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

enum { FA_TILE_SKIP = 0, FA_TILE_FULL = 1, FA_TILE_PARTIAL = 2 };
enum { FA_MASKK_NONE = 0, FA_MASKK_CAUSAL = 1, FA_MASKK_SLIDING = 2 };

// Rows [r0, r1) (already clipped to N, r0 < r1) against keys [c0, c0 + bc).
FA_HD int fa_classify(int r0, int r1, int c0, int bc, int N, int mask_kind,
                      int window) {
  if (r0 >= r1 || c0 >= N) return FA_TILE_SKIP;
  const int c1 = c0 + bc;          // exclusive end before clipping to N
  const bool tail = c1 > N;        // some keys of the block do not exist
  const int cl = tail ? N : c1;    // exclusive end of existing keys
  if (mask_kind == FA_MASKK_NONE) return tail ? FA_TILE_PARTIAL : FA_TILE_FULL;
  // causal part: some pair j <= i  <=>  c0 <= r1 - 1
  if (c0 > r1 - 1) return FA_TILE_SKIP;
  bool all = (cl - 1 <= r0);       // every existing key <= the smallest row
  if (mask_kind == FA_MASKK_SLIDING) {
    // union of the rows' windows is [r0 - window + 1, r1 - 1]
    if (cl - 1 < r0 - window + 1) return FA_TILE_SKIP;
    all = all && (c0 >= r1 - window);  // c0 >= (r1 - 1) - window + 1
  }
  return (all && !tail) ? FA_TILE_FULL : FA_TILE_PARTIAL;
}

// Key-block range [*lo, *hi) (in blocks of bc keys) that holds any key
// visible to some row of [r0, r1).
FA_HD void fa_key_block_range(int r0, int r1, int bc, int N, int mask_kind,
                              int window, int* lo, int* hi) {
  const int nb = (N + bc - 1) / bc;
  if (r0 >= r1) {
    *lo = 0;
    *hi = 0;
    return;
  }
  if (mask_kind == FA_MASKK_NONE) {
    *lo = 0;
    *hi = nb;
    return;
  }
  int h = (r1 - 1) / bc + 1;  // block holding key r1 - 1, plus one
  *hi = h < nb ? h : nb;
  if (mask_kind == FA_MASKK_SLIDING) {
    const int first = r0 - window + 1;  // oldest key visible to row r0
    *lo = first > 0 ? first / bc : 0;
  } else {
    *lo = 0;
  }
}
