// Internal interface between the host API (fa_api.cpp) and the gfx950
// kernels (fa_fwd.hip, fa_fwd8.hip, fa_bwd.hip, fa_decode.hip).  Not part
// of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "tile_class.h"

struct FaFwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  unsigned char* tiles;   // optional tile-decision record (nullptr: off)
  int BH;                 // batch * heads
  int kv_group;           // query heads per key/value head (H / H_kv); the
                          // K/V slice of query slice bh is bh / kv_group
  int N;                  // sequence length
  int mask_kind;          // FA_MASKK_*
  int window;             // sliding window (keys), >= 1 when sliding
  float scale_log2;       // scale * log2(e)
  float v_scale;          // E4M3 inputs: factor applied to O (1 otherwise)
  int n_row_tiles;        // ceil(N / rows_per_workgroup)
  int xcd_split;          // 1: give each XCD its own heads (BH % 8 == 0)
  int heavy_first;        // 1: longest row tiles launched first (masks)
  // Persistent launches (the 16-bit kernel at d <= 128): n_groups groups of
  // wg_per_group workgroups (grid n_groups * wg_per_group); group x = blockIdx
  // mod n_groups takes tiles_per_group tiles (8 groups: the XCDs, each with
  // its own BH / 8 heads; 1 group: all tiles).
  int n_groups;
  int wg_per_group;
  int tiles_per_group;
  int kv_major;           // numbering of a group's row tiles: 0 heads fastest,
                          // 1 K/V head by K/V head, 2 window teams
  int kv_share;           // query heads of one K/V head within a group (numbered
                          // fastest under kv_major = 1)
  int team;               // kv_major = 2: workgroups per team (window / rows per
                          // workgroup)
};

// Backward pass (fa_bwd.hip).
struct FaBwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;       // gradient of the loss with respect to o
  const float* lse;
  float* delta;           // [BH][N]: receives <dout_i, o_i>
  void* dq;
  void* dk;
  void* dv;
  int BH;                 // batch * query heads
  int kv_group;           // query heads per key/value head (H / H_kv): query
                          // slice bh reads key/value slice bh / kv_group
  int N;
  int mask_kind;
  int window;
  float scale;
  float scale_log2;       // scale * log2(e), at least FLT_MIN
  int n_q_tiles;          // ceil(N / (FA_BWD_DQ_WAVES * 32)): query tiles of the dq pass
  int n_k_tiles;          // ceil(N / (FA_BWD_WAVES * 32)): key tiles of the dk/dv pass
  int heavy_first;        // 1: longest query tiles of the dq pass first (masks)
  int kv_parts;           // dk/dv workgroups per key tile: part j of kv_parts takes
                          // query heads [j g / kv_parts, (j + 1) g / kv_parts) of
                          // the g = kv_group heads that share the key/value head
  float* part_scratch;    // kv_parts > 1: fp32 partial sums of dk (not yet times
                          // scale) and then of dv, each [kv_parts][BH / kv_group][N][d]
};
constexpr int FA_BWD_WAVES = 4;     // wavefronts per workgroup, dk/dv pass (one per SIMD)
constexpr int FA_BWD_DQ_WAVES = 8;  // wavefronts per workgroup, dq pass (two per SIMD)

// Decoding against a key/value cache (fa_decode.hip).
struct FaDecodeParams {
  const void* q;          // [B][H][Nq][D]
  const void* k;          // [B][H_kv][Nk][D]
  const void* v;
  void* o;                // [B][H][Nq][D]
  float* lse;             // [B][H][Nq]
  float* ws;              // [n_chunks][rows][D] partial o, then [n_chunks][rows] partial lse
  int H;
  int H_kv;
  int group;              // H / H_kv
  int Nq;
  int Nk;
  int mask_kind;
  int window;
  float scale_log2;
  int kb_lo;              // first 32-key block any query sees
  int n_blocks;           // 32-key blocks from kb_lo to the end of the cache
  int chunk_blocks;       // blocks per chunk
  int n_chunks;
  int n_items;            // B * H_kv * n_chunks work items (one wavefront each)
  long long rows;         // B * H * Nq
};
constexpr int FA_DECODE_KEYS = 32;
constexpr int FA_DECODE_WAVES = 3;
// Bytes of the file-scope device array that fa_decode_noalloc uses for the
// chunk partials in place of a caller's workspace (8 MiB per GPU, held until
// the process ends).
constexpr long long FA_DECODE_SCRATCH_BYTES = 8LL << 20;
// Device address of that array on the current device (looked up once per
// device, with the device current, by hipGetSymbolAddress).
hipError_t fa_decode_scratch(void** ptr);

// Tile geometry.  Work is skipped per row block of 32 query rows (one
// 32x32 matrix-core tile of rows); each wavefront owns one row block.
constexpr int FA_ROW_BLOCK = 32;         // query rows per row block
constexpr int FA_WAVES_32 = 4;           // wavefronts per workgroup, f32
constexpr int FA_WAVES_16 = 8;           // wavefronts per workgroup, f16/bf16
constexpr int FA_WAVES_WIDE = 4;         // wavefronts per workgroup, f16/bf16 at d = 256
constexpr int FA_KEYS_16 = 64;           // keys per K/V block, f16/bf16
constexpr int FA_KEYS_32 = 32;           // keys per K/V block, f32
constexpr int FA_KEYS_8 = 64;            // keys per K/V block, E4M3
constexpr int FA_STAGES_16 = 3;          // depth of the K and V rings in LDS, f16/bf16

// Input dtype codes: 0 f32, 1 f16, 2 bf16 (as in fa.h), 3 E4M3 (fa_fwd_fp8).
constexpr int FA_DT_E4M3 = 3;

// keys per K/V block for an input dtype code (0 = f32) and head dim
constexpr int fa_keys_per_block(int in_dtype, int d) {
  return in_dtype == 0 ? FA_KEYS_32 : FA_KEYS_16;
}

// query rows per workgroup for an input dtype code (0 = f32) and head dim
constexpr int fa_rows_per_wg(int in_dtype, int d) {
  return (in_dtype == 0 ? FA_WAVES_32 : d == 256 ? FA_WAVES_WIDE : FA_WAVES_16) * FA_ROW_BLOCK;
}

// The forward launches with one persistent workgroup per compute unit: the
// f16/bf16 kernel at d = 64 and 128 and the E4M3 kernel (d = 128).  The
// fp32 and d = 256 kernels are launched with one workgroup per row tile.
constexpr bool fa_fwd_persistent(int in_dtype, int d) {
  return (in_dtype == 1 || in_dtype == 2 || in_dtype == FA_DT_E4M3) && d <= 128;
}

// Work order of the forward, shared by the host (launch plan, schedule
// export) and the kernels.
//
// Plain launch: workgroup b takes one row tile.  With every XCD owning its
// own BH / 8 heads (xcd_split; blockIdx b runs on XCD b mod 8) the tiles
// of XCD x are numbered s = b / 8 with heads fastest; otherwise s = b over
// all heads.  Rank s / heads is the tile's place in launch order; under a
// mask the longest row tiles (highest qt) go first.
FA_HD void fa_plain_tile_of(const FaFwdParams& p, int b, int* bh, int* qt) {
  const int T = p.n_row_tiles;
  int rank;
  if (p.xcd_split) {
    const int hpx = p.BH >> 3;
    const int s = b >> 3;
    *bh = (b & 7) * hpx + s % hpx;
    rank = s / hpx;
  } else {
    *bh = b % p.BH;
    rank = b / p.BH;
  }
  *qt = p.heavy_first ? (T - 1 - rank) : rank;
}

// Persistent launch: tile k of workgroup g, false when g has no k-th tile.
// Within its group (g mod n_groups: the XCD when every XCD owns BH / 8
// heads) the tiles are numbered s = 0 .. tiles_per_group-1 and the group's
// J workgroups take them in a snake: round r covers s = rJ .. rJ+J-1,
// forwards on even rounds and backwards on odd ones, so a workgroup that
// drew a long tile next draws a short one.  Numbering (row tiles longest
// first under a mask):
//   kv_major = 0: heads fastest, s = rank * heads + head.  Every prefix is
//     sorted longest first, which balances any mix of tile lengths.
//   kv_major = 1: the group's heads form sets of G = kv_share query heads
//     that read one K/V head; s = set * G T + rank * G + head in set.  The
//     J tiles of a round then read one K/V head (or whole sets when G T <
//     J), start together and stream the same key/value blocks, so the
//     group's L2 serves most of them from one fetch; the rank changes every
//     G tiles, so a round also holds tiles of similar length.  Balanced when
//     every pair of snake rounds pairs position t with 2J-1-t at equal
//     summed length: no mask, or causal with G T a multiple or divisor of
//     2J.  (G = heads per group gives the kv_major = 0 order.)
//   kv_major = 2 (sliding window of S row tiles exactly, S = team): no
//     snake.  The group's J workgroups form J / S teams of S; team t takes
//     heads t, t + J/S, ... in turn, and member i of a team takes the row
//     tiles of a head with rank = i mod S, one after the other.  With D =
//     row tile / key block, a tile of rank r >= S reads key blocks
//     (r - S) D .. (r + 1) D - 1 and a tile of rank r < S blocks
//     0 .. (r + 1) D - 1.  On even heads of the team member i takes ranks
//     i, i + S, i + 2S, ...: its first tile ends after (i + 1) D blocks,
//     when its next one (from block i D on) reads the block every other
//     member reads at that moment, so the whole team streams the same
//     key/value block at the same time from then on and the L2 serves it
//     from one fetch.  On odd heads member i takes ranks i + S, i + 2S, ...
//     and last rank S - 1 - i: it starts i D blocks after member 0 and its
//     first tile i D blocks further in (aligned again); its last tile is
//     (S - i) D blocks long, so that every member's two heads add to the
//     same number of blocks.  Needs an even number of heads per team and T
//     a multiple of S.
// Once a workgroup's s passes the end, every later one does too.
FA_HD bool fa_persist_tile_of(const FaFwdParams& p, int g, int k, int* bh, int* qt) {
  const int x = g % p.n_groups, j = g / p.n_groups;
  const int J = p.wg_per_group;
  const int T = p.n_row_tiles;
  const int hpg = p.BH / p.n_groups;  // heads per group
  if (p.kv_major == 2) {
    const int S = p.team, n_team = J / S, M = T / S;  // M: tiles per head and member
    const int team = j / S, i = j - team * S;
    const int hh = k / M, kk = k - hh * M;
    if (hh >= hpg / n_team) return false;
    *bh = x * hpg + hh * n_team + team;
    *qt = !(hh & 1) ? i + kk * S : (kk < M - 1 ? i + (kk + 1) * S : S - 1 - i);
    return true;
  }
  const int s = (k & 1) ? (k + 1) * J - 1 - j : k * J + j;
  if (s >= p.tiles_per_group) return false;
  int head, rank;
  if (p.kv_major) {
    const int G = p.kv_share, per = G * T;
    const int set = s / per, r = s - set * per;
    rank = r / G;
    head = set * G + (r - rank * G);
  } else {
    rank = s / hpg;
    head = s - rank * hpg;
  }
  *bh = x * hpg + head;
  *qt = p.heavy_first ? (T - 1 - rank) : rank;
  return true;
}

// Plan of a forward launch on a device with `cus` compute units: sets
// xcd_split, heavy_first and, for the persistent launch, one workgroup per
// compute unit (fewer when there are fewer tiles), a multiple of the 8
// groups when every XCD owns its own heads, and the numbering.  Requires
// BH, kv_group, N, window (sliding) and n_row_tiles = ceil(N / rows_wg);
// key blocks of FA_KEYS_16 (= FA_KEYS_8) keys.
inline void fa_fwd_plan(FaFwdParams& p, int mask_kind, int cus, int rows_wg) {
  p.xcd_split = (p.BH % 8 == 0) ? 1 : 0;
  p.heavy_first = mask_kind != FA_MASKK_NONE ? 1 : 0;
  const long long total = (long long)p.BH * p.n_row_tiles;
  p.n_groups = p.xcd_split ? 8 : 1;
  long long g = total < cus ? total : cus;
  g = g / p.n_groups * p.n_groups;
  if (g < p.n_groups) g = p.n_groups;
  p.wg_per_group = (int)(g / p.n_groups);
  p.tiles_per_group = (int)(total / p.n_groups);
  // Query heads of a group that read one K/V head: the group's heads start
  // at a multiple of hpg and K/V heads change every kv_group heads, so sets
  // of gcd(kv_group, hpg) consecutive heads each read one K/V head.
  int a = p.kv_group, b = p.BH / p.n_groups;
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  p.kv_share = a;
  // K/V head by K/V head when that keeps the snake balanced: tiles of one
  // length (no mask), or causal lengths with G T and 2J dividing one
  // another.  Sliding windows keep heads fastest: their short tiles sit at
  // each head's start and must spread over all workgroups.
  const long long GT = (long long)p.kv_share * p.n_row_tiles, J2 = 2LL * p.wg_per_group;
  p.kv_major = mask_kind == FA_MASKK_NONE ||
               (mask_kind == FA_MASKK_CAUSAL && (GT % J2 == 0 || J2 % GT == 0));
  // Sliding windows of a whole number S of row tiles (and row tiles of a
  // whole number of key blocks, N a multiple of the row tile): window teams
  // when the workgroups split into teams of S, every team gets an even
  // number of heads and every head S-aligned ranks (fa_persist_tile_of).
  p.team = 0;
  if (mask_kind == FA_MASKK_SLIDING && rows_wg % FA_KEYS_16 == 0 && p.window % rows_wg == 0 &&
      p.N % rows_wg == 0) {
    const int S = p.window / rows_wg, J = p.wg_per_group, hpg = p.BH / p.n_groups;
    if (S >= 1 && J % S == 0 && hpg % (2 * (J / S)) == 0 && p.n_row_tiles % S == 0 &&
        (long long)J * (hpg / (J / S)) * (p.n_row_tiles / S) == (long long)p.tiles_per_group) {
      p.kv_major = 2;
      p.team = S;
    }
  }
}

// head dims built for an input dtype code: 64 and 128, 256 for f16/bf16,
// 128 only for E4M3
constexpr bool fa_head_dim_built(int in_dtype, int d) {
  if (in_dtype == FA_DT_E4M3) return d == 128;
  return d == 64 || d == 128 || (d == 256 && in_dtype != 0);
}

// dtype codes as in fa.h
hipError_t fa_launch_fwd(int in_dtype, int out_dtype, int d,
                         const FaFwdParams& p, hipStream_t stream);
hipError_t fa_launch_fwd8(int out_dtype, int d, const FaFwdParams& p, hipStream_t stream);
hipError_t fa_launch_probe8(int which, const void* a, const void* b, float* d,
                            hipStream_t stream);
hipError_t fa_launch_bwd(int in_dtype, int d, const FaBwdParams& p, hipStream_t stream);
hipError_t fa_launch_decode(int in_dtype, int d, const FaDecodeParams& p, hipStream_t stream);
hipError_t fa_launch_probe(int which, const void* a, const void* b, float* d,
                           hipStream_t stream);
hipError_t fa_launch_mfma_ceiling(int n_blocks, int iters, unsigned long long* clk, float* sink,
                                  hipStream_t stream);
