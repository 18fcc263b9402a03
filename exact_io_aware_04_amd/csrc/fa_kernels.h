// Internal interface between the host API (fa_api.cpp) and the gfx950
// kernels (fa_fwd.hip, fa_fwd8.hip, fa_bwd.hip, fa_decode.hip).  Not part
// of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

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
