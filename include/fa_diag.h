/*
 * Diagnostics and host-side planners of the attention library (the same
 * shared object as include/fa.h): a forward that also records its tile
 * decisions, the work order and backward split the launches use, and two
 * device probes of the matrix core.  None of them is needed to compute
 * attention; they expose what the kernels do so that it can be checked.
 * Status codes, dtype and mask codes as in include/fa.h.
 */
#ifndef FA_DIAG_H_
#define FA_DIAG_H_

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Same as fa_fwd, and records the tile decisions the kernel took: for every
 * (b, h), row block rb of tile_rows rows and key block kb of tile_keys keys
 * (see fa_tile_shape), tiles[((b*H + h) * R + rb) * C + kb] is set to
 * FA_TILE_* + 1 (1 skipped, 2 full, 3 partial) by the wave that owns the
 * row block, with R = ceil(N / tile_rows) and C = ceil(N / tile_keys).  The
 * caller zero-fills `tiles` (B*H*R*C bytes, device memory) beforehand;
 * entries of key blocks outside the workgroup's visited range stay 0.  A
 * diagnostic for the tile-skip structure; not for timing.
 */
int fa_fwd_record_tiles(const void* q, const void* k, const void* v, void* o,
                        float* lse, int B, int H, int N, int d, float scale,
                        int mask_kind, int window, int in_dtype, int out_dtype,
                        unsigned char* tiles, void* stream);

/*
 * Host-side export of the forward's work order (no device call): which row
 * tiles each workgroup of the fa_fwd / fa_fwd_gqa / fa_fwd_fp8 launch for
 * (B, H, H_kv, N, d, in_dtype, mask_kind, window) takes (H_kv = H for
 * fa_fwd and fa_fwd_fp8; window read only for the sliding mask), on a
 * device with `compute_units` compute units, in the order it takes them.  A row tile is
 * rows_per_workgroup query rows (fa_tile_shape) of one (batch, head) slice.
 * *n_workgroups receives the grid size G and *max_tiles the largest number
 * R of tiles any workgroup takes (R = 1 where each workgroup takes one
 * tile: f32 inputs, d = 256).  With `out` non-null (host memory of
 * out_len >= 2*G*R ints) out[2(g*R + k)] and out[2(g*R + k) + 1] receive the
 * batch*head index and the row tile index of workgroup g's k-th tile, or
 * -1 and -1 after its last one.  Every row tile appears exactly once.  The
 * order is a performance choice (load balance, L2 reuse of each head's
 * keys and values), never a numerical one: each tile's output depends on
 * its own rows only.  FA_ERR_INVALID_ARG for sizes < 1, N >= 2^30, H not
 * a multiple of H_kv, a bad enum, a sliding window < 1, a null
 * n_workgroups or max_tiles, or out_len < 2*G*R with out non-null;
 * FA_ERR_UNSUPPORTED for a head dim not built for in_dtype.
 */
int fa_fwd_schedule(int B, int H, int H_kv, int N, int d, int in_dtype, int mask_kind,
                    int window, int compute_units, int* n_workgroups, int* max_tiles, int* out,
                    long long out_len);

/*
 * Split of the backward's dk/dv pass that fa_bwd_gqa chooses on a device
 * with `compute_units` compute units: *parts receives the number of
 * workgroups each 128-key tile's query heads are divided over (1: no split).
 * The split is taken when a group has g = H / H_kv >= 8 query heads and the
 * B * H_kv * ceil(N / 128) tiles give fewer than four workgroups per compute
 * unit; then parts = min(g / 4, ceil(4 * compute_units / tiles)).  Host
 * only; no device call.  FA_ERR_INVALID_ARG for B, H, N, compute_units < 1,
 * N >= 2^30, an H_kv that does not divide H, or a null `parts`.
 */
int fa_bwd_kv_parts(int B, int H, int H_kv, int N, int compute_units, int* parts);

/*
 * Diagnostic: one 32x32 output block of a matrix-core product, to check the
 * operand and accumulator lane layouts the kernels rely on.  which = 0:
 * bf16 32x32x16; 1: f16 32x32x16; 2: f32 32x32x2; 3: E4M3 32x32x64.  a and
 * b are device pointers to 64 lanes x (8 for which 0/1, 1 for which 2, 32
 * bytes for which 3) elements in lane order, d a device pointer to 64 lanes
 * x 16 floats in lane order.  which = 4 checks the transposing LDS byte
 * read instead: a holds 512 bytes, lane l addresses byte 8l, and d receives
 * the 8 bytes each lane gets back (64 lanes x 8 floats; b must be non-null
 * and is not read).  The kernel is launched on `stream` with one
 * wavefront.
 */
int fa_probe_mfma(int which, const void* a, const void* b, float* d,
                  void* stream);

/*
 * Diagnostic: the matrix-core ceiling of this device.  Launches n_blocks
 * workgroups of 256 threads (two per CU fill every SIMD twice); each
 * wavefront issues iters x 8 independent bf16 32x32x16 products (32768 FLOP
 * each) and touches no memory in between.  clocks (device, n_blocks x 4
 * u64): per workgroup the shader clock counter before / after the loop and
 * the 100 MHz real-time counter before / after.  sink (device, n_blocks x
 * 256 floats) receives the accumulators so the work is not optimised away.
 * Sustained FLOP/s = n_blocks * 4 * iters * 8 * 32768 / elapsed time; shader
 * clock = clock delta / real-time delta * 100 MHz.
 */
int fa_mfma_ceiling(int n_blocks, int iters, unsigned long long* clocks, float* sink,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_DIAG_H_ */
