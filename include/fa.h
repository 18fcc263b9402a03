/*
 * fa.h -- C ABI of the fused exact attention forward library (libfa.so),
 * gfx950 (MI355X) only.
 *
 * What is computed.  "FlashAttention (NL)", section "Problemen met standaard
 * attention", defines attention as softmax(Q K^T / sqrt(d_k)) V.  Sections
 * "Tiling en blokgewijze verwerking", "Online berekening van Softmax" and
 * "Samensmelting van bewerkingen in één CUDA-kernel" of the same page give
 * the method: Q, K, V are processed in blocks held in on-chip memory, a
 * running row maximum and a running sum of exponentials make the blockwise
 * softmax exact, and QK^T, masking, softmax and the product with V run in one
 * fused kernel that writes only the final result, so the N x N score matrix
 * never reaches device memory.  For every (b, h, i):
 *
 *   s_ij     = scale * <q[b,h,i,:], k[b,h,j,:]>      for visible j
 *   o[b,h,i] = sum_j exp(s_ij) v[b,h,j,:] / sum_j exp(s_ij)
 *   lse[b,h,i] = ln sum_j exp(s_ij)       (natural log, always fp32)
 *
 * lse is the online-softmax pair (running maximum m, exponent sum l) folded
 * into one number, m + ln l; it is what a backward pass would recompute the
 * probabilities from.
 *
 * Visibility of key j to query i (mask_kind):
 *   FA_MASK_NONE     every j in [0, N)
 *   FA_MASK_CAUSAL   j <= i
 *   FA_MASK_SLIDING  i - window < j <= i: the `window` most recent keys
 *                    including the query's own position (the local window of
 *                    the "Sparse Attention" glossary page, "Abgrenzung &
 *                    Vergleiche").  window >= N is the causal mask.
 *
 * Layout.  q, k, v, o: contiguous row-major [B][H][N][d] (d innermost).
 * lse: contiguous [B][H][N] float.  All pointers are device pointers (for
 * example from PyTorch), 16-byte aligned; outputs must not overlap inputs.
 *
 * Ownership and memory.  The caller owns every buffer.  The library
 * allocates no device memory and keeps no workspace: apart from o and lse
 * nothing of size O(N) or O(N^2) is written ("Complexiteit en optimaliteit":
 * memory O(N) instead of O(N^2)).
 *
 * Streams.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns once it is enqueued: outputs are valid after
 * the stream is synchronised.  The only global state is per-thread error
 * text, so calls from several host threads are safe.
 *
 * Errors.  Nothing is thrown or aborted across the ABI.  Arguments are
 * checked on the host before any HIP call, so a bad argument returns
 * FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED without touching the device.  A
 * HIP failure returns FA_ERR_HIP (or FA_ERR_NO_DEVICE) and fa_last_error()
 * holds the runtime's text.
 */
#ifndef FA_H_
#define FA_H_

#ifdef __cplusplus
extern "C" {
#endif

enum { FA_DTYPE_F32 = 0, FA_DTYPE_F16 = 1, FA_DTYPE_BF16 = 2,
       FA_DTYPE_E4M3 = 3 /* 8-bit float inputs of fa_fwd_fp8 only */ };
enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_SLIDING = 2 };
enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum, misalignment */
  FA_ERR_UNSUPPORTED = 2, /* valid request the library does not implement  */
  FA_ERR_NO_DEVICE = 3,   /* no usable gfx950 device                        */
  FA_ERR_HIP = 4          /* the HIP runtime reported an error              */
};

/*
 * Fused attention forward (the operation above).
 *   q, k, v    [B][H][N][d] of in_dtype
 *   o          [B][H][N][d] of out_dtype (out_dtype == in_dtype, or F32)
 *   lse        [B][H][N] float
 *   B, H, N    >= 1, with B*H*N*d < 2^62 and N < 2^30
 *   d          64 or 128, and 256 for F16/BF16 inputs (the head size that
 *              "FlashAttention (NL)", section "FlashAttention-2 (2023)",
 *              names among the extensions); else FA_ERR_UNSUPPORTED
 *   scale      finite and >= 0 (1/sqrt(d) in the page's formula; 0 gives
 *              uniform weights over the visible keys)
 *   mask_kind  FA_MASK_*; window >= 1 when FA_MASK_SLIDING, ignored otherwise
 *   in_dtype   FA_DTYPE_F32, FA_DTYPE_F16 or FA_DTYPE_BF16
 *   out_dtype  in_dtype or FA_DTYPE_F32 (F32 inputs need F32 output)
 *   stream     hipStream_t or NULL
 * Arithmetic: products on the matrix cores in the input precision with fp32
 * accumulation; softmax statistics in fp32; probabilities are rounded to the
 * input precision (round to nearest even) before the product with V, and O is
 * divided by the sum of those rounded weights.  lse uses the sum of the
 * unrounded probabilities with bf16 inputs and the sum of the rounded ones
 * with fp16 inputs (fp16 rounding moves it by at most 2^-11 relative, i.e.
 * lse by at most 4.9e-4).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int mask_kind, int window,
           int in_dtype, int out_dtype, void* stream);

/*
 * Same operation when several query heads share one key/value head: the
 * multi-query attention that "FlashAttention (NL)", section
 * "FlashAttention-2 (2023)", names among the extensions (H_kv = 1), and its
 * grouped form (1 <= H_kv <= H, H_kv divides H).  Query head h of batch
 * entry b attends with key/value head h / (H / H_kv) of that entry
 * (consecutive groups of H / H_kv query heads share one):
 *
 *   s_ij = scale * <q[b,h,i,:], k[b,h/g,j,:]>,   o and lse as above, g = H/H_kv
 *
 *   q, o, lse  [B][H][N][d], [B][H][N][d], [B][H][N] as in fa_fwd
 *   k, v       [B][H_kv][N][d] of in_dtype
 * Every other argument, the arithmetic and the errors are those of fa_fwd
 * (H_kv outside [1, H] or not dividing H: FA_ERR_INVALID_ARG).  fa_fwd is
 * this call with H_kv = H.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int mask_kind,
               int window, int in_dtype, int out_dtype, void* stream);

/*
 * Forward pass with 8-bit floating-point inputs: the FP8 precision that
 * "FlashAttention (NL)", section "FlashAttention-3 (2024)", names for the
 * Hopper version.  q, k, v hold OCP E4M3 codes (1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent field 0 is subnormal, m 2^-9;
 * S.1111.111 is NaN; no infinities; largest finite 448), the format of
 * gfx950's 8-bit matrix instructions and of torch.float8_e4m3fn.  With
 * x(c) the value of code c:
 *
 *   s_ij = scale * <x(q[b,h,i,:]), x(k[b,h/g,j,:])>     for visible j
 *   o[b,h,i] = v_scale * sum_j exp(s_ij) x(v[b,h/g,j,:]) / sum_j exp(s_ij)
 *   lse[b,h,i] = ln sum_j exp(s_ij)
 *
 * so per-tensor dequantisation factors fold into the call: scale = softmax
 * scale * q factor * k factor, v_scale = v factor.
 *   q [B][H][N][d], k, v [B][H_kv][N][d]: E4M3 bytes, no NaN codes
 *   o [B][H][N][d] of out_dtype (F32, F16 or BF16); lse [B][H][N] float
 *   d = 128 (else FA_ERR_UNSUPPORTED); v_scale finite (else
 *   FA_ERR_INVALID_ARG); H_kv, masks, scale, alignment, stream, ownership
 *   and errors as in fa_fwd_gqa.
 * Arithmetic: both products on the E4M3 matrix instructions with fp32
 * accumulation (the hardware sums the 64 products of one instruction to
 * about 2^-12 of the largest of them); softmax statistics in fp32; the
 * probabilities, scaled by 2^3 relative to the running reference, are rounded
 * to E4M3 (nearest even) before the product with V, and O is divided by the
 * fp32 sum of the unrounded ones.  Each weight therefore carries a relative
 * error up to 2^-4 (normal range), or an absolute one up to 2^-13 of the
 * largest weight of its row (subnormal range); lse is not affected by that
 * rounding.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, float v_scale,
               int mask_kind, int window, int out_dtype, void* stream);

/*
 * Decoding against a key/value cache: Nq queries per head at the last Nq
 * positions of a cache of Nk keys -- query i sits at position Nk - Nq + i
 * and sees the keys fa_fwd's mask gives that position (causal: j <= Nk - Nq
 * + i; sliding: the `window` keys up to it; none: all Nk).  Query head h
 * reads key/value head h / (H / H_kv), as in fa_fwd_gqa; Nq = Nk is fa_fwd_gqa.
 * The cache is split over the keys into chunks whose partial results
 * (normalised o and lse per chunk) go to `workspace` and are merged with the
 * online-softmax rescale of "FlashAttention (NL)", section "Online
 * berekening van Softmax"; streaming a KV cache during generation is the
 * workload of the engines named in section "Gespecialiseerde oplossingen".
 *   q, o       [B][H][Nq][d] of dtype;  lse [B][H][Nq] float
 *   k, v       [B][H_kv][Nk][d] of dtype
 *   1 <= Nq <= Nk < 2^30;  (H / H_kv) * Nq <= 32 (else FA_ERR_UNSUPPORTED)
 *   d          64 or 128;  dtype FA_DTYPE_F16 or FA_DTYPE_BF16
 *   workspace  device memory of at least fa_decode_workspace_bytes(...)
 *              bytes, 16-byte aligned, overlapping no other argument; its
 *              contents on entry do not matter and are left undefined.
 *              fa_decode_workspace_bytes bounds every mask_kind and window
 *              for the sizes given (-1 for invalid sizes)
 * Other arguments, arithmetic and errors as for fa_fwd.
 */
long long fa_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d);
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int H_kv, int Nq, int Nk, int d, float scale,
              int mask_kind, int window, int dtype, void* workspace,
              long long workspace_bytes, void* stream);

/*
 * fa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and arguments without the workspace.  The chunk partials
 * go to a file-scope device array of 8 MiB (FA_DECODE_SCRATCH_BYTES) that
 * every GPU the library runs on holds until the process ends.  The call
 * allocates nothing.  Sizes whose partials need more than 8 MiB
 * (fa_decode_workspace_bytes(...) > 8 MiB bounds them) return
 * FA_ERR_INVALID_ARG before any device call.  All calls on one GPU share its
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  Other arguments, arithmetic and
 * errors as for fa_decode.
 */
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int H_kv, int Nq, int Nk, int d, float scale,
                      int mask_kind, int window, int dtype, void* stream);

/*
 * Backward pass of fa_fwd: the gradients dq, dk, dv of o with respect to q,
 * k and v for an output gradient dout (of a loss L: dout = dL/do).  With
 * P_ij the attention weights of fa_fwd (0 where masked):
 *
 *   dP_ij   = <dout[b,h,i,:], v[b,h,j,:]>
 *   D_i     = sum_j P_ij dP_ij            (= <dout_i, o_i>)
 *   dS_ij   = P_ij (dP_ij - D_i)
 *   dq[b,h,i] = scale sum_j dS_ij k[b,h,j]
 *   dk[b,h,j] = scale sum_i dS_ij q[b,h,i]
 *   dv[b,h,j] = sum_i P_ij dout[b,h,i]
 *
 * P is recomputed tile by tile from q, k and the lse of the forward call
 * rather than stored (the recomputation of "Memory-Optimized Flash Attention
 * AI", section "How it works"); no N x N matrix is written.
 *   q, k, v    [B][H][N][d] of dtype: the forward call's inputs
 *   o, lse     the forward call's outputs ([B][H][N][d] of dtype, [B][H][N]
 *              float)
 *   dout       [B][H][N][d] of dtype
 *   dq, dk, dv [B][H][N][d] of dtype: results
 *   delta      [B][H][N] float, caller-owned workspace: receives D_i
 *   B, H, N, scale, mask_kind, window: as passed to fa_fwd
 *   d          64 or 128 (else FA_ERR_UNSUPPORTED)
 *   dtype      FA_DTYPE_F16 or FA_DTYPE_BF16 (F32: FA_ERR_UNSUPPORTED)
 * Results and delta must not overlap any input or each other; pointers
 * 16-byte aligned (lse, delta 4-byte).  Arithmetic: products on the matrix
 * cores in the input precision with fp32 accumulation; P and dS are rounded
 * to the input precision before the products that use them.  Work is
 * enqueued on `stream`; errors as for fa_fwd.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           float* delta, int B, int H, int N, int d, float scale,
           int mask_kind, int window, int dtype, void* stream);

/*
 * Backward pass of fa_fwd_gqa: the same gradients when query head h of batch
 * entry b reads key/value head h / (H / H_kv).  dq is per query head as in
 * fa_bwd; dk and dv of a key/value head sum, over the H / H_kv query heads
 * that read it, the terms fa_bwd would give each of them (the chain rule
 * through the shared operand):
 *
 *   dk[b,g,j] = scale sum_{h: h/(H/H_kv) = g} sum_i dS^h_ij q[b,h,i]
 *   dv[b,g,j] = sum_{h: h/(H/H_kv) = g} sum_i P^h_ij dout[b,h,i]
 *
 *   k, v, dk, dv  [B][H_kv][N][d] of dtype; every other argument as in fa_bwd
 *   H_kv          1 <= H_kv <= H, dividing H (else FA_ERR_INVALID_ARG)
 * A key/value head's dk, dv accumulate in fp32 over all of its query heads
 * and are rounded once.  With 8 or more query heads per key/value head and
 * fewer than four dk/dv workgroups (one per key/value head and 128 keys) per
 * compute unit, the query heads of a key tile are split over up to
 * (H / H_kv) / 4 workgroups whose fp32 partial sums are kept in dq's memory
 * until a final kernel adds them (dq is written afterwards): the sum order,
 * and so the last bit of dk and dv, depends on that split.  fa_bwd is this
 * call with H_kv = H.
 */
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv,
               float* delta, int B, int H, int H_kv, int N, int d, float scale,
               int mask_kind, int window, int dtype, void* stream);

/*
 * Tile geometry the dispatcher uses for (d, in_dtype): rows handled by one
 * workgroup, rows handled by one wavefront (the granularity at which work is
 * skipped), and keys per K/V block.  Host only; no device call.
 */
int fa_tile_shape(int d, int in_dtype, int* rows_per_workgroup,
                  int* rows_per_wave, int* keys_per_block);

/*
 * Host-side tile map for (N, d, in_dtype, mask_kind, window): out[rb * C + kb]
 * = FA_TILE_SKIP / FA_TILE_FULL / FA_TILE_PARTIAL (0 / 1 / 2) for row block
 * rb (rows_per_wave rows) and key block kb (keys_per_block keys), with
 * R = ceil(N / rows_per_wave) and C = ceil(N / keys_per_block).  `out` is
 * host memory of R*C bytes.  No device call.  (fa_fwd_record_tiles in
 * fa_diag.h records the decisions the kernel itself takes.)
 */
int fa_tile_map(int N, int d, int in_dtype, int mask_kind, int window,
                unsigned char* out);

/* Name of a status code ("FA_OK", ...).  Static storage. */
const char* fa_status_string(int status);

/* Detail text of the last failing call on this host thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
