// Fused attention backward pass for gfx950 (MI355X, CDNA4): the gradients
// dq, dk, dv of o = softmax(scale q k^T + mask) v for an output gradient do.
//
// The method: intermediate results are recomputed when they are needed
// rather than stored ("Memory-Optimized Flash Attention AI", section "How it
// works").  Here the probabilities P are recomputed tile by tile from q, k
// and the lse the forward pass wrote (the running maximum and exponent sum of
// "FlashAttention (NL)", section "Online berekening van Softmax", folded into
// one number), so no N x N matrix is read or written.  With
//   dP = do v^T,  D_i = sum_j P_ij dP_ij = <do_i, o_i>,  dS = P (dP - D):
//   dq = scale dS k,   dk = scale dS^T q,   dv = P^T do.
// Kernels, launched in this order on one stream:
//   fa_bwd_delta_kernel   D_i = <do_i, o_i> in fp32, one pass over do and o
//   fa_bwd_dkdv_kernel    per 128-key tile, over its query blocks (of the
//                         query heads that share the key/value head, or of
//                         one part of them): S, dP, dS, dv^T += do^T P,
//                         dk^T += q^T dS (lane = key)
//   fa_bwd_combine_kernel only when a tile's query heads are split over
//                         several workgroups: adds their fp32 partials,
//                         which sit in dq's memory
//   fa_bwd_dq_kernel      per 256-row query tile, over its key blocks:
//                         S^T, dP^T, dS^T, dq^T += k^T dS^T (lane = query);
//                         last, since it overwrites that memory
// S and dP are formed in both loop kernels (seven matrix products per
// query-block / key-block pair instead of five), so that no partial dq is
// accumulated across workgroups.
//
// gfx950 mapping: wavefronts of 64 lanes with 32 rows (or keys) each -- 8
// per workgroup, two per SIMD, for dq; 4, one per SIMD with the two
// accumulator sets in AGPRs, for dk/dv; the resident operands (q and do rows,
// or k and v rows) stay in VGPRs as matrix-core fragments, the streamed
// blocks (k and v, or q and do) go HBM -> LDS directly (buffer_load_dwordx4
// with the LDS destination), double-buffered.  Every streamed block is read
// both as 16-byte row pieces (score operands) and transposed by
// ds_read_b64_tr_b16 (gradient operands); one 16-byte chunk swizzle serves
// both without bank conflicts (see bswz).
#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_kernels.h"
#include "tile_class.h"

namespace {

constexpr int BW = FA_BWD_WAVES;      // wavefronts per workgroup, dk/dv pass
constexpr int BWQ = FA_BWD_DQ_WAVES;  // wavefronts per workgroup, dq pass
constexpr int BR = 32;            // rows (or keys) per wavefront
constexpr int BB = 64;            // rows (or keys) per streamed block
constexpr float LOG2E = 1.44269504088896340736f;
#define FA_BWD_GRAD_AHEAD 6       // dk/dv gradient products: operand reads ahead

// Chunk swizzle of a streamed block row r (chunk position = chunk ^ bswz(r)).
// 16-byte row reads take one chunk of 16 consecutive rows per 16 lanes;
// transposing reads take 4 chunks of 4 consecutive rows per half wavefront.
// d = 128 (16 chunks, rows start on one bank): 4(r mod 4) sends the 4 rows of
// a transposing read to different 4-chunk groups and (r / 4) mod 4 completes
// a permutation of 16 over 16 rows.  d = 64 (8 chunks, rows alternate between
// two bank halves): the same with row r / 2 of each half.
template <int D>
__device__ __forceinline__ int bswz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Query-block range [lo, hi) (blocks of bq rows) holding every query that
// sees some key of [k0, k1): none -> all; causal -> i >= k0; sliding ->
// k0 <= i <= k1 - 2 + window.
__device__ __forceinline__ void query_block_range(int k0, int k1, int bq, int N, int mask_kind,
                                                  int window, int* lo, int* hi) {
  const int nb = (N + bq - 1) / bq;
  if (k0 >= k1 || k0 >= N) {
    *lo = *hi = 0;
  } else if (mask_kind == FA_MASKK_NONE) {
    *lo = 0;
    *hi = nb;
  } else if (mask_kind == FA_MASKK_CAUSAL) {
    *lo = k0 / bq;
    *hi = nb;
  } else {
    *lo = k0 / bq;
    const long long last = min((long long)N - 1, (long long)k1 - 2 + window);
    *hi = (int)(last / bq) + 1;
  }
}

// Byte offsets of this lane's reads of a streamed block (any 32-row group):
// rowrd[s]: 16-byte piece of row l32, chunk 2s + half (a score operand);
// trlo[cb], trhi[cb]: transposing 8-byte reads at rows 4 half + t and
// 8 + 4 half + t, columns 32 cb + 16 (g mod 2) + 4 q .. + 3 (a gradient
// operand: lane (column, half) receives the 8 rows that match the P^T / dS^T
// operands built from the score accumulators).
template <int D>
struct ReadOffsets {
  unsigned rowrd[D / 16], trlo[D / 32], trhi[D / 32];
  __device__ __forceinline__ ReadOffsets(int lane) {
    constexpr int ROWB = 2 * D;
    const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) rowrd[s] = l32 * ROWB + 16 * ((2 * s + half) ^ bswz<D>(l32));
    const int g = lane >> 4, t = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int c = 4 * cb + 2 * (g & 1) + (q >> 1);
      const int rl = 4 * half + t, rh = rl + 8;
      trlo[cb] = rl * ROWB + 16 * (c ^ bswz<D>(rl)) + 8 * (q & 1);
      trhi[cb] = rh * ROWB + 16 * (c ^ bswz<D>(rh)) + 8 * (q & 1);
    }
  }
};

// Transposed operand (32 columns x 16 rows) of block rows rbase .. rbase+15.
__device__ __forceinline__ fa_u32x4 tr_operand(const FA_AS3 unsigned char* blk, unsigned lo,
                                               unsigned hi) {
  const fa_i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)(blk + lo));
  const fa_i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)(blk + hi));
  const fa_u32x2 x = __builtin_bit_cast(fa_u32x2, a), y = __builtin_bit_cast(fa_u32x2, b);
  return fa_u32x4{x.x, x.y, y.x, y.y};
}

// Block of 64 rows starting at row r0 of a [N][D] matrix -> LDS (rows past N
// read as zeros).  Each of the NW wavefronts loads every NW-th kilobyte;
// piece i lies NW kilobytes (a multiple of 16 rows) further, which leaves
// bswz unchanged, so one global offset per lane serves all pieces.
template <int D, int NW>
__device__ __forceinline__ void load_block(const unsigned char* base, int r0, int N, unsigned off,
                                           FA_AS3 unsigned char* dst, int wave) {
  constexpr int ROWB = 2 * D, TILEB = BB * ROWB, LPW = TILEB / (NW * 1024);
  static_assert(LPW >= 1 && LPW * NW * 1024 == TILEB, "pieces must cover the block");
  // (wave-uniform, and held in scalar registers: a byte count left in a
  // vector register makes the descriptor per-lane, and each load a loop)
  const int nb = __builtin_amdgcn_readfirstlane(max(min(N - r0, BB), 0) * ROWB);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (r0 < N ? (size_t)r0 * ROWB : 0)), 0, nb, FA_BUF_WORD3);
#pragma unroll
  for (int i = 0; i < LPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_AS3 void*)(dst + (i * NW + wave) * 1024), 16,
                                             (int)off, i * NW * 1024, 0, 0);
}

template <int D>
__device__ __forceinline__ unsigned load_offset(int wave, int lane) {
  constexpr int ROWB = 2 * D;
  const int o = wave * 1024 + 16 * lane;
  const int r = o / ROWB, pos = (o % ROWB) / 16;
  return r * ROWB + 16 * (pos ^ bswz<D>(r));
}

// Fragment slices of one [D] row (16 bytes at 32 s + 16 half): the B operand
// of a product whose output columns are rows of that matrix.
template <int D>
__device__ __forceinline__ void row_fragments(const unsigned char* row, int half, fa_u32x4 (&f)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = *(const fa_u32x4*)(row + s * 32 + half * 16);
}

// Transposed accumulators (32 columns per block x 32 rows) -> rows of a
// [N][D] matrix in the 16-bit type, times `mul`.
template <int DT, int D>
__device__ __forceinline__ void store_rows(void* out, size_t row, const fa_f32x16 (&acc)[D / 32],
                                           float mul, int half) {
  unsigned char* dst = (unsigned char*)out + row * D * 2;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = cb * 32 + 8 * g + 4 * half;
      *(fa_u32x2*)(dst + c * 2) = pack4<DT>(acc[cb][4 * g] * mul, acc[cb][4 * g + 1] * mul,
                                            acc[cb][4 * g + 2] * mul, acc[cb][4 * g + 3] * mul);
    }
}

// The same accumulators as fp32 (row = 32-bit elements of one [D] row).
template <int D>
__device__ __forceinline__ void store_rows_f32(float* dst, const fa_f32x16 (&acc)[D / 32], int half) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = cb * 32 + 8 * g + 4 * half;
      *(fa_f32x4*)(dst + c) = fa_f32x4{acc[cb][4 * g], acc[cb][4 * g + 1], acc[cb][4 * g + 2],
                                       acc[cb][4 * g + 3]};
    }
}

// ---------------------------------------------------------------------------
// D_i = <do_i, o_i>
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ void __launch_bounds__(256) fa_bwd_delta_kernel(FaBwdParams p) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements (16 bytes) each
  constexpr int RPB = 256 / LPR;
  const long long rows = (long long)p.BH * p.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = ((size_t)row * D + c * 8) * 2;
    const fa_u32x4 a = *(const fa_u32x4*)((const unsigned char*)p.dout + off);
    const fa_u32x4 b = *(const fa_u32x4*)((const unsigned char*)p.o + off);
    if constexpr (DT == 2) {
      const fa_bf16x8 x = __builtin_bit_cast(fa_bf16x8, a), y = __builtin_bit_cast(fa_bf16x8, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (float)x[i] * (float)y[i];
    } else {
      const fa_f16x8 x = __builtin_bit_cast(fa_f16x8, a), y = __builtin_bit_cast(fa_f16x8, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (float)x[i] * (float)y[i];
    }
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && c == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dq: one workgroup per (batch*head, 256-row query tile); eight wavefronts,
// two per SIMD (the hardware overlaps one's VALU work with the other's
// matrix products), sharing each K/V block in LDS
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ void __launch_bounds__(BWQ * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_bwd_dq_kernel(FaBwdParams p) {
  constexpr int NKB = BB / 32, NCB = D / 32, NQF = D / 16, ROWB = 2 * D, TILEB = BB * ROWB;
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILEB], ks1[TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[TILEB], vs1[TILEB];
  auto kbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? ks0 : ks1); };
  auto vbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? vs0 : vs1); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int N = p.N;
  const int bh = blockIdx.x % p.BH, rank = blockIdx.x / p.BH;
  const int qt = p.heavy_first ? p.n_q_tiles - 1 - rank : rank;
  const int q0 = qt * BWQ * BR, q1 = min(q0 + BWQ * BR, N);
  const int qb0 = q0 + wave * BR, qb1 = min(qb0 + BR, N);
  const int qi = qb0 + l32, qr = min(qi, N - 1);

  // query slice bh reads key/value slice bh / g (g = H / H_kv)
  const size_t head = (size_t)bh * N * ROWB;
  const size_t kvhead = (size_t)(bh / p.kv_group) * N * ROWB;
  const unsigned char* Qh = (const unsigned char*)p.q + head;
  const unsigned char* Kh = (const unsigned char*)p.k + kvhead;
  const unsigned char* Vh = (const unsigned char*)p.v + kvhead;
  const unsigned char* dOh = (const unsigned char*)p.dout + head;

  fa_u32x4 qf[NQF], dof[NQF];
  row_fragments<D>(Qh + (size_t)qr * ROWB, half, qf);
  row_fragments<D>(dOh + (size_t)qr * ROWB, half, dof);
  const float lse2 = p.lse[(size_t)bh * N + qr] * LOG2E;
  const float dlt = p.delta[(size_t)bh * N + qr];
  const float c2 = p.scale_log2;

  int kv_lo, kv_hi;
  fa_key_block_range(q0, q1, BB, N, p.mask_kind, p.window, &kv_lo, &kv_hi);
  const unsigned loff = load_offset<D>(wave, lane);
  const ReadOffsets<D> rd(lane);

  fa_f32x16 acc[NCB];  // dq^T: acc[cb] holds columns 32cb.., row qi
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  load_block<D, BWQ>(Kh, kv_lo * BB, N, loff, kbuf(0), wave);
  load_block<D, BWQ>(Vh, kv_lo * BB, N, loff, vbuf(0), wave);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto step = [&](int kt, int s) {
    if (kt + 1 < kv_hi) {
      load_block<D, BWQ>(Kh, (kt + 1) * BB, N, loff, kbuf(s ^ 1), wave);
      load_block<D, BWQ>(Vh, (kt + 1) * BB, N, loff, vbuf(s ^ 1), wave);
    }
    const int cls = fa_classify(qb0, qb1, kt * BB, BB, N, p.mask_kind, p.window);
    if (cls != FA_TILE_SKIP) {
      const FA_AS3 unsigned char* kc = kbuf(s);
      const FA_AS3 unsigned char* vc = vbuf(s);
      // S^T = K Q^T and dP^T - D = V dO^T - D (keys x rows)
      fa_f32x16 sc[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[kb][r] = 0.f;
          dp[kb][r] = -dlt;
        }
#pragma unroll
      for (int sl = 0; sl < NQF; ++sl)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const fa_u32x4 ka = *(const FA_AS3 fa_u32x4*)(kc + kb * 32 * ROWB + rd.rowrd[sl]);
          const fa_u32x4 va = *(const FA_AS3 fa_u32x4*)(vc + kb * 32 * ROWB + rd.rowrd[sl]);
          sc[kb] = mma16<DT>(ka, qf[sl], sc[kb]);
          dp[kb] = mma16<DT>(va, dof[sl], dp[kb]);
        }
      // P^T = 2^(s c2 - lse log2 e), 0 where masked; dS^T = P^T (dP^T - D)
      // (s[kb][r] is key kt*64 + 32kb + 8(r/4) + 4half + r%4 of row qi)
      // (boundary blocks: one wave-uniform branch around the mask, so the
      // dq accumulators see one code path)
      float pr[NKB][16];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[kb][r] = exp2_hw(__builtin_fmaf(sc[kb][r], c2, -lse2));
      if (cls == FA_TILE_PARTIAL) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kt * BB + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            // visible under the mask (bitwise operators: no branches)
            const bool vis = (j < N) & ((p.mask_kind == FA_MASKK_NONE) |
                                        ((j <= qi) & ((p.mask_kind == FA_MASKK_CAUSAL) |
                                                      (j > qi - p.window))));
            pr[kb][r] = vis ? pr[kb][r] : 0.f;
          }
      }
      fa_u32x4 dsf[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = pr[kb][r] * dp[kb][r];
        dsf[kb][0] = pack8<DT>(&ds[0]);
        dsf[kb][1] = pack8<DT>(&ds[8]);
      }
      // dq^T += K^T dS^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const FA_AS3 unsigned char* blk = kc + (32 * kb + 16 * t) * ROWB;
            acc[cb] = mma16<DT>(tr_operand(blk, rd.trlo[cb], rd.trhi[cb]), dsf[kb][t], acc[cb]);
          }
    }
    __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(0));
    barrier_nofence();
  };
  for (int kt = kv_lo;;) {
    step(kt, 0);
    if (++kt >= kv_hi) break;
    step(kt, 1);
    if (++kt >= kv_hi) break;
  }
  if (qi < N) store_rows<DT, D>(p.dq, (size_t)bh * N + qi, acc, p.scale, half);
}

// ---------------------------------------------------------------------------
// dk, dv: one workgroup per (batch*head, 128-key tile)
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ void __launch_bounds__(BW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
fa_bwd_dkdv_kernel(FaBwdParams p) {
  constexpr int NQB = BB / 32, NCB = D / 32, NQF = D / 16, ROWB = 2 * D, TILEB = BB * ROWB;
  __shared__ __attribute__((aligned(1024))) unsigned char qs0[TILEB], qs1[TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char os0[TILEB], os1[TILEB];
  __shared__ __attribute__((aligned(256))) float ls[2][BB], dl[2][BB];  // -lse log2 e, D
  auto qbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? qs0 : qs1); };
  auto obuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? os0 : os1); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int N = p.N;
  // key/value slice bkv; the query slices bkv g .. bkv g + g - 1 read it, and
  // this workgroup takes those of part `part` (low key tiles, which see the
  // most queries, come first)
  const int BHkv = p.BH / p.kv_group;
  const int bkv = blockIdx.x % BHkv, rest = blockIdx.x / BHkv;
  const int part = rest % p.kv_parts, kt = rest / p.kv_parts;
  const int j_lo = part * p.kv_group / p.kv_parts, j_hi = (part + 1) * p.kv_group / p.kv_parts;
  const int k0 = kt * BW * BR, k1 = min(k0 + BW * BR, N);
  const int kw0 = k0 + wave * BR;
  const int kj = kw0 + l32, kr = min(kj, N - 1);

  const size_t kvhead = (size_t)bkv * N * ROWB;
  const unsigned char* Kh = (const unsigned char*)p.k + kvhead;
  const unsigned char* Vh = (const unsigned char*)p.v + kvhead;
  const unsigned char* Qh;
  const unsigned char* dOh;
  const float* lse_h;
  const float* dl_h;

  fa_u32x4 kf[NQF], vf[NQF];
  row_fragments<D>(Kh + (size_t)kr * ROWB, half, kf);
  row_fragments<D>(Vh + (size_t)kr * ROWB, half, vf);
  const float c2 = p.scale_log2;

  int qlo, qhi;
  query_block_range(k0, k1, BB, N, p.mask_kind, p.window, &qlo, &qhi);
  const unsigned loff = load_offset<D>(wave, lane);
  const ReadOffsets<D> rd(lane);

  fa_f32x16 dva[NCB], dka[NCB];  // dv^T, dk^T: columns 32cb.., key kj
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) dva[cb][r] = dka[cb][r] = 0.f;
    asm volatile("" : "+a"(dva[cb]));  // placement only: the matrix core's AGPRs
    asm volatile("" : "+a"(dka[cb]));
  }

  // query block qt -> slot b: q and do rows, and lse and D of its 64 rows
  // (one 4-byte load per lane by waves 0 and 1).  Rows past N read as zeros
  // and contribute nothing below, since their q and do rows are zero.  D
  // goes to LDS by DMA; lse arrives in a register of wave 0 (lane = row)
  // and is stored to LDS as -lse log2 e by put_lse before the barrier that
  // ends the step, so the exponent below is one FMA per score
  float lse_next = 0.f;
  auto load = [&](int qt, int b) {
    load_block<D, BW>(Qh, qt * BB, N, loff, qbuf(b), wave);
    load_block<D, BW>(dOh, qt * BB, N, loff, obuf(b), wave);
    const int r0 = qt * BB;
    if (wave == 0) {
      lse_next = r0 + lane < N ? lse_h[r0 + lane] : 0.f;
    } else if (wave == 1) {
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(dl_h + (r0 < N ? r0 : 0)), 0,
          __builtin_amdgcn_readfirstlane(max(min(N - r0, BB), 0) * 4), FA_BUF_WORD3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_AS3 void*)&dl[b][0], 4, lane * 4, 0, 0, 0);
    }
  };
  auto put_lse = [&](int b) {
    if (wave == 0) ls[b][lane] = -lse_next * LOG2E;
  };
  auto step = [&](int qt, int s) {
    if (qt + 1 < qhi) load(qt + 1, s ^ 1);
    const int cls = fa_classify(qt * BB, min(qt * BB + BB, N), kw0, BR, N, p.mask_kind, p.window);
    if (cls != FA_TILE_SKIP) {
      const FA_AS3 unsigned char* qc = qbuf(s);
      const FA_AS3 unsigned char* oc = obuf(s);
      // S = Q K^T and dP = dO V^T (rows x keys); s[qb][r] is row
      // qt*64 + 32qb + 8(r/4) + 4half + r%4 and key kj
      fa_f32x16 sc[NQB], dp[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[qb][r] = dp[qb][r] = 0.f;
#pragma unroll
      for (int sl = 0; sl < NQF; ++sl)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const fa_u32x4 qa = *(const FA_AS3 fa_u32x4*)(qc + qb * 32 * ROWB + rd.rowrd[sl]);
          const fa_u32x4 oa = *(const FA_AS3 fa_u32x4*)(oc + qb * 32 * ROWB + rd.rowrd[sl]);
          sc[qb] = mma16<DT>(qa, kf[sl], sc[qb]);
          dp[qb] = mma16<DT>(oa, vf[sl], dp[qb]);
        }
      // P = 2^(s c2 - lse log2 e), 0 where masked: boundary blocks take one
      // (wave-uniform) branch around the mask of all 64 rows, which leaves
      // the gradient accumulators untouched (one code path for them, so the
      // register allocator keeps them in place)
      float pr[NQB][16];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const fa_f32x4 l4 = *(const FA_AS3 fa_f32x4*)&ls[s][32 * qb + 8 * a + 4 * half];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pr[qb][4 * a + e] = exp2_hw(__builtin_fmaf(sc[qb][4 * a + e], c2, l4[e]));
        }
      if (cls == FA_TILE_PARTIAL) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = qt * BB + 32 * qb + 8 * (r >> 2) + 4 * half + (r & 3);
            // visible under the mask (bitwise operators: no branches)
            const bool vis = (kj < N) & ((p.mask_kind == FA_MASKK_NONE) |
                                         ((kj <= i) & ((p.mask_kind == FA_MASKK_CAUSAL) |
                                                       (kj > i - p.window))));
            pr[qb][r] = vis ? pr[qb][r] : 0.f;
          }
      }
      // dS = P (dP - D)
      fa_u32x4 pf[NQB][2], dsf[NQB][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float ds[16];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const fa_f32x4 d4 = *(const FA_AS3 fa_f32x4*)&dl[s][32 * qb + 8 * a + 4 * half];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ds[4 * a + e] = pr[qb][4 * a + e] * (dp[qb][4 * a + e] - d4[e]);
        }
        pf[qb][0] = pack8<DT>(&pr[qb][0]);
        pf[qb][1] = pack8<DT>(&pr[qb][8]);
        dsf[qb][0] = pack8<DT>(&ds[0]);
        dsf[qb][1] = pack8<DT>(&ds[8]);
      }
      // dv^T += dO^T P, dk^T += Q^T dS.  Product j: (qb, t, cb) = j / 2, dv
      // (j even) or dk (j odd); its transposed operand is read R products
      // ahead, so the wave (alone on its SIMD) does not wait out the LDS
      // latency before every product.  The group barriers keep that order.
      {
        constexpr int R = FA_BWD_GRAD_AHEAD, NG = 2 * NQB * 2 * NCB;
        fa_u32x4 op[R + 1];
#pragma unroll
        for (int i = 0; i < NG + R; ++i) {
          if (i < NG) {
            const int g = i / 2, cb = g % NCB, t = (g / NCB) % 2, qb = g / NCB / 2;
            const int rb = (32 * qb + 16 * t) * ROWB;
            op[i % (R + 1)] = tr_operand((i & 1 ? qc : oc) + rb, rd.trlo[cb], rd.trhi[cb]);
          }
          if (i >= R) {
            const int j = i - R, g = j / 2, cb = g % NCB, t = (g / NCB) % 2, qb = g / NCB / 2;
            if (j & 1)
              dka[cb] = mma16<DT>(op[j % (R + 1)], dsf[qb][t], dka[cb]);
            else
              dva[cb] = mma16<DT>(op[j % (R + 1)], pf[qb][t], dva[cb]);
          }
        }
#pragma unroll
        for (int i = 0; i < NG + R; ++i) {
          if (i < NG) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          if (i >= R) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }
    if (qt + 1 < qhi) put_lse(s ^ 1);
    __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(0));
    barrier_nofence();
  };
  // every query slice of the part in turn, all into the same dk, dv (the
  // last step of a slice ends with a barrier, so its slots are free)
  for (int j = j_lo; j < j_hi; ++j) {
    const int bh = bkv * p.kv_group + j;
    const size_t head = (size_t)bh * N * ROWB;
    Qh = (const unsigned char*)p.q + head;
    dOh = (const unsigned char*)p.dout + head;
    lse_h = p.lse + (size_t)bh * N;
    dl_h = p.delta + (size_t)bh * N;
    load(qlo, 0);
    put_lse(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int qt = qlo;;) {
      step(qt, 0);
      if (++qt >= qhi) break;
      step(qt, 1);
      if (++qt >= qhi) break;
    }
  }
  if (kj >= N) return;
  if (p.kv_parts == 1) {
    store_rows<DT, D>(p.dk, (size_t)bkv * N + kj, dka, p.scale, half);
    store_rows<DT, D>(p.dv, (size_t)bkv * N + kj, dva, 1.f, half);
  } else {
    const size_t plane = (size_t)p.kv_parts * BHkv * N * D;  // floats per tensor
    const size_t row = ((size_t)part * BHkv + bkv) * N + kj;
    store_rows_f32<D>(p.part_scratch + row * D, dka, half);
    store_rows_f32<D>(p.part_scratch + plane + row * D, dva, half);
  }
}

// dk, dv = the sums of the kv_parts fp32 partials (dk times scale), rounded
// once to the input type; thread t takes 8 consecutive elements of dk (first
// half of the grid) or dv (second half)
template <int DT>
__global__ void __launch_bounds__(256) fa_bwd_combine_kernel(FaBwdParams p, long long n8) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= 2 * n8) return;
  const bool is_dv = t >= n8;
  const long long e = (is_dv ? t - n8 : t) * 8;     // element index in [BHkv][N][d]
  const size_t plane = (size_t)p.kv_parts * n8 * 8;  // floats per tensor
  const float* src = p.part_scratch + (is_dv ? plane : 0) + e;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < p.kv_parts; ++j) {
    const fa_f32x4 a = *(const fa_f32x4*)(src + (size_t)j * n8 * 8);
    const fa_f32x4 b = *(const fa_f32x4*)(src + (size_t)j * n8 * 8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += a[i];
      acc[4 + i] += b[i];
    }
  }
  const float mul = is_dv ? 1.f : p.scale;
  unsigned char* dst = (unsigned char*)(is_dv ? p.dv : p.dk) + e * 2;
  *(fa_u32x2*)dst = pack4<DT>(acc[0] * mul, acc[1] * mul, acc[2] * mul, acc[3] * mul);
  *(fa_u32x2*)(dst + 8) = pack4<DT>(acc[4] * mul, acc[5] * mul, acc[6] * mul, acc[7] * mul);
}

template <int DT, int D>
hipError_t launch_bwd(const FaBwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.BH * p.N;
  const unsigned dgrid = (unsigned)((rows + 256 / (D / 8) - 1) / (256 / (D / 8)));
  hipLaunchKernelGGL((fa_bwd_delta_kernel<DT, D>), dim3(dgrid), dim3(256), 0, stream, p);
  // dk/dv (and the sum of its partials) before dq: with kv_parts > 1 the
  // partials live in dq's memory, which the dq pass then overwrites
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<DT, D>),
                     dim3((unsigned)(p.BH / p.kv_group * p.n_k_tiles * p.kv_parts)), dim3(BW * 64),
                     0, stream, p);
  if (p.kv_parts > 1) {
    const long long n8 = (long long)(p.BH / p.kv_group) * p.N * D / 8;
    hipLaunchKernelGGL((fa_bwd_combine_kernel<DT>), dim3((unsigned)((2 * n8 + 255) / 256)), dim3(256),
                       0, stream, p, n8);
  }
  hipLaunchKernelGGL((fa_bwd_dq_kernel<DT, D>), dim3((unsigned)(p.BH * p.n_q_tiles)), dim3(BWQ * 64),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t fa_launch_bwd(int in_dtype, int d, const FaBwdParams& p, hipStream_t stream) {
  if (in_dtype == 1) return d == 64 ? launch_bwd<1, 64>(p, stream) : launch_bwd<1, 128>(p, stream);
  return d == 64 ? launch_bwd<2, 64>(p, stream) : launch_bwd<2, 128>(p, stream);
}
