// Fused exact attention forward pass for gfx950 (MI355X, CDNA4).
//
// The method ("FlashAttention (NL)"): Q, K, V are split into blocks that fit
// in on-chip memory and are loaded one after the other (section "Tiling en
// blokgewijze verwerking"); a running row maximum and a running sum of
// exponentials are updated block by block so the softmax comes out exact
// (section "Online berekening van Softmax"); QK^T, masking, softmax and the
// product with V run in one fused kernel that writes only the final result
// (section "Samensmelting van bewerkingen in één CUDA-kernel").
//
// gfx950 mapping (one workgroup = 4 wavefronts of 64 lanes, 128 query rows,
// two workgroups per CU):
//  * Each wavefront owns 32 query rows for the whole key loop.  Its Q rows
//    stay in VGPRs as matrix-core operands, loaded once from HBM.
//  * K/V blocks of 64 keys go HBM -> LDS directly (buffer_load_dwordx4 with
//    the LDS destination: no VGPR staging, no VALU), double-buffered: block
//    t+1 is in flight while block t is computed, one barrier per block.  The
//    buffer descriptor of each block ends at key N, so keys past the end read
//    as zeros.  Rows are stored with an XOR swizzle of their 16-byte chunks
//    (the swizzle is applied on the global side, since the LDS side of these
//    loads is lane-contiguous) so that both LDS read patterns below run at
//    the minimum number of LDS cycles.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: in the 32x32 accumulator every lane then
//    holds one query row (lane mod 32) and 16 of its keys, so the row max and
//    row sum are in-lane reductions plus one exchange between the two lane
//    halves (v_permlane32_swap).
//  * O^T = V^T P^T: the probabilities are rounded to the input type and used
//    straight from the accumulator registers as the B operand; the V^T
//    operand is read from the row-major V block with ds_read_b64_tr_b16
//    (within each 16-lane group, lane j receives element j mod 4 of the
//    8-byte pieces addressed by lanes 4t + j/4, t = 0..3), at the keys that
//    match the accumulator's row order, so no data moves between the two
//    matrix products.
//  * The softmax runs in base 2 with scale*log2(e) folded into one FMA.  The
//    reference maximum is raised only when a row maximum exceeds it by more
//    than 8 (base-2 units); in between, probabilities may reach 2^8, which
//    fp32 accumulators and bf16/f16 operands hold exactly as well as values
//    <= 1.  Output and row sum share the same reference, so the result is
//    the same softmax; the O rescale is skipped on almost every block.
//  * Tiles are classified with integer range tests (tile_class.h): fully
//    masked key blocks are never visited, fully visible ones run without a
//    per-element mask, only boundary blocks evaluate the mask predicate.
//  * Work order: longest row tiles first for masked inputs, and, when
//    batch*heads is a multiple of 8, every XCD (blockIdx mod 8) processes its
//    own set of heads so that a head's K/V stays within one L2.
// fp32 inputs use v_mfma_f32_32x32x2f32 in a simpler kernel of the same
// structure (register-staged K/V, V row-major in LDS, 32-key blocks).
#include <hip/hip_runtime.h>

#include "fa_kernels.h"
#include "tile_class.h"

typedef __bf16 fa_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 fa_f16x8 __attribute__((ext_vector_type(8)));
typedef float fa_f32x16 __attribute__((ext_vector_type(16)));
typedef float fa_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int fa_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int fa_u32x2 __attribute__((ext_vector_type(2)));
typedef short fa_i16x4 __attribute__((ext_vector_type(4)));

#define FA_AS3 __attribute__((address_space(3)))
#define FA_NEG_INF (-__builtin_inff())
#define FA_LN2 0.69314718055994530942f
#define FA_RESCALE_THRESHOLD 8.0f
// buffer descriptor word 3 for raw (unformatted, unswizzled) buffer access
#define FA_BUF_WORD3 0x00020000
// s_waitcnt with vmcnt(0) only (expcnt and lgkmcnt at their "no wait" maxima)
#define FA_WAIT_VMCNT0 0x0F70

namespace {

// ---------------------------------------------------------------------------
// matrix-core products, conversions, lane-half exchange
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ fa_f32x16 mma16(fa_u32x4 a, fa_u32x4 b, fa_f32x16 c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(fa_bf16x8, a), __builtin_bit_cast(fa_bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(fa_f16x8, a), __builtin_bit_cast(fa_f16x8, b), c, 0, 0, 0);
}

// Round 8 floats to the 16-bit input type (nearest even), packed in 4 words.
template <int DT>
__device__ __forceinline__ fa_u32x4 pack8(const float* x) {
  if constexpr (DT == 2) {
    fa_bf16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (__bf16)x[i];
    return __builtin_bit_cast(fa_u32x4, h);
  } else {
    fa_f16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)x[i];
    return __builtin_bit_cast(fa_u32x4, h);
  }
}

template <int DT>
__device__ __forceinline__ fa_u32x2 pack4(float a, float b, float c, float d) {
  if constexpr (DT == 2) {
    __bf16 h[4] = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    return __builtin_bit_cast(fa_u32x2, h);
  } else {
    _Float16 h[4] = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    return __builtin_bit_cast(fa_u32x2, h);
  }
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + lo + hi of a packed pair of 16-bit values (one v_dot2c with (1, 1)).
template <int DT>
__device__ __forceinline__ float sum2(unsigned int pair, float acc) {
  if constexpr (DT == 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
  }
}

// Lanes l and l^32 hold the same query row: combine their values.  The swap
// leaves each lane with its own value in one result and its partner's in the
// other, so max / sum of the two results is the pair's max / sum.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// pieces shared by both kernels
// ---------------------------------------------------------------------------

// Work item of this workgroup: (batch*head, first query row).
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
  q0 = qt * FA_ROWS_PER_WG;
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

// Online-softmax step on one key block: row maximum, reference update with
// O rescale (rare), probabilities p = 2^(s*scale*log2e - m).
template <int NKB, int NCB>
__device__ __forceinline__ void softmax_block(fa_f32x16 (&s)[NKB], float (&pr)[NKB][16],
                                              fa_f32x16 (&acc)[NCB], float& m_ref, float& l_lane,
                                              float& lq_lane, float c2) {
  float mx = FA_NEG_INF;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = pair_max(mx);
  const float mxs = mx * c2;
  const bool need = mxs > m_ref + FA_RESCALE_THRESHOLD;
  if (__ballot(need)) {
    const float m_new = fmaxf(m_ref, mxs);
    const float alpha = (m_new == m_ref) ? 1.f : exp2_hw(m_ref - m_new);
    m_ref = m_new;
    l_lane *= alpha;
    lq_lane *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
  }
  const float m_use = (m_ref == FA_NEG_INF) ? 0.f : m_ref;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[kb][r] = exp2_hw(__builtin_fmaf(s[kb][r], c2, -m_use));
}

// O = O^T / l (sum of the probabilities used in the product with V),
// lse = (m + log2 l) ln 2 (sum of the unrounded probabilities).
template <int DT, int D, bool OUT_F32>
__device__ __forceinline__ void store_output(const FaFwdParams& p, const fa_f32x16 (&acc)[D / 32],
                                             float m_ref, float l_lane, float lq_lane, int bh,
                                             int qi, int half) {
  const int N = p.N;
  const float l_tot = pair_sum(l_lane);
  const float lq_tot = pair_sum(lq_lane);
  const float inv = lq_tot > 0.f ? 1.f / lq_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * FA_LN2 : FA_NEG_INF;
  if (qi >= N) return;
  const size_t row = (size_t)bh * N + qi;
  unsigned char* Orow = (unsigned char*)p.o + row * D * (OUT_F32 ? 4 : 2);
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = cb * 32 + 8 * g + 4 * half;
      const float o0 = acc[cb][4 * g] * inv, o1 = acc[cb][4 * g + 1] * inv;
      const float o2 = acc[cb][4 * g + 2] * inv, o3 = acc[cb][4 * g + 3] * inv;
      if constexpr (OUT_F32) {
        const fa_f32x4 val = {o0, o1, o2, o3};
        *(fa_f32x4*)(Orow + c * 4) = val;
      } else {
        *(fa_u32x2*)(Orow + c * 2) = pack4<DT>(o0, o1, o2, o3);
      }
    }
  if (half == 0) p.lse[row] = lse;
}

// ---------------------------------------------------------------------------
// bf16 / f16 kernel
// ---------------------------------------------------------------------------

// 16-byte chunk swizzles (row r): K rows are read 16 rows x one chunk per
// 16 lanes, V rows 8 rows x 4 chunks per wavefront by the transposing read.
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

template <int DT, int D, bool OUT_F32>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd16_kernel(FaFwdParams p) {
  constexpr int BC = FA_KEYS_16;   // keys per block
  constexpr int NKB = BC / 32;     // 32-key groups per block
  constexpr int NCB = D / 32;      // 32-column output blocks
  constexpr int NQF = D / 16;      // 16-deep slices of the QK^T contraction
  constexpr int ROWB = 2 * D;      // bytes of one K/V row
  constexpr int TILEB = BC * ROWB; // bytes of one K or V block
  constexpr int LPW = TILEB / (FA_WAVES * 1024);  // 1 KB loads per wave per matrix
  static_assert(LPW * FA_WAVES * 1024 == TILEB, "loads must cover the block");
  // LDS: K and V, double-buffered, as four separate objects so that the
  // compiler can tell the block being read from the one being filled (and
  // does not wait for the prefetch before reading the current block)
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILEB], ks1[TILEB], vs0[TILEB], vs1[TILEB];
  // (the lambdas below take the buffer index as a plain int: every call
  // passes a constant, so the selections fold away after inlining)
  auto kbuf = [&](int b) { return (FA_AS3 unsigned char*)(b ? ks1 : ks0); };
  auto vbuf = [&](int b) { return (FA_AS3 unsigned char*)(b ? vs1 : vs0); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int N = p.N;

  int bh, q0;
  work_item(p, bh, q0);
  const int q1 = min(q0 + FA_ROWS_PER_WG, N);
  const int qw0 = q0 + wave * FA_ROWS_PER_WAVE;
  const int qw1 = min(qw0 + FA_ROWS_PER_WAVE, N);
  const int qi = qw0 + l32;  // this lane's query row

  const size_t head_bytes = (size_t)N * ROWB;
  const unsigned char* Qh = (const unsigned char*)p.q + (size_t)bh * head_bytes;
  const unsigned char* Kh = (const unsigned char*)p.k + (size_t)bh * head_bytes;
  const unsigned char* Vh = (const unsigned char*)p.v + (size_t)bh * head_bytes;

  int kv_lo, kv_hi;
  fa_key_block_range(q0, q1, BC, N, p.mask_kind, p.window, &kv_lo, &kv_hi);

  // Q fragment ks holds q[qi][16 ks + 8 half .. +7]; rows past N read row
  // N-1 (no branch) and are never stored.
  fa_u32x4 qf[NQF];
  {
    const unsigned char* qrow = Qh + (size_t)min(qi, N - 1) * ROWB;
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks) qf[ks] = *(const fa_u32x4*)(qrow + ks * 32 + half * 16);
  }

  // Global byte offsets (within a block) of this lane's 16 bytes in each of
  // the wave's LPW one-kilobyte LDS pieces, swizzle applied.
  unsigned koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int o = (i * FA_WAVES + wave) * 1024 + 16 * lane;
    const int r = o / ROWB, pos = (o % ROWB) / 16;
    koff[i] = r * ROWB + 16 * (pos ^ kswz<D>(r));
    voff[i] = r * ROWB + 16 * (pos ^ vswz<D>(r));
  }
  // LDS read offsets: K slice s of row l32 (chunk 2s + half); V^T pieces for
  // output block cb (row 4half + t, columns 32cb + 16(lane/16 mod 2) + 4q).
  unsigned kread[NQF], vread[NCB];
#pragma unroll
  for (int s = 0; s < NQF; ++s) kread[s] = l32 * ROWB + 16 * ((2 * s + half) ^ kswz<D>(l32));
  {
    const int g = lane >> 4, t = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      vread[cb] = (4 * half + t) * ROWB + 64 * (cb ^ (D == 128 ? t : (t >> 1))) + 32 * (g & 1) + 8 * q;
  }

  // Block kt -> LDS buffer buf.  The descriptor's base is the block's first
  // key and its size stops at key N, so rows past N read as zeros.  (The
  // offsets are passed as int prvalues: handing the builtin the captured
  // array element itself keeps hipcc's host pass from emitting the kernel's
  // launch stub.)
  auto issue = [&](int kt, int buf) {
    FA_AS3 unsigned char* const kdst = kbuf(buf);
    FA_AS3 unsigned char* const vdst = vbuf(buf);
    const int k0 = kt * BC;
    const int nb = (min(N - k0, BC)) * ROWB;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kh + (size_t)k0 * ROWB), 0, nb, FA_BUF_WORD3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vh + (size_t)k0 * ROWB), 0, nb, FA_BUF_WORD3);
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (FA_AS3 void*)(kdst + (i * FA_WAVES + wave) * 1024), 16, (int)koff[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (FA_AS3 void*)(vdst + (i * FA_WAVES + wave) * 1024), 16, (int)voff[i], 0, 0, 0);
  };

  fa_f32x16 acc[NCB];  // O^T: block cb holds columns 32cb.., row qi
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float m_ref = FA_NEG_INF;  // reference maximum (base-2 scaled units)
  float l_lane = 0.f;        // this lane's part of the exponent sum
  float lq_lane = 0.f;       // same, of the probabilities as rounded for P V
  const float c2 = p.scale_log2;
  const int n_row_blocks = (N + FA_ROWS_PER_WAVE - 1) / FA_ROWS_PER_WAVE;
  const int n_key_blocks = (N + BC - 1) / BC;
  const int row_block = qw0 / FA_ROWS_PER_WAVE;

  // One key block: prefetch the next into the other buffer, compute this one
  // (unless fully masked for this wave), wait for the prefetch, barrier.
  auto body = [&](int kt, int buf) {
    FA_AS3 unsigned char* const kcur = kbuf(buf);
    FA_AS3 unsigned char* const vcur = vbuf(buf);
    if (kt + 1 < kv_hi) issue(kt + 1, 1 - buf);
    const int k0 = kt * BC;
    const int cls = fa_classify(qw0, qw1, k0, BC, N, p.mask_kind, p.window);
    if (p.tiles && lane == 0 && qw0 < N)
      p.tiles[((size_t)bh * n_row_blocks + row_block) * n_key_blocks + kt] = (unsigned char)(cls + 1);
    if (cls != FA_TILE_SKIP) {
      // S^T = K Q^T: s[kb][r] is key k0 + 32kb + 8(r/4) + 4half + r%4
      fa_f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NQF; ++ks) {
          const fa_u32x4 a = *(const FA_AS3 fa_u32x4*)(kcur + kb * 32 * ROWB + kread[ks]);
          s[kb] = mma16<DT>(a, qf[ks], s[kb]);
        }
      }
      if (cls == FA_TILE_PARTIAL) apply_mask<NKB>(s, k0, qi, half, N, p.mask_kind, p.window);
      float pr[NKB][16];
      softmax_block<NKB, NCB>(s, pr, acc, m_ref, l_lane, lq_lane, c2);

      // Two row sums.  The output is normalised by the sum of the ROUNDED
      // probabilities (the values the matrix core multiplies V with; two per
      // dot2), so output and normaliser use identical weights: constant V
      // comes out exact and a dominant key is selected exactly.  lse uses the
      // sum of the unrounded probabilities, which rounding to 16 bits would
      // otherwise move by up to 2^-9.
      // B operand (kb, t): slots 0..7 = registers 8t..8t+7, i.e. keys
      // 32kb + 16t + {4half + 0..3, 8 + 4half + 0..3}.
      fa_u32x4 pf[NKB][2];
      float psum = 0.f, qsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          pf[kb][t] = pack8<DT>(&pr[kb][8 * t]);
#pragma unroll
          for (int w = 0; w < 4; ++w) qsum = sum2<DT>(pf[kb][t][w], qsum);
#pragma unroll
          for (int i = 0; i < 8; ++i) psum += pr[kb][8 * t + i];
        }
      l_lane += psum;
      lq_lane += qsum;

      // O^T += V^T P^T; the A operand holds V at the same keys: rows
      // 32kb + 16t + 4half + 0..3 (first read) and + 8 (second read).
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            FA_AS3 unsigned char* vp = vcur + (32 * kb + 16 * t) * ROWB + vread[cb];
            const fa_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)vp);
            const fa_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)(vp + 8 * ROWB));
            const fa_u32x2 l2 = __builtin_bit_cast(fa_u32x2, lo), h2 = __builtin_bit_cast(fa_u32x2, hi);
            const fa_u32x4 a = {l2.x, l2.y, h2.x, h2.y};
            acc[cb] = mma16<DT>(a, pf[kb][t], acc[cb]);
          }
    }
    __builtin_amdgcn_s_waitcnt(FA_WAIT_VMCNT0);
    __syncthreads();
  };

  // Every workgroup has at least one key block: row q0 < N always sees key
  // q0 itself (the diagonal is visible under every mask).
  issue(kv_lo, 0);
  // Q fragments and the first block have landed before the loop starts, so
  // the loop's prefetch never waits behind them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = kv_lo;;) {
    body(kt, 0);
    if (++kt >= kv_hi) break;
    body(kt, 1);
    if (++kt >= kv_hi) break;
  }
  store_output<DT, D, OUT_F32>(p, acc, m_ref, l_lane, lq_lane, bh, qi, half);
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2f32; one contraction element per lane)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, D == 128 ? 1 : 2)))
fa_fwd32_kernel(FaFwdParams p) {
  constexpr int BC = FA_KEYS_32;       // keys per block (one 32-key group)
  constexpr int NCB = D / 32;
  constexpr int NQF = D / 2;           // 2-deep slices of the QK^T contraction
  constexpr int LD = D + 4;            // padded LDS row (floats)
  constexpr int CPR = D / 4;           // 16-byte chunks per row
  constexpr int LPT = BC * CPR / 256;  // staged loads per thread per matrix
  static_assert(LPT * (256 / CPR) == BC, "staging must cover the block");
  __shared__ __attribute__((aligned(16))) float smem32[2][2][BC][LD];  // [buf][K|V]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int N = p.N;

  int bh, q0;
  work_item(p, bh, q0);
  const int q1 = min(q0 + FA_ROWS_PER_WG, N);
  const int qw0 = q0 + wave * FA_ROWS_PER_WAVE;
  const int qw1 = min(qw0 + FA_ROWS_PER_WAVE, N);
  const int qi = qw0 + l32;
  const size_t head = (size_t)bh * N * D;
  const float* Qh = (const float*)p.q + head;
  const float* Kh = (const float*)p.k + head;
  const float* Vh = (const float*)p.v + head;

  int kv_lo, kv_hi;
  fa_key_block_range(q0, q1, BC, N, p.mask_kind, p.window, &kv_lo, &kv_hi);

  float qf[NQF];  // q[qi][2 ks + half]
  {
    const float* qrow = Qh + (size_t)min(qi, N - 1) * D;
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks) qf[ks] = qrow[2 * ks + half];
  }

  const int cc = tid % CPR, jg = tid / CPR;  // chunk, row group of this thread
  fa_u32x4 kst[LPT], vst[LPT];
  // keys past N load row N-1: only boundary blocks hold them, where the mask
  // gives them probability 0 and their finite values contribute 0 * v = 0
  auto gload = [&](int kt) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int j = min(kt * BC + jg * LPT + r, N - 1);
      kst[r] = *(const fa_u32x4*)(Kh + (size_t)j * D + cc * 4);
      vst[r] = *(const fa_u32x4*)(Vh + (size_t)j * D + cc * 4);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      *(fa_u32x4*)&smem32[buf][0][jg * LPT + r][cc * 4] = kst[r];
      *(fa_u32x4*)&smem32[buf][1][jg * LPT + r][cc * 4] = vst[r];
    }
  };

  fa_f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float m_ref = FA_NEG_INF, l_lane = 0.f, lq_lane = 0.f;
  const float c2 = p.scale_log2;
  const int n_row_blocks = (N + FA_ROWS_PER_WAVE - 1) / FA_ROWS_PER_WAVE;
  const int n_key_blocks = (N + BC - 1) / BC;
  const int row_block = qw0 / FA_ROWS_PER_WAVE;

  gload(kv_lo);
  lstore(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = kv_lo; kt < kv_hi; ++kt) {
    const int buf = (kt - kv_lo) & 1;
    const bool has_next = kt + 1 < kv_hi;
    const int k0 = kt * BC;
    const int cls = fa_classify(qw0, qw1, k0, BC, N, p.mask_kind, p.window);
    if (p.tiles && lane == 0 && qw0 < N)
      p.tiles[((size_t)bh * n_row_blocks + row_block) * n_key_blocks + kt] = (unsigned char)(cls + 1);
    if (has_next) gload(kt + 1);
    if (cls != FA_TILE_SKIP) {
      fa_f32x16 s[1];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[0][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NQF; ++ks)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(smem32[buf][0][l32][2 * ks + half], qf[ks], s[0], 0, 0, 0);
      if (cls == FA_TILE_PARTIAL) apply_mask<1>(s, k0, qi, half, N, p.mask_kind, p.window);
      float pr[1][16];
      softmax_block<1, NCB>(s, pr, acc, m_ref, l_lane, lq_lane, c2);
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) psum += pr[0][r];
      l_lane += psum;
      lq_lane += psum;  // fp32 products use p unrounded
      // O^T += V^T P^T, one key pair {8(r/4) + r%4, +4} per product
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              smem32[buf][1][8 * (r >> 2) + 4 * half + (r & 3)][cb * 32 + l32], pr[0][r], acc[cb], 0, 0, 0);
    }
    if (has_next) lstore(buf ^ 1);
    __syncthreads();
  }
  store_output<0, D, true>(p, acc, m_ref, l_lane, lq_lane, bh, qi, half);
}

// One wavefront, one product: lane-order operands in, lane-order accumulator
// out (16 floats per lane).
template <int WHICH>
__global__ void __launch_bounds__(64) fa_probe_kernel(const void* a, const void* b, float* d) {
  const int l = threadIdx.x;
  fa_f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = 0.f;
  if constexpr (WHICH == 2) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(((const float*)a)[l], ((const float*)b)[l], c, 0, 0, 0);
  } else {
    const fa_u32x4 av = ((const fa_u32x4*)a)[l];
    const fa_u32x4 bv = ((const fa_u32x4*)b)[l];
    c = mma16<WHICH == 0 ? 2 : 1>(av, bv, c);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) d[l * 16 + r] = c[r];
}

// Matrix-core ceiling: back-to-back independent bf16 32x32x16 products (8
// accumulator chains per wave), no memory traffic.  Thread 0 of each
// workgroup records the shader clock counter and the 100 MHz real-time
// counter before and after the loop.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_mfma_ceiling_kernel(int iters, unsigned long long* clk, float* sink) {
  const float x = 0.001f * (float)(threadIdx.x & 7);
  fa_bf16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (__bf16)x;
  const fa_u32x4 a = __builtin_bit_cast(fa_u32x4, h);
  fa_f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  unsigned long long c0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    c0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mma16<2>(a, a, acc[j]);
  if (threadIdx.x == 0) {
    const unsigned long long c1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[blockIdx.x * 4 + 0] = c0;
    clk[blockIdx.x * 4 + 1] = c1;
    clk[blockIdx.x * 4 + 2] = r0;
    clk[blockIdx.x * 4 + 3] = r1;
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += acc[j][r];
  sink[blockIdx.x * 256 + threadIdx.x] = t;
}

template <int DT, int D, bool OUT_F32>
hipError_t launch(const FaFwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.BH * p.n_row_tiles));
  if constexpr (DT == 0)
    hipLaunchKernelGGL((fa_fwd32_kernel<D>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fa_fwd16_kernel<DT, D, OUT_F32>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t fa_launch_fwd(int in_dtype, int out_dtype, int d, const FaFwdParams& p,
                         hipStream_t stream) {
  const bool of32 = (out_dtype == 0);
  switch (in_dtype) {
    case 0:
      return d == 64 ? launch<0, 64, true>(p, stream) : launch<0, 128, true>(p, stream);
    case 1:
      if (d == 64) return of32 ? launch<1, 64, true>(p, stream) : launch<1, 64, false>(p, stream);
      return of32 ? launch<1, 128, true>(p, stream) : launch<1, 128, false>(p, stream);
    default:
      if (d == 64) return of32 ? launch<2, 64, true>(p, stream) : launch<2, 64, false>(p, stream);
      return of32 ? launch<2, 128, true>(p, stream) : launch<2, 128, false>(p, stream);
  }
}

hipError_t fa_launch_probe(int which, const void* a, const void* b, float* d,
                           hipStream_t stream) {
  if (which == 0)
    hipLaunchKernelGGL(fa_probe_kernel<0>, dim3(1), dim3(64), 0, stream, a, b, d);
  else if (which == 1)
    hipLaunchKernelGGL(fa_probe_kernel<1>, dim3(1), dim3(64), 0, stream, a, b, d);
  else
    hipLaunchKernelGGL(fa_probe_kernel<2>, dim3(1), dim3(64), 0, stream, a, b, d);
  return hipGetLastError();
}

hipError_t fa_launch_mfma_ceiling(int n_blocks, int iters, unsigned long long* clk, float* sink,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(fa_mfma_ceiling_kernel, dim3(n_blocks), dim3(256), 0, stream, iters, clk, sink);
  return hipGetLastError();
}
