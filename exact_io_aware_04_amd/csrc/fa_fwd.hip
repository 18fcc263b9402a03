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
// gfx950 mapping, bf16/f16 inputs (one workgroup = 8 wavefronts of 64
// lanes, 256 query rows, one workgroup per CU, two wavefronts per SIMD):
//  * Each wavefront owns 32 query rows for the whole key loop.  Its Q rows
//    stay in VGPRs as matrix-core operands, loaded once from HBM.
//  * The two wavefronts of a SIMD run half a key block apart: while one
//    issues its matrix products, the other computes its softmax, so the
//    matrix core and the vector ALU are busy at the same time.  A workgroup
//    barrier between half steps keeps the two groups (waves 0-3 and 4-7) in
//    opposite phases.
//  * K/V blocks of 64 keys go HBM -> LDS directly (buffer_load_dwordx4 with
//    the LDS destination: no VGPR staging, no VALU) into rings of three
//    slots each; block kt+2 is loaded while block kt is computed, K by the
//    leading and V by the trailing wavefronts, each at the end of its
//    softmax phase (at d = 64, where the matrix phase is the shorter half,
//    the leading wavefronts load both at the end of their matrix phase).
//    The buffer descriptor of each block ends at key N, so
//    keys past the end read as zeros.  Rows are stored with an XOR swizzle of
//    their 16-byte chunks (applied on the global side, since the LDS side of
//    these loads is lane-contiguous) so that both LDS read patterns below
//    run at the minimum number of LDS cycles.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: in the 32x32 accumulator every lane then
//    holds one query row (lane mod 32) and 16 of its keys, so the row max and
//    row sum are in-lane reductions plus one exchange between the two lane
//    halves (v_permlane32_swap).  The accumulators start from -m/(scale
//    log2 e) for the row's reference m, so each probability needs one
//    multiply and one exponential.
//  * O^T = V^T P^T: the probabilities are rounded to the input type and used
//    straight from the accumulator registers as the B operand; the V^T
//    operand is read from the row-major V block with ds_read_b64_tr_b16
//    (within each 16-lane group, lane j receives element j mod 4 of the
//    8-byte pieces addressed by lanes 4t + j/4, t = 0..3), at the keys that
//    match the accumulator's row order, so no data moves between the two
//    matrix products.  The row sums of the rounded probabilities come from
//    the matrix core too: one 16x16x32 product per P^T operand, with an A
//    operand of ones and zeros that picks each lane's own row.
//  * The softmax runs in base 2.  The reference maximum is set to the exact
//    row maximum on a row's first block and on boundary blocks, and otherwise
//    kept while every probability stays below 2^8 (checked through the lane
//    sums); fp32 accumulators and bf16/f16 operands hold such values as
//    exactly as values <= 1.  Output and row sum share the same reference,
//    so the result is the same softmax; the O rescale is skipped on almost
//    every block.
//  * Tiles are classified with integer range tests (tile_class.h): fully
//    masked key blocks are never visited by a workgroup, and give a wave
//    probabilities of exactly 0 where only some of its rows see them; fully
//    visible ones run without a per-element mask, only boundary blocks
//    evaluate the mask predicate.
//  * Work order: one persistent workgroup per compute unit walks a list of
//    row tiles, longest first for masked inputs (paired long with short),
//    and, when batch*heads is a multiple of 8, every XCD (blockIdx mod 8)
//    processes its own set of heads so that a head's K/V stays within one
//    L2.  The K/V blocks of consecutive tiles stream through the same LDS
//    rings, so the next tile's first blocks load during the current one.
// fp32 inputs use v_mfma_f32_32x32x2f32 in a simpler kernel (4 wavefronts,
// 128 query rows, register-staged and double-buffered K/V, 32-key blocks,
// the reference raised only when a row maximum exceeds it by more than 8).
#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_fwd_common.h"
#include "fa_kernels.h"
#include "tile_class.h"

#define FA_RESCALE_THRESHOLD 8.0f

namespace {

// ---------------------------------------------------------------------------
// pieces shared by both kernels
// ---------------------------------------------------------------------------

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

// O = O^T / lq (row sum of the probabilities used in the product with V),
// lse = (m + log2 l) ln 2 (l: row sum of the unrounded probabilities).
template <int DT, int D, bool OUT_F32>
__device__ __forceinline__ void store_output(const FaFwdParams& p, const fa_f32x16 (&acc)[D / 32],
                                             float m_ref, float l_tot, float lq_tot, int bh,
                                             int qi, int half) {
  const int N = p.N;
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

// 16-bit output of one wave's 32 rows through 16 rows of LDS scratch
// (`stage`, 32 D bytes private to the wave), in two rounds of 16 rows.  Straight from
// the accumulators each store instruction would cover 32 rows with 16 bytes
// each; restaged, each covers 4 (d = 128) or 8 (d = 64) whole rows.  Round
// j: the lanes of rows 16j .. 16j+15 write their 4-column pieces (row r at
// r * 2D bytes, 16-byte chunk c at position c ^ (r mod chunks per row), so
// that the 32 writing lanes of one instruction hit distinct banks), then
// every lane reads one 16-byte chunk and stores it (rows past N skipped).
// lse as in store_output.
template <int DT, int D>
__device__ __forceinline__ void store_output_staged(const FaFwdParams& p, const fa_f32x16 (&acc)[D / 32],
                                                    float m_ref, float l_tot, float lq_tot, int bh,
                                                    int qb0, int lane, FA_AS3 unsigned char* stage) {
  constexpr int ROWB = 2 * D, CPR = ROWB / 16;  // bytes and 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                  // rows per read instruction
  const int N = p.N;
  const int l32 = lane & 31, half = lane >> 5;
  const int qi = qb0 + l32;
  const float inv = lq_tot > 0.f ? 1.f / lq_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * FA_LN2 : FA_NEG_INF;
  unsigned char* O = (unsigned char*)p.o + ((size_t)bh * N) * ROWB;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if ((l32 >> 4) == j) {
      const int r = l32 & 15;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = (4 * cb + g) ^ (r & (CPR - 1));
          *(FA_AS3 fa_u32x2*)(stage + r * ROWB + 16 * ch + 8 * half) =
              pack4<DT>(acc[cb][4 * g] * inv, acc[cb][4 * g + 1] * inv, acc[cb][4 * g + 2] * inv,
                        acc[cb][4 * g + 3] * inv);
        }
    }
    __builtin_amdgcn_s_waitcnt(FA_WAITCNT_LGKM0);
    fa_u32x4 val[16 / RPI];  // all reads first, one wait, then the stores
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i)
      val[i] = *(const FA_AS3 fa_u32x4*)(stage + (i * RPI + lane / CPR) * ROWB + 16 * (lane % CPR));
    __builtin_amdgcn_s_waitcnt(FA_WAITCNT_LGKM0);
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int r = i * RPI + lane / CPR, pos = lane % CPR;
      const int row = qb0 + 16 * j + r;
      if (row < N) *(fa_u32x4*)(O + (size_t)row * ROWB + 16 * (pos ^ (r & (CPR - 1)))) = val[i];
    }
  }
  if (half == 0 && qi < N) p.lse[(size_t)bh * N + qi] = lse;
}

// ---------------------------------------------------------------------------
// bf16 / f16 kernel
// ---------------------------------------------------------------------------


// Row sums of the rounded probabilities on the matrix core.  A P^T operand
// of the 32x32x16 product (lane l: row l mod 32, 8 keys of half l / 32) is
// also a valid B operand of v_mfma_f32_16x16x32_{bf16,f16}, where lane l
// holds 8 of the 32 contraction indices of slice l / 16 for output column
// l mod 16; the A operand of lane l covers row l mod 16 over the same slice.
// Slices 0 and 2 hold rows 0..15 of P, slices 1 and 3 rows 16..31.  An A
// operand that is all ones in the lanes where slice parity ((l >> 4) & 1)
// equals ((l >> 2) & 1), zero elsewhere, makes output rows 0-3 and 8-11 the
// sums of rows n and rows 4-7 and 12-15 those of rows n + 16, and lane l
// holds rows 4(l / 16)..+3 of column l mod 16: every register of the 4-word
// accumulator then carries the sum of the lane's own row l mod 32.  Half the
// matrix-core cycles of a 32x32x16 product.
template <int DT>
__device__ __forceinline__ fa_u32x4 rowsum_selector(int lane) {
  constexpr unsigned ONE2 = DT == 2 ? 0x3F803F80u : 0x3C003C00u;
  const unsigned v = (((lane >> 4) ^ (lane >> 2)) & 1) ? 0u : ONE2;
  return fa_u32x4{v, v, v, v};
}
template <int DT>
__device__ __forceinline__ fa_f32x4 rowsum_mma(fa_u32x4 sel, fa_u32x4 b, fa_f32x4 c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(fa_bf16x8, sel), __builtin_bit_cast(fa_bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(fa_f16x8, sel), __builtin_bit_cast(fa_f16x8, b), c, 0, 0, 0);
}

// Largest of a block's rounded fp16 probabilities, as its bit pattern:
// non-negative fp16 values order like their bits, and infinity and NaN
// sort above every finite value.  Packed 16-bit maxima, then the larger
// half.
#define FA_F16_BITS_256 0x5C00u  // 256.0 in fp16
typedef unsigned short fa_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ fa_u16x2 u16_pair(unsigned w) { return __builtin_bit_cast(fa_u16x2, w); }
__device__ __forceinline__ fa_u16x2 u16_max(fa_u16x2 a, fa_u16x2 b) {
  return __builtin_elementwise_max(a, b);
}
__device__ __forceinline__ unsigned max_f16_bits(const fa_u32x4 (&pf)[2][2]) {
  // (each word is read into a scalar first: hipcc took element 0 for every
  // index when the vector element went to __builtin_bit_cast directly)
  fa_u16x2 m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned a = pf[0][0][i], b = pf[0][1][i], c = pf[1][0][i], d = pf[1][1][i];
    m[i] = u16_max(u16_max(u16_pair(a), u16_pair(b)), u16_max(u16_pair(c), u16_pair(d)));
  }
  const fa_u16x2 r = u16_max(u16_max(m[0], m[1]), u16_max(m[2], m[3]));
  return max((unsigned)r.x, (unsigned)r.y);
}

// Matrix phase of one wavefront: S^T = K Q^T over the current key block (QK)
// and O^T += V^T P^T over the previous one (PV), as one software-pipelined
// sequence of products whose LDS operands are read FA_OPND_AHEAD products
// ahead.  The wavefront issues its products while its SIMD partner computes
// a softmax, so nothing else hides the LDS latency.  The scores come first:
// the softmax that follows waits only for them, while the P V products are
// still executing.  Product order: Q K by contraction slice s, then key
// group kb (the score accumulators starting from sc0); then P V by (kb,
// half t), then output block cb, so consecutive products update different
// accumulators; last, four row-sum products (rowsum_mma) add the block's
// rounded probabilities to the row sums lsum.  The
// K operand of (s, kb) is one 16-byte read of row
// 32kb + l32, chunk 2s + half; the V^T operand of (kb, t, cb) two
// transposing reads at rows 32kb + 16t + 4half + 0..3 and + 8 (the keys of
// the P^T operand).
#define FA_OPND_AHEAD 6
template <int DT, int D>
__device__ __forceinline__ void matrix_phase(fa_f32x16 (&acc)[D / 32], fa_f32x16 (&sc)[2],
                                             fa_f32x4& lsum, const fa_u32x4& sel,
                                             const fa_f32x16& sc0,
                                             const fa_u32x4 (&pf)[2][2], const fa_u32x4 (&qf)[D / 16],
                                             const FA_AS3 unsigned char* kcur,
                                             const FA_AS3 unsigned char* vcur,
                                             const unsigned (&kread)[D / 16],
                                             const unsigned (&vread)[D / 32]) {
  constexpr int NCB = D / 32, NQF = D / 16, ROWB = 2 * D;
  constexpr int NQK = 2 * NQF;
  constexpr int NOPS = NQK + 4 * NCB;
  constexpr int R = FA_OPND_AHEAD;
  constexpr int NSLOT = R + 1;  // the slot being filled is never the one being read
  fa_u32x4 opnd[NSLOT];
  sc[0] = sc0;
  sc[1] = sc0;
#pragma unroll
  for (int i = 0; i < NOPS + R; ++i) {
    if (i >= R) {  // product i - R
      const int j = i - R;
      if (j < NQK) {
        const int sl = j / 2, kb = j % 2;
        sc[kb] = mma16<DT>(opnd[j % NSLOT], qf[sl], sc[kb]);
      } else {
        const int q = j - NQK, cb = q % NCB, kb = q / NCB / 2, t = q / NCB % 2;
        acc[cb] = mma16<DT>(opnd[j % NSLOT], pf[kb][t], acc[cb]);
      }
    }
    if (i < NOPS) {  // operand of product i
      if (i < NQK) {
        const int sl = i / 2, kb = i % 2;
        opnd[i % NSLOT] = *(const FA_AS3 fa_u32x4*)(kcur + kb * 32 * ROWB + kread[sl]);
      } else {
        const int q = i - NQK, cb = q % NCB, kb = q / NCB / 2, t = q / NCB % 2;
        const FA_AS3 unsigned char* vp = vcur + (32 * kb + 16 * t) * ROWB + vread[cb];
        const fa_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)vp);
        const fa_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)(vp + 8 * ROWB));
        const fa_u32x2 l2 = __builtin_bit_cast(fa_u32x2, lo), h2 = __builtin_bit_cast(fa_u32x2, hi);
        opnd[i % NSLOT] = fa_u32x4{l2.x, l2.y, h2.x, h2.y};
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // row sums of the rounded probabilities
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) lsum = rowsum_mma<DT>(sel, pf[kb][t], lsum);
}

// Eight wavefronts, 32 query rows each, two per SIMD.  The two wavefronts of
// a SIMD run half a key block apart ("ping-pong"): while one issues the
// matrix products of a block, the other computes the softmax of its block,
// so the matrix cores and the vector ALUs work at the same time.  Wavefronts
// 0-3 lead, 4-7 trail; a workgroup barrier between half steps keeps the two
// groups in opposite phases.
//
// Persistent: one workgroup per compute unit walks its list of row tiles
// (fa_persist_tile_of; under a causal mask or none, the tiles an XCD runs
// together read one key/value head, and under a sliding window of whole row
// tiles each team of workgroups reads the same key/value block at the same
// time, so the XCD's L2 serves their common key and value blocks once from
// HBM).  The K/V blocks of consecutive tiles form one stream
// through the LDS rings: the first two blocks of the next tile are loaded
// during the last two steps of the current one, so a new tile starts with
// its first blocks in LDS and no workgroup launch in between.
template <int DT, int D, bool OUT_F32>
__global__ void __launch_bounds__(FA_WAVES_16 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd16_kernel(FaFwdParams p) {
  constexpr int NW = FA_WAVES_16;
  constexpr int ROWS_WG = NW * FA_ROW_BLOCK;
  constexpr int BC = FA_KEYS_16;   // keys per block
  constexpr int NKB = BC / 32;     // 32-key groups per block
  constexpr int NCB = D / 32;      // 32-column output blocks
  constexpr int NQF = D / 16;      // 16-deep slices of the QK^T contraction
  constexpr int ROWB = 2 * D;      // bytes of one K/V row
  constexpr int TILEB = BC * ROWB; // bytes of one K or V block
  constexpr int NL = NW / 2;       // wavefronts loading each matrix (K: leading, V: trailing)
  constexpr int LPW = TILEB / (NL * 1024);  // 1 KB loads per loading wave per block
  static_assert(LPW * NL * 1024 == TILEB, "loads must cover the block");
  static_assert(NL * 1024 / ROWB % 16 == 0, "pieces must be a multiple of 16 rows apart");
  static_assert(NW == 8 && FA_STAGES_16 == 3, "schedule below: 2 x 4 wavefronts, rings of 3");
  // One workgroup barrier per key block at d = 64 (where the softmax phase
  // takes about twice as long as the matrix phase), two at d = 128; the
  // step loop below describes both schedules.
  constexpr bool ONE_BARRIER = D == 64;
  // fp16 inputs: lse from the sum of the rounded probabilities (see the
  // softmax phase), and no unrounded sum.
  constexpr bool F16_SUMS = DT == 1;
  // LDS: rings of three K and three V blocks, as separate objects so that
  // the compiler can tell the slots being read from the ones being filled
  // (and does not wait for the prefetches before reading)
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILEB], ks1[TILEB], ks2[TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[TILEB], vs1[TILEB], vs2[TILEB];
  // (the lambdas below take the slot index as a plain int: every call passes
  // a constant, so the selections fold away after inlining)
  auto kbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? ks0 : b == 1 ? ks1 : ks2); };
  auto vbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? vs0 : b == 1 ? vs1 : vs2); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave < NW / 2;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int N = p.N;
  const size_t head_bytes = (size_t)N * ROWB;

  // Global byte offset (within a block) of this lane's 16 bytes in a loading
  // wave's first one-kilobyte LDS piece, swizzle applied.  Piece i lies 4 KB
  // (16 or 32 rows) further on both sides: the swizzles depend on row bits
  // that a multiple of 16 rows leaves unchanged.
  unsigned koff, voff;
  {
    const int o = (wave % NL) * 1024 + 16 * lane;
    const int r = o / ROWB, pos = (o % ROWB) / 16;
    koff = r * ROWB + 16 * (pos ^ kswz<D>(r));
    voff = r * ROWB + 16 * (pos ^ vswz<D>(r));
  }
  const unsigned my_off = lead ? koff : voff;
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

  // K or V block kt of a head -> LDS slot.  The descriptor's base is the
  // block's first key and its size stops at key N, so rows past N read as
  // zeros (a block wholly past N, the padding of a one-block tile, reads
  // zeros only).  (The offsets are passed as int prvalues: handing the
  // builtin the captured array element itself keeps hipcc's host pass from
  // emitting the kernel's launch stub.)
  auto issue = [&](const unsigned char* base, unsigned off, FA_AS3 unsigned char* dst, int kt) {
    const int k0 = kt * BC;
    // (readfirstlane: the clamp would otherwise become a vector instruction
    // and the descriptor a per-lane value)
    const int nb = __builtin_amdgcn_readfirstlane(max(min(N - k0, BC), 0) * ROWB);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)k0 * ROWB), 0, nb, FA_BUF_WORD3);
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (FA_AS3 void*)(dst + (i * NL + wave % NL) * 1024), 16, (int)off, i * NL * 1024, 0, 0);
  };

  const fa_u32x4 sel = rowsum_selector<DT>(lane);
  const float c2 = p.scale_log2;
  const float inv_c2 = 1.f / p.scale_log2;
  const int n_row_blocks = (N + FA_ROW_BLOCK - 1) / FA_ROW_BLOCK;
  const int n_key_blocks = (N + BC - 1) / BC;

  // Tile state.  A tile is (bh, q0): batch*head bh, query rows q0 ..
  // q0+ROWS_WG-1.  Its key blocks kv_lo .. kv_end-1 are those some of its
  // rows see; the tile runs at least two (kv_hi = max(kv_end, kv_lo + 2):
  // the padding block, if any, lies past N and is skipped by every wave),
  // so that the next tile's first two blocks can always be loaded during the
  // last two steps of this one.  Query slice bh = b H + h reads key/value
  // slice b H_kv + h / g = bh / g.
  struct Tile {
    int bh, q0, kv_lo, kv_end, kv_hi;
    const unsigned char *Kh, *Vh;
  };
  auto make_tile = [&](int bh_, int q0_) {
    Tile t;
    t.bh = bh_;
    t.q0 = q0_;
    fa_key_block_range(q0_, min(q0_ + ROWS_WG, N), BC, N, p.mask_kind, p.window, &t.kv_lo,
                       &t.kv_end);
    t.kv_hi = max(t.kv_end, t.kv_lo + 2);
    const size_t kv_bytes = (size_t)(bh_ / p.kv_group) * head_bytes;
    t.Kh = (const unsigned char*)p.k + kv_bytes;
    t.Vh = (const unsigned char*)p.v + kv_bytes;
    return t;
  };

  int tile_k = 0, nbh = 0, nq0 = 0;
  {
    int bh0, q00;
    if (!persist_tile(p, 0, bh0, q00, ROWS_WG)) return;  // no work for this workgroup
    nbh = bh0;
    nq0 = q00;
  }
  Tile cur = make_tile(nbh, nq0);
  bool has_next = persist_tile(p, 1, nbh, nq0, ROWS_WG);
  Tile nxt = make_tile(has_next ? nbh : cur.bh, has_next ? nq0 : cur.q0);

  // Carried between tiles and steps: the output accumulators, the row's
  // reference (base 2) and sums, the scores of the current block (matrix
  // phase -> softmax phase) and its rounded probabilities (softmax phase ->
  // the next matrix phase).  s[kb][r] is key k0 + 32kb + 8(r/4) + 4half +
  // r%4 of row qi; P^T operand (kb, t) holds registers 8t..8t+7 of s[kb],
  // i.e. keys 32kb + 16t + {4half + 0..3, 8 + 4half + 0..3}.
  fa_f32x16 acc[NCB];  // O^T: acc[cb] holds columns 32cb.., row qi
  float m_ref, l_lane;
  fa_f32x4 lsum;
  fa_f32x16 sc[NKB];
  fa_u32x4 pf[NKB][2];
  // Start value of the score accumulators: -m_use / c2 in all 16 registers
  // (m_use = m_ref, or 0 while the row has seen no key), so that the matrix
  // core delivers t / c2 with t = s c2 - m_use, the exponent of the
  // probability, and the softmax needs one multiply per score instead of an
  // FMA with the per-row reference (one VGPR operand instead of two: beside
  // the partner wave's matrix products every VALU instruction with two or
  // more VGPR operands costs one extra issue cycle of four).
  fa_f32x16 sc0;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) pf[kb][t] = fa_u32x4{0u, 0u, 0u, 0u};

  // Prologue of the first tile: its first two K and V blocks into ring slots
  // 0 and 1, and zeros in V slot 2, which the first step's (probability 0)
  // P V product reads.  Later tiles find their first two blocks already
  // loaded, and their first P V product reads the previous tile's last V
  // block (finite values, times probability 0).
  issue(lead ? cur.Kh : cur.Vh, my_off, lead ? kbuf(0) : vbuf(0), cur.kv_lo);
  // (at d = 64 the second V block is loaded by the first step)
  if (D != 64 || lead) issue(lead ? cur.Kh : cur.Vh, my_off, lead ? kbuf(1) : vbuf(1), cur.kv_lo + 1);
#pragma unroll
  for (int i = 0; i < TILEB / (NW * 64 * 16); ++i)
    *(FA_AS3 fa_u32x4*)(vbuf(2) + (i * NW * 64 + tid) * 16) = fa_u32x4{0u, 0u, 0u, 0u};
  static_assert(TILEB % (NW * 64 * 16) == 0, "zero fill must cover the slot");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Q fragment ks holds q[qi][16 ks + 8 half .. +7] of the current tile;
  // rows past N read row N-1 (no branch) and are never stored.
  fa_u32x4 qf[NQF];
  auto load_q = [&](int bh_, int q0_) {
    const int row = min(q0_ + wave * FA_ROW_BLOCK + l32, N - 1);
    const unsigned char* qrow = (const unsigned char*)p.q + (size_t)bh_ * head_bytes + (size_t)row * ROWB;
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks) qf[ks] = *(const fa_u32x4*)(qrow + ks * 32 + half * 16);
  };
  load_q(cur.bh, cur.q0);

  int ph = 0;  // ring slot of the current tile's first block
  for (;;) {
    const int bh = cur.bh, q0 = cur.q0;
    const int kv_lo = cur.kv_lo, kv_hi = cur.kv_hi, kv_end = cur.kv_end;
    const int q1 = min(q0 + ROWS_WG, N);
    // this wave's rows qb0 .. qb1-1; this lane's row qi
    const int qb0 = q0 + wave * FA_ROW_BLOCK;
    const int qb1 = min(qb0 + FA_ROW_BLOCK, N);
    const int qi = qb0 + l32;
    (void)q1;
    // Fully visible key blocks of this wave's rows form one range
    // [full_lo, full_hi) (the classes along the keys run SKIP, PARTIAL,
    // FULL, PARTIAL, SKIP); blocks inside it need no classification in the
    // loop.  Both ends are found within eight blocks of the tile's ends,
    // else the range is left empty (every block classified).
    int full_lo = kv_lo, full_hi = kv_end;
    for (int it = 0; it < 8 && full_lo < kv_end &&
                     fa_classify(qb0, qb1, full_lo * BC, BC, N, p.mask_kind, p.window) != FA_TILE_FULL;
         ++it)
      ++full_lo;
    for (int it = 0; it < 8 && full_hi > full_lo &&
                     fa_classify(qb0, qb1, (full_hi - 1) * BC, BC, N, p.mask_kind, p.window) != FA_TILE_FULL;
         ++it)
      --full_hi;
    if (full_lo >= full_hi ||
        fa_classify(qb0, qb1, full_lo * BC, BC, N, p.mask_kind, p.window) != FA_TILE_FULL ||
        fa_classify(qb0, qb1, (full_hi - 1) * BC, BC, N, p.mask_kind, p.window) != FA_TILE_FULL) {
      full_lo = kv_lo;
      full_hi = kv_lo;
    }

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    // reference (base 2) and this lane's sum of unrounded probabilities; the
    // row sums of the rounded ones accumulate on the matrix core, in lsum
    m_ref = FA_NEG_INF;
    l_lane = 0.f;
    lsum = fa_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) sc0[r] = 0.f;

    // Tile-decision record (fa_fwd_record_tiles): the class of key block kt
    // for this wave's row block, plus one.
    auto record = [&](int kt, int cls) {
      if (lane == 0 && qb0 < N)
        p.tiles[((size_t)bh * n_row_blocks + qb0 / FA_ROW_BLOCK) * n_key_blocks + kt] =
            (unsigned char)(cls + 1);
    };
    // Matrix phase of step kt: O^T += V^T P^T for block kt-1 (V slot vs) and
    // S^T = K Q^T for block kt (K slot ks).  It runs in full even where the
    // row block sees no key of one of the blocks (the workgroup's barriers
    // pace every wave anyway, and one code path keeps the registers in
    // place): the probabilities of a skipped block are 0, which adds exactly
    // 0 to O, and the scores of a skipped block are never used.
    auto phase_mfma = [&](int ks, int vs) {
      matrix_phase<DT, D>(acc, sc, lsum, sel, sc0, pf, qf, kbuf(ks), vbuf(vs), kread, vread);
    };
    // Softmax phase of block kt (classification cls).  Fast path (fully
    // visible block, row already started): p = 2^t straight from the scores;
    // a lane's sum of its 32 probabilities at most 2^8 bounds each of them
    // by 2^8 (no score more than 8 base-2 units above the reference).  Exact
    // path (boundary block, a row's first block, or a lane's sum above 2^8,
    // infinite or NaN): mask, row maximum, new reference at the exact
    // maximum, rescale of O and the sums, probabilities again.
    auto phase_softmax = [&](int kt, int cls) {
      if (cls == FA_TILE_SKIP) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) pf[kb][t] = fa_u32x4{0u, 0u, 0u, 0u};
        return;
      }
      float pr[NKB][16];
      float psum = 0.f;
      bool exact = cls == FA_TILE_PARTIAL || __ballot(m_ref == FA_NEG_INF);
      if (!exact) {
        if constexpr (F16_SUMS) {
          // fp16: the probabilities are rounded first and the largest of
          // them bounds the block (no unrounded sum is needed)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) pr[kb][r] = exp2_hw(sc[kb][r] * c2);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              pf[kb][t] = pack8<DT>(&pr[kb][8 * t]);
              // (an empty statement that makes the packed words opaque, so
              // that the maximum reads the registers the products read
              // instead of converting every probability a second time)
              asm("" : "+v"(pf[kb][t]));
            }
          exact = __ballot(max_f16_bits(pf) > FA_F16_BITS_256);
        } else {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              pr[kb][r] = exp2_hw(sc[kb][r] * c2);
              psum = kb == 0 && r == 0 ? pr[kb][r] : psum + pr[kb][r];  // (no 0 + p)
            }
          exact = __ballot(!(psum <= 256.f));
        }
      }
      if (exact) {
        if (cls == FA_TILE_PARTIAL) apply_mask<NKB>(sc, kt * BC, qi, half, N, p.mask_kind, p.window);
        const float m_use = m_ref == FA_NEG_INF ? 0.f : m_ref;
        float mx = FA_NEG_INF;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        mx = pair_max(mx) * c2;  // block maximum of t (-inf: nothing visible)
        const float m_new = fmaxf(m_ref, mx == FA_NEG_INF ? FA_NEG_INF : m_use + mx);
        // O and the sums are rescaled only where the reference rises above
        // a finite one (a row that has seen no key holds zeros); the
        // wavefront skips the multiplies when no lane needs them
        const bool rise = m_new > m_ref && m_ref != FA_NEG_INF;
        if (__ballot(rise)) {
          const float alpha = rise ? exp2_hw(m_ref - m_new) : 1.f;
          l_lane *= alpha;
#pragma unroll
          for (int r = 0; r < 4; ++r) lsum[r] *= alpha;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        }
        m_ref = m_new;
        const float shift = m_ref == FA_NEG_INF ? 0.f : m_use - m_ref;
        psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pr[kb][r] = exp2_hw(__builtin_fmaf(sc[kb][r], c2, shift));
            if constexpr (!F16_SUMS) psum = kb == 0 && r == 0 ? pr[kb][r] : psum + pr[kb][r];
          }
        const float mn = m_ref == FA_NEG_INF ? 0.f : -m_ref * inv_c2;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc0[r] = mn;
      }
      // Row sums.  The output is normalised by the sum of the ROUNDED
      // probabilities (the values the matrix core multiplies V with; summed
      // on the matrix core in the next matrix phase), so output and
      // normaliser use identical weights: constant V comes out exact and a
      // dominant key is selected exactly.  With bf16 inputs lse uses the sum
      // of the unrounded probabilities, which rounding to bf16 would move by
      // up to 2^-9 (relative); fp16 rounding moves it by at most 2^-11, so
      // with fp16 inputs lse comes from the rounded sum as well.
      if (!F16_SUMS || exact) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) pf[kb][t] = pack8<DT>(&pr[kb][8 * t]);
      }
      if constexpr (!F16_SUMS) l_lane += psum;
    };

    // Loads.  The blocks of this tile and the next form one stream through
    // the rings: block kt of this tile lives in slot (ph + kt - kv_lo) mod
    // 3, the next tile's first block in slot (ph + kv_hi - kv_lo) mod 3.
    // For d = 128 (d = 64: below): at the end of its softmax phase kt (where it would otherwise wait at the
    // barrier) a leading wave issues its share of the K block two places
    // further in the stream, a trailing wave its share of that V block, into
    // the slots of block kt-1, whose last reader (matrix phase kt-1 for K,
    // matrix phase kt for V) has passed a barrier since: block kt+2 of this
    // tile, or for kt = kv_hi-2 and kv_hi-1 the next tile's first two
    // blocks; the last step (kt = kv_hi, P V only) issues nothing.  The wait
    // that follows lets these stay in flight, so the wave's loads of the
    // previous step have landed (loads complete in issue order).
    // (each wave loads one matrix: the leading ones K, the trailing ones V;
    // the values are the same in every lane, which readfirstlane makes
    // visible to the compiler, keeping the buffer descriptors in SGPRs)
    const unsigned char* my_cur = uniform_ptr(lead ? cur.Kh : cur.Vh);
    const unsigned char* my_nxt = uniform_ptr(lead ? nxt.Kh : nxt.Vh);
    const int nxt_lo = __builtin_amdgcn_readfirstlane(nxt.kv_lo);
    auto issued = [&](int kt) { return kt + 2 < kv_hi || (kt < kv_hi && has_next); };
    auto issue_step = [&](int kt, int s) {
      if (issued(kt)) {
        const bool here = kt + 2 < kv_hi;
        issue(here ? my_cur : my_nxt, my_off, lead ? kbuf((s + 2) % 3) : vbuf((s + 2) % 3),
              here ? kt + 2 : nxt_lo + (kt + 2 - kv_hi));
      }
    };
    auto wait_step = [&](int kt) {
      if (issued(kt))
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(LPW));
      else
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(0));
    };
    // At d = 64 the matrix phase is the shorter half by far (half the
    // products of d = 128 beside the same softmax), so the copies leave
    // the softmax half altogether: at the end of its matrix phase kt a
    // leading wave issues its shares of both V(kt+1), into the V slot of
    // block kt-2 (last read by matrix phase kt-1 of both groups, which
    // ended at a barrier before this phase), and K(kt+2), into the K slot
    // of block kt-1 (last read by the trailing waves' matrix phase kt-1),
    // then waits for its copies of the previous step, which matrix phase
    // kt+1 reads first.  The trailing waves copy nothing.  In the V stream
    // position kt+1 is this tile's block or, for kt = kv_hi-1, the next
    // tile's first; the next tile's second is loaded by its own first step.
    // (A later tile's first K copy waits for a barrier: see the step loop.)
    const unsigned char* k_cur = uniform_ptr(cur.Kh);
    const unsigned char* k_nxt = uniform_ptr(nxt.Kh);
    const unsigned char* v_cur = uniform_ptr(cur.Vh);
    const unsigned char* v_nxt = uniform_ptr(nxt.Vh);
    auto issue_k64 = [&](int kt, int s) {
      const bool here = kt + 2 < kv_hi;
      issue(here ? k_cur : k_nxt, koff, kbuf((s + 2) % 3), here ? kt + 2 : nxt_lo + (kt + 2 - kv_hi));
    };
    auto matrix_end64 = [&](int kt, int s) {
      const bool iv = kt + 1 < kv_hi || (kt < kv_hi && has_next);
      const bool ik = issued(kt) && !(kt == kv_lo && tile_k > 0);
      if (iv) {
        const bool here = kt + 1 < kv_hi;
        issue(here ? v_cur : v_nxt, voff, vbuf((s + 1) % 3), here ? kt + 1 : nxt_lo);
      }
      if (ik) issue_k64(kt, s);
      if (iv && ik)
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(2 * LPW));
      else if (iv || ik)
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(LPW));
      else
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(0));
    };

    // Every wave runs, for kt = kv_lo .. kv_hi, matrix phase kt (scores of
    // block kt, P V of block kt-1) and softmax phase kt.
    //
    // d = 128: two workgroup barriers per step, one after each phase.  The
    // trailing waves pass one barrier before their first step, the leading
    // ones one after their last, so a trailing wave's matrix phase kt runs
    // beside the leading waves' softmax phase kt, and its softmax phase kt
    // beside their matrix phase kt+1.  In half steps h (the intervals
    // between consecutive barriers; h = 2(kt - kv_lo) is the leading waves'
    // matrix phase kt): matrix phase kt reads K(kt) and V(kt-1) in h and
    // h + 1; K(kt+2) is issued at the end of h + 1 and V(kt+2) at the end of
    // h + 2, after every wave has finished its LDS reads of the slots they
    // replace (lgkmcnt(0) before each barrier); K(kt+1) and V(kt+1), issued
    // in the previous step, are waited for before the barriers that end
    // h + 1 and h + 2, ahead of matrix phases kt+1 and kt+2 that read them.
    //
    // d = 64 (ONE_BARRIER): one barrier per step, after the softmax phase in
    // a leading wave and between the two phases in a trailing one.  In
    // interval I(kt) (between the barriers of steps kt-1 and kt) a leading
    // wave runs matrix phase kt and then softmax phase kt, a trailing wave
    // softmax phase kt-1 and then matrix phase kt: program order keeps the
    // two waves of a SIMD in opposite phases, and since the softmax is the
    // longer phase by far at d = 64, a leading wave starts its softmax as
    // soon as its products are issued instead of waiting at a barrier for
    // its partner's softmax.  The copies (issued at the end of a leading
    // wave's matrix phase, described above) keep their slots: V(kt+1) goes
    // into the slot of V(kt-2), last read in I(kt-1), K(kt+2) into that of
    // K(kt-1), also last read in I(kt-1); the wait that follows covers the
    // copies of step kt-1, read from I(kt+1) on.  On a later tile's first
    // step the K slot being replaced holds the leading waves' staged output
    // of the previous tile, which the other leading waves may still be
    // reading back: that copy is issued at the start of the next step,
    // after the barrier, and the next step's wait covers it.  On a tile's
    // first step both groups start with a matrix phase.
    //
    // Tiles follow each other with the same barrier count in both groups.
    auto step = [&](int kt, int s) {
      int cls_cur = FA_TILE_FULL;
      if (kt < full_lo || kt >= full_hi) {
        cls_cur = kt < kv_end ? fa_classify(qb0, qb1, kt * BC, BC, N, p.mask_kind, p.window)
                              : FA_TILE_SKIP;
        if (p.tiles && kt < kv_end) record(kt, cls_cur);
      }
      if constexpr (ONE_BARRIER) {
        if (lead && tile_k > 0 && kt == kv_lo + 1 && issued(kv_lo)) issue_k64(kv_lo, (s + 2) % 3);
      }
      phase_mfma(s, (s + 2) % 3);
      if (D == 64 && lead) matrix_end64(kt, s);
      if (!ONE_BARRIER || !lead) {
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_LGKM0);
        barrier_nofence();
      }
      phase_softmax(kt, cls_cur);
      if constexpr (D != 64) {
        issue_step(kt, s);
        wait_step(kt);
      }
      if (!ONE_BARRIER || lead) {
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_LGKM0);
        barrier_nofence();
      }
    };

    if (p.tiles)
      for (int kt = full_lo; kt < full_hi; ++kt) record(kt, FA_TILE_FULL);
    if (!ONE_BARRIER && !lead) barrier_nofence();
    // steps kt = kv_lo .. kv_hi; step kt uses ring slot (ph + kt - kv_lo)
    // mod 3 (entered at the slot of the tile's first block)
    {
      int kt = kv_lo;
      int entry = ph;
      for (;;) {
        if (entry == 0) {
          step(kt, 0);
          if (++kt > kv_hi) break;
        }
        if (entry <= 1) {
          step(kt, 1);
          if (++kt > kv_hi) break;
        }
        step(kt, 2);
        if (++kt > kv_hi) break;
        entry = 0;
      }
    }
    // The next tile's Q rows: loaded before this tile's output is stored
    // (and, with two barriers per step, before the leading waves' last
    // barrier, where they wait for the trailing waves' last softmax phase).
    // A load inside the step loop would make the compiler wait for it
    // before every score product.
    if (has_next) load_q(nxt.bh, nxt.q0);
    if (!ONE_BARRIER && lead) barrier_nofence();
    if constexpr (OUT_F32) {
      store_output<DT, D, OUT_F32>(p, acc, m_ref, F16_SUMS ? lsum[0] : pair_sum(l_lane), lsum[0], bh, qi, half);
    } else {
      // Scratch for the restaged output: ring slot (ph + kv_hi - kv_lo + 2)
      // mod 3, which holds this tile's last block -- K no longer read, V
      // read next only by the next tile's first step, with probability 0
      // (any finite values do) -- and is refilled no earlier than the end
      // of that step's softmax phase.  Waves 0-3 use the K slot, 4-7 the V
      // slot, 16 rows each (4 KB at d = 128, 2 KB at d = 64: a slot holds 64
      // rows).
      static_assert(NL * 16 * ROWB <= TILEB, "four 16-row stages must fit in one slot");
      const int sl = (ph + (kv_hi - kv_lo) + 2) % 3;
      FA_AS3 unsigned char* stage = (lead ? kbuf(sl) : vbuf(sl)) + (wave % NL) * (16 * ROWB);
      store_output_staged<DT, D>(p, acc, m_ref, F16_SUMS ? lsum[0] : pair_sum(l_lane), lsum[0], bh, qb0,
                                 lane, stage);
    }

    if (!has_next) break;
    ph = (ph + (kv_hi - kv_lo)) % 3;
    cur = nxt;
    ++tile_k;
    has_next = persist_tile(p, tile_k + 1, nbh, nq0, ROWS_WG);
    if (has_next) nxt = make_tile(nbh, nq0);
  }
}

// ---------------------------------------------------------------------------
// bf16 / f16 kernel, head dim 256
// ---------------------------------------------------------------------------
// Four wavefronts of 32 query rows, one per SIMD: at d = 256 a wave's output
// accumulators alone take 128 registers (kept in AGPRs) and its Q fragments
// 64, so two waves of this size do not fit on a SIMD and the ping-pong of
// the kernel above is not available.  Each wave overlaps its own softmax
// with its own matrix products instead.  Step kt: the score products of
// block kt; then the P V products of block kt-1 (and its rounded row sums)
// issued one by one between the instructions of block kt's fast softmax;
// then, if needed, the exact path (which rescales O after the P V products
// of block kt-1 have landed).  K and V are double-buffered in LDS
// (128 KiB): at the top of step kt every wave issues its share of K(kt+1)
// and V(kt), into the slots of K(kt-1) and V(kt-2), whose last readers
// finished before the barrier that ended step kt-1.
template <int DT, bool OUT_F32>
__global__ void __launch_bounds__(FA_WAVES_WIDE * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
fa_fwd16_wide_kernel(FaFwdParams p) {
  constexpr int D = 256;
  constexpr int NW = FA_WAVES_WIDE;
  constexpr int ROWS_WG = NW * FA_ROW_BLOCK;
  constexpr int BC = FA_KEYS_16;   // keys per block
  constexpr int NKB = BC / 32;     // 32-key groups per block
  constexpr int NCB = D / 32;      // 32-column output blocks
  constexpr int NQF = D / 16;      // 16-deep slices of the QK^T contraction
  constexpr int NQK = NKB * NQF;   // score products per block
  constexpr int NPV = NKB * 2 * NCB;  // P V products per block
  constexpr int ROWB = 2 * D;      // bytes of one K/V row
  constexpr int TILEB = BC * ROWB; // bytes of one K or V block
  constexpr int LPW = TILEB / (NW * 1024);  // one-kilobyte loads per wave per block
  static_assert(NW == 4 && LPW == 8 && NKB == 2, "load layout below: 8 pieces of 2 rows per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILEB], ks1[TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[TILEB], vs1[TILEB];
  auto kbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? ks0 : ks1); };
  auto vbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? vs0 : vs1); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int N = p.N;

  int bh, q0;
  work_item<ROWS_WG>(p, bh, q0);
  const int q1 = min(q0 + ROWS_WG, N);
  const int qb0 = q0 + wave * FA_ROW_BLOCK;
  const int qb1 = min(qb0 + FA_ROW_BLOCK, N);
  const int qi = qb0 + l32;

  const size_t head_bytes = (size_t)N * ROWB;
  const size_t kv_bytes = (size_t)(bh / p.kv_group) * head_bytes;
  const unsigned char* Qh = (const unsigned char*)p.q + (size_t)bh * head_bytes;
  const unsigned char* Kh = (const unsigned char*)p.k + kv_bytes;
  const unsigned char* Vh = (const unsigned char*)p.v + kv_bytes;

  int kv_lo, kv_hi;
  fa_key_block_range(q0, q1, BC, N, p.mask_kind, p.window, &kv_lo, &kv_hi);

  fa_u32x4 qf[NQF];  // q[qi][16 ks + 8 half .. +7]; rows past N read row N-1
  {
    const unsigned char* qrow = Qh + (size_t)min(qi, N - 1) * ROWB;
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks) qf[ks] = *(const fa_u32x4*)(qrow + ks * 32 + half * 16);
  }

  // Loads: piece i (0..7) of wave w is rows r0 = 2w + 8(i mod 2) + 16(i/2)
  // and r0 + 1 (lanes 0-31 and 32-63, 16 bytes each).  The swizzles depend
  // on row bits 0-3 only, which 16(i/2) leaves unchanged: two global offsets
  // per matrix serve all eight pieces, the rest goes into the scalar offset
  // (which the descriptor's range check includes).
  unsigned koff[2], voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 2 * wave + 8 * j + half;
    koff[j] = r * ROWB + 16 * (l32 ^ kswz<D>(r));
    voff[j] = r * ROWB + 16 * (l32 ^ vswz<D>(r));
  }
  unsigned kread[NQF], vread[NCB];
#pragma unroll
  for (int s = 0; s < NQF; ++s) kread[s] = l32 * ROWB + 16 * ((2 * s + half) ^ kswz<D>(l32));
  {
    const int g = lane >> 4, t = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      vread[cb] = (4 * half + t) * ROWB + 64 * (cb ^ t) + 32 * (g & 1) + 8 * q;
  }

  // K or V block kt -> LDS slot (descriptor ends at key N: rows past N read 0)
  auto issue = [&](const unsigned char* base, unsigned off0, unsigned off1,
                   FA_AS3 unsigned char* dst, int kt) {
    const int k0 = kt * BC;
    const int nb = (min(N - k0, BC)) * ROWB;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)k0 * ROWB), 0, nb, FA_BUF_WORD3);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r0 = 2 * wave + 8 * (i & 1) + 16 * (i >> 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_AS3 void*)(dst + r0 * ROWB), 16,
                                               (int)((i & 1) ? off1 : off0), (i >> 1) * 16 * ROWB,
                                               0, 0);
    }
  };

  fa_f32x16 acc[NCB];  // O^T: acc[cb] holds columns 32cb.., row qi
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    asm volatile("" : "+a"(acc[cb]));  // placement only: the matrix core's AGPRs
  }
  float m_ref = FA_NEG_INF, l_lane = 0.f;
  fa_f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
  const fa_u32x4 sel = rowsum_selector<DT>(lane);
  const float c2 = p.scale_log2;
  const float inv_c2 = 1.f / p.scale_log2;
  const int n_row_blocks = (N + FA_ROW_BLOCK - 1) / FA_ROW_BLOCK;
  const int n_key_blocks = (N + BC - 1) / BC;

  // score accumulators start from -m_use / c2 (see the kernel above)
  float sc_start = 0.f;
  fa_f32x16 sc[NKB];
  fa_u32x4 pf[NKB][2];  // rounded probabilities of the previous block
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) pf[kb][t] = fa_u32x4{0u, 0u, 0u, 0u};

  // One step (K slot s holds K(kt), V slot s holds V(kt-1)).
  auto step = [&](int kt, int s) {
    int cls = FA_TILE_SKIP;
    if (kt < kv_hi) {
      cls = fa_classify(qb0, qb1, kt * BC, BC, N, p.mask_kind, p.window);
      if (p.tiles && lane == 0 && qb0 < N)
        p.tiles[((size_t)bh * n_row_blocks + qb0 / FA_ROW_BLOCK) * n_key_blocks + kt] =
            (unsigned char)(cls + 1);
    }
    if (kt + 1 < kv_hi) issue(Kh, koff[0], koff[1], kbuf(s ^ 1), kt + 1);
    if (kt < kv_hi) issue(Vh, voff[0], voff[1], vbuf(s ^ 1), kt);

    // S^T = K Q^T over block kt (stale and unused in the step after the last
    // block); LDS operands read FA_OPND_AHEAD products ahead
    {
      constexpr int R = FA_OPND_AHEAD;
      fa_u32x4 opnd[R + 1];
      const FA_AS3 unsigned char* kcur = kbuf(s);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = sc_start;
#pragma unroll
      for (int i = 0; i < NQK + R; ++i) {
        if (i >= R) {
          const int j = i - R;
          sc[j % 2] = mma16<DT>(opnd[j % (R + 1)], qf[j / 2], sc[j % 2]);
        }
        if (i < NQK)
          opnd[i % (R + 1)] = *(const FA_AS3 fa_u32x4*)(kcur + (i % 2) * 32 * ROWB + kread[i / 2]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // O^T += V^T P^T over block kt-1 (V slot s; probabilities 0 in the first
    // step, whose slot holds zeros) and its rounded row sums, interleaved with
    // the fast softmax of block kt: p = 2^t straight from the scores
    float pr[NKB][16];
    float psum = 0.f;
    {
      // V^T operand of product j (output block j mod NCB, keys of P^T
      // operand (kb, t)), read FA_OPND_AHEAD products ahead
      constexpr int R = FA_OPND_AHEAD;
      fa_u32x4 opnd[R + 1];
      const FA_AS3 unsigned char* vcur = vbuf(s);
#pragma unroll
      for (int i = 0; i < NPV + R; ++i) {
        if (i < NPV) {
          const int cb = i % NCB, kb = i / NCB / 2, t = i / NCB % 2;
          const FA_AS3 unsigned char* vp = vcur + (32 * kb + 16 * t) * ROWB + vread[cb];
          const fa_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)vp);
          const fa_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)(vp + 8 * ROWB));
          const fa_u32x2 l2 = __builtin_bit_cast(fa_u32x2, lo), h2 = __builtin_bit_cast(fa_u32x2, hi);
          opnd[i % (R + 1)] = fa_u32x4{l2.x, l2.y, h2.x, h2.y};
        }
        if (i >= R) {
          const int j = i - R, cb = j % NCB, kb = j / NCB / 2, t = j / NCB % 2;
          acc[cb] = mma16<DT>(opnd[j % (R + 1)], pf[kb][t], acc[cb]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) lsum = rowsum_mma<DT>(sel, pf[kb][t], lsum);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[kb][r] = exp2_hw(sc[kb][r] * c2);
          psum += pr[kb][r];
        }
      // issue order: the first R operand reads, then per product one
      // operand read R ahead, the product and a share of the softmax
#pragma unroll
      for (int j = 0; j < R; ++j) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int j = 0; j < NPV + 4; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix product
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
      }
    }

    const bool exact = cls == FA_TILE_PARTIAL || __ballot(m_ref == FA_NEG_INF) ||
                       __ballot(!(psum <= 256.f));
    if (cls == FA_TILE_SKIP) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) pf[kb][t] = fa_u32x4{0u, 0u, 0u, 0u};
    } else {
      if (exact) {
        if (cls == FA_TILE_PARTIAL) apply_mask<NKB>(sc, kt * BC, qi, half, N, p.mask_kind, p.window);
        const float m_use = m_ref == FA_NEG_INF ? 0.f : m_ref;
        float mx = FA_NEG_INF;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        mx = pair_max(mx) * c2;
        const float m_new = fmaxf(m_ref, mx == FA_NEG_INF ? FA_NEG_INF : m_use + mx);
        if (__ballot(m_new > m_ref)) {
          // rescale O and the sums, which now hold block kt-1
          const float alpha = m_new > m_ref ? (m_ref == FA_NEG_INF ? 0.f : exp2_hw(m_ref - m_new)) : 1.f;
          l_lane *= alpha;
#pragma unroll
          for (int r = 0; r < 4; ++r) lsum[r] *= alpha;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        }
        m_ref = m_new;
        const float shift = m_ref == FA_NEG_INF ? 0.f : m_use - m_ref;
        psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pr[kb][r] = exp2_hw(__builtin_fmaf(sc[kb][r], c2, shift));
            psum += pr[kb][r];
          }
        sc_start = m_ref == FA_NEG_INF ? 0.f : -m_ref * inv_c2;
      }
      // O is normalised by the sum of the rounded probabilities (on the
      // matrix core), lse by the sum of the unrounded ones
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) pf[kb][t] = pack8<DT>(&pr[kb][8 * t]);
      l_lane += psum;
    }
    // this step's loads have landed and every wave is done with its LDS
    // reads before the next step reads them or overwrites the slots read here
    __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(0));
    barrier_nofence();
  };

  // Every workgroup has at least one key block (the diagonal is visible).
  // Prologue: K of the first block, and zeros in the V slot that the first
  // step's (probability 0) P V products read.
  issue(Kh, koff[0], koff[1], kbuf(0), kv_lo);
#pragma unroll
  for (int i = 0; i < TILEB / (NW * 64 * 16); ++i)
    *(FA_AS3 fa_u32x4*)(vbuf(0) + (i * NW * 64 + tid) * 16) = fa_u32x4{0u, 0u, 0u, 0u};
  static_assert(TILEB % (NW * 64 * 16) == 0, "zero fill must cover the slot");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = kv_lo;;) {
    step(kt, 0);
    if (++kt > kv_hi) break;
    step(kt, 1);
    if (++kt > kv_hi) break;
  }
  store_output<DT, D, OUT_F32>(p, acc, m_ref, pair_sum(l_lane), lsum[0], bh, qi, half);
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2f32; one contraction element per lane)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(FA_WAVES_32 * 64)
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
  work_item<FA_WAVES_32 * FA_ROW_BLOCK>(p, bh, q0);
  const int q1 = min(q0 + FA_WAVES_32 * FA_ROW_BLOCK, N);
  const int qw0 = q0 + wave * FA_ROW_BLOCK;
  const int qw1 = min(qw0 + FA_ROW_BLOCK, N);
  const int qi = qw0 + l32;
  const size_t head = (size_t)bh * N * D;
  const size_t kv_head = (size_t)(bh / p.kv_group) * N * D;  // see the 16-bit kernel
  const float* Qh = (const float*)p.q + head;
  const float* Kh = (const float*)p.k + kv_head;
  const float* Vh = (const float*)p.v + kv_head;

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
  const int n_row_blocks = (N + FA_ROW_BLOCK - 1) / FA_ROW_BLOCK;
  const int n_key_blocks = (N + BC - 1) / BC;
  const int row_block = qw0 / FA_ROW_BLOCK;

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
  store_output<0, D, true>(p, acc, m_ref, pair_sum(l_lane), pair_sum(lq_lane), bh, qi, half);
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
    hipLaunchKernelGGL((fa_fwd32_kernel<D>), grid, dim3(FA_WAVES_32 * 64), 0, stream, p);
  else if constexpr (D == 256)
    hipLaunchKernelGGL((fa_fwd16_wide_kernel<DT, OUT_F32>), grid, dim3(FA_WAVES_WIDE * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fa_fwd16_kernel<DT, D, OUT_F32>),
                       dim3((unsigned)(p.n_groups * p.wg_per_group)), dim3(FA_WAVES_16 * 64), 0,
                       stream, p);
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
      if (d == 256) return of32 ? launch<1, 256, true>(p, stream) : launch<1, 256, false>(p, stream);
      return of32 ? launch<1, 128, true>(p, stream) : launch<1, 128, false>(p, stream);
    default:
      if (d == 64) return of32 ? launch<2, 64, true>(p, stream) : launch<2, 64, false>(p, stream);
      if (d == 256) return of32 ? launch<2, 256, true>(p, stream) : launch<2, 256, false>(p, stream);
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
