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
// gfx950 mapping (one workgroup = 4 wavefronts of 64 lanes, 128 query rows):
//  * Each wavefront owns 32 query rows for the whole key loop.  Its Q rows
//    stay in VGPRs as matrix-core operands, loaded once from HBM.
//  * K/V blocks are streamed HBM -> VGPR staging -> LDS with 16-byte loads,
//    double-buffered: the loads of block t+1 are in flight while block t is
//    computed, one barrier per block.  K is kept row-major in LDS; V is
//    written transposed (key index contiguous) so that it can feed the
//    matrix core as the A operand of O^T = V^T P^T.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: in the 32x32 accumulator every lane then
//    holds one query row (lane mod 32) and 16 of its keys, so the row max and
//    row sum are in-lane reductions plus a single exchange with lane ^ 32.
//  * The probabilities are rounded to the input type and used straight from
//    the accumulator registers as the B operand of the P V product: the
//    contraction index is permuted identically in both operands, so no data
//    moves between the two matrix products.
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
// fp32 inputs use v_mfma_f32_32x32x2f32 with the same structure (V row-major
// in LDS, since that instruction takes one contraction element per lane).
#include <hip/hip_runtime.h>

#include "fa_kernels.h"
#include "tile_class.h"

typedef __bf16 fa_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 fa_f16x8 __attribute__((ext_vector_type(8)));
typedef float fa_f32x16 __attribute__((ext_vector_type(16)));
typedef float fa_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int fa_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int fa_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short fa_u16;

#define FA_NEG_INF (-__builtin_inff())
#define FA_LN2 0.69314718055994530942f
#define FA_RESCALE_THRESHOLD 8.0f

namespace {

// ---------------------------------------------------------------------------
// matrix-core products and element conversions
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

// ---------------------------------------------------------------------------
// geometry
// ---------------------------------------------------------------------------
template <int DT, int D>
struct Geo {
  static constexpr bool F32 = (DT == 0);
  static constexpr int BC = F32 ? FA_KEYS_32 : FA_KEYS_16;  // keys per block
  static constexpr int NKB = BC / 32;                        // 32-key groups
  static constexpr int ESZ = F32 ? 4 : 2;                    // element bytes
  static constexpr int EPC = 16 / ESZ;                       // elements / 16B
  static constexpr int CPR = D / EPC;                        // 16B chunks / row
  static constexpr int LPT = BC * CPR / 256;                 // loads / thread
  static constexpr int KLD = D + EPC;                        // K row stride (elems)
  static constexpr int VLD = F32 ? (D + EPC) : (BC + 4);     // V / V^T row stride
  static constexpr int VROWS = F32 ? BC : D;
  static constexpr int KBYTES = BC * KLD * ESZ;              // one K buffer
  static constexpr int VBYTES = VROWS * VLD * ESZ;           // one V buffer
  static constexpr int LDS = 2 * (KBYTES + VBYTES);
  // wavefronts per SIMD the register budget is sized for (2 -> 256 VGPRs)
  static constexpr int WPE = (F32 && D == 128) ? 1 : 2;
  static_assert(LPT * (256 / CPR) == BC, "staging must cover the block");
  static_assert(F32 || LPT == 2 || LPT == 4, "transpose packs 2 or 4 rows");
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int DT, int D, bool OUT_F32>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(Geo<DT, D>::WPE, Geo<DT, D>::WPE)))
fa_fwd_kernel(FaFwdParams p) {
  using G = Geo<DT, D>;
  constexpr int BC = G::BC;
  constexpr int NKB = G::NKB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int N = p.N;

  // ---- work item: (batch*head, row tile) --------------------------------
  const int T = p.n_row_tiles;
  const int b = blockIdx.x;
  int bh, rank;
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
  const int q0 = qt * FA_ROWS_PER_WG;
  const int q1 = min(q0 + FA_ROWS_PER_WG, N);
  const int qw0 = q0 + wave * FA_ROWS_PER_WAVE;
  const int qw1 = min(qw0 + FA_ROWS_PER_WAVE, N);
  const int qi = qw0 + l32;  // this lane's query row

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const unsigned char* Qb = (const unsigned char*)p.q + head_off * G::ESZ;
  const unsigned char* Kb = (const unsigned char*)p.k + head_off * G::ESZ;
  const unsigned char* Vb = (const unsigned char*)p.v + head_off * G::ESZ;

  int kv_lo, kv_hi;
  fa_key_block_range(q0, q1, BC, N, p.mask_kind, p.window, &kv_lo, &kv_hi);

  // ---- Q operand fragments, loaded once -----------------------------------
  // 16-bit: fragment ks holds q[qi][16 ks + 8 half .. +7]
  // f32:    fragment ks holds q[qi][2 ks + half]
  constexpr int NQF = G::F32 ? D / 2 : D / 16;
  fa_u32x4 qf16[G::F32 ? 1 : NQF];
  float qf32[G::F32 ? NQF : 1];
  // Rows past N read row N-1 instead (no branch); their results are never
  // stored.
  const size_t qrow = (size_t)min(qi, N - 1) * D;
  if constexpr (G::F32) {
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks) qf32[ks] = ((const float*)Qb)[qrow + 2 * ks + half];
  } else {
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks)
      qf16[ks] = *(const fa_u32x4*)(Qb + (qrow + ks * 16 + half * 8) * 2);
  }

  // ---- K/V staging -------------------------------------------------------
  const int cc = tid % G::CPR;  // 16-byte chunk within a row
  const int jg = tid / G::CPR;  // row group: rows jg*LPT .. jg*LPT+LPT-1
  fa_u32x4 kst[G::LPT], vst[G::LPT];

  // Keys past N load row N-1 (no branch): such keys only occur in boundary
  // blocks, where the mask gives them probability exactly 0, and the finite
  // values loaded there contribute 0 * v = 0 to the product with V.
  auto gload = [&](int kt) {
    const int k0 = kt * BC;
#pragma unroll
    for (int r = 0; r < G::LPT; ++r) {
      const int j = min(k0 + jg * G::LPT + r, N - 1);
      const size_t off = ((size_t)j * D + cc * G::EPC) * G::ESZ;
      kst[r] = *(const fa_u32x4*)(Kb + off);
      vst[r] = *(const fa_u32x4*)(Vb + off);
    }
  };

  auto lstore = [&](int buf) {
    unsigned char* kbuf = smem + buf * G::KBYTES;
    unsigned char* vbuf = smem + 2 * G::KBYTES + buf * G::VBYTES;
#pragma unroll
    for (int r = 0; r < G::LPT; ++r)
      *(fa_u32x4*)(kbuf + ((jg * G::LPT + r) * G::KLD + cc * G::EPC) * G::ESZ) = kst[r];
    if constexpr (G::F32) {
#pragma unroll
      for (int r = 0; r < G::LPT; ++r)
        *(fa_u32x4*)(vbuf + ((jg * G::LPT + r) * G::VLD + cc * G::EPC) * G::ESZ) = vst[r];
    } else {
      // V^T[c][j]: the LPT rows of this thread become LPT consecutive keys of
      // each of its 8 columns.
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int c = cc * 8 + 2 * w;
        unsigned char* lo_dst = vbuf + (c * G::VLD + jg * G::LPT) * 2;
        unsigned char* hi_dst = lo_dst + G::VLD * 2;
        if constexpr (G::LPT == 4) {
          fa_u32x2 lo, hi;
          lo.x = (vst[0][w] & 0xffffu) | (vst[1][w] << 16);
          lo.y = (vst[2][w] & 0xffffu) | (vst[3][w] << 16);
          hi.x = (vst[0][w] >> 16) | (vst[1][w] & 0xffff0000u);
          hi.y = (vst[2][w] >> 16) | (vst[3][w] & 0xffff0000u);
          *(fa_u32x2*)lo_dst = lo;
          *(fa_u32x2*)hi_dst = hi;
        } else {
          *(unsigned int*)lo_dst = (vst[0][w] & 0xffffu) | (vst[1][w] << 16);
          *(unsigned int*)hi_dst = (vst[0][w] >> 16) | (vst[1][w] & 0xffff0000u);
        }
      }
    }
  };

  // ---- running state ----------------------------------------------------
  fa_f32x16 acc[D / 32];  // O^T: block cb holds columns 32cb.., row qi
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float m_ref = FA_NEG_INF;  // reference maximum (base-2 scaled units)
  float l_lane = 0.f;        // this lane's part of the exponent sum
  float lq_lane = 0.f;       // same, of the probabilities as rounded for P V
  const float c2 = p.scale_log2;

  const int n_row_blocks = (N + FA_ROWS_PER_WAVE - 1) / FA_ROWS_PER_WAVE;
  const int n_key_blocks = (N + BC - 1) / BC;
  const int row_block = qw0 / FA_ROWS_PER_WAVE;

  // Every workgroup has at least one key block: row q0 < N always sees key
  // q0 itself (the diagonal is visible under every mask).
  gload(kv_lo);
  lstore(0);
  // All loads issued so far (Q fragments included) have landed: the loop's
  // prefetch of the next block then never has to wait behind them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kt = kv_lo; kt < kv_hi; ++kt) {
    const int buf = (kt - kv_lo) & 1;
    const bool has_next = kt + 1 < kv_hi;
    const int k0 = kt * BC;
    const int cls = fa_classify(qw0, qw1, k0, BC, N, p.mask_kind, p.window);
    if (p.tiles && lane == 0 && qw0 < N)
      p.tiles[((size_t)bh * n_row_blocks + row_block) * n_key_blocks + kt] =
          (unsigned char)(cls + 1);
    if (has_next) gload(kt + 1);

    if (cls != FA_TILE_SKIP) {
      const unsigned char* kbuf = smem + buf * G::KBYTES;
      const unsigned char* vbuf = smem + 2 * G::KBYTES + buf * G::VBYTES;

      // ---- S^T = K Q^T: s[kb][r] is key k0 + 32kb + 8(r/4) + 4half + r%4
      fa_f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        if constexpr (G::F32) {
#pragma unroll
          for (int ks = 0; ks < NQF; ++ks) {
            const float a = *(const float*)(kbuf + ((kb * 32 + l32) * G::KLD + 2 * ks + half) * 4);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf32[ks], s[kb], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < NQF; ++ks) {
            const fa_u32x4 a = *(const fa_u32x4*)(kbuf + ((kb * 32 + l32) * G::KLD + ks * 16 + half * 8) * 2);
            s[kb] = mma16<DT>(a, qf16[ks], s[kb]);
          }
        }
      }

      // ---- mask (boundary blocks only): invisible scores become -inf, which
      // the exponential below maps to exactly 0 (scale_log2 > 0)
      if (cls == FA_TILE_PARTIAL) {
        // row qi sees keys jlo..jhi; key j is visible iff 0 <= j-jlo <= span
        const int jhi = p.mask_kind == FA_MASKK_NONE ? N - 1 : min(qi, N - 1);
        const int jlo = p.mask_kind == FA_MASKK_SLIDING ? max(qi - p.window + 1, 0) : 0;
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

      // ---- row maximum over this block (both lane halves)
      float mx = FA_NEG_INF;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = mx * c2;

      // ---- raise the reference maximum when a row outgrows it
      const bool need = mxs > m_ref + FA_RESCALE_THRESHOLD;
      if (__ballot(need)) {
        const float m_new = fmaxf(m_ref, mxs);
        const float alpha = (m_new == m_ref) ? 1.f : exp2_hw(m_ref - m_new);
        m_ref = m_new;
        l_lane *= alpha;
        lq_lane *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
      }
      const float m_use = (m_ref == FA_NEG_INF) ? 0.f : m_ref;

      // ---- probabilities p = 2^(s*scale*log2e - m)
      float pr[NKB][16];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[kb][r] = exp2_hw(__builtin_fmaf(s[kb][r], c2, -m_use));

      // ---- O^T += V^T P^T
      if constexpr (G::F32) {
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) psum += pr[0][r];
        l_lane += psum;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jrow = 8 * (r >> 2) + 4 * half + (r & 3);
            const float a = *(const float*)(vbuf + (jrow * G::VLD + cb * 32 + l32) * 4);
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pr[0][r], acc[cb], 0, 0, 0);
          }
      } else {
        // B operand (kb, t): slots 0..7 = registers 8t..8t+7, i.e. keys
        // 32kb + 16t + {4half + 0..3, 8 + 4half + 0..3}; the A operand takes
        // V^T at the same keys.
        // Two row sums.  The output is normalised by the sum of the ROUNDED
        // probabilities (the values the matrix core multiplies V with; two per
        // dot2 instruction), so output and normaliser use identical weights:
        // constant V comes out exact and a dominant key is selected exactly.
        // lse uses the sum of the unrounded fp32 probabilities, which rounding
        // to 16 bits would otherwise shift by up to 2^-9.
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
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const unsigned char* row = vbuf + ((cb * 32 + l32) * G::VLD + kb * 32 + 16 * t + 4 * half) * 2;
              const fa_u32x2 lo = *(const fa_u32x2*)row;
              const fa_u32x2 hi = *(const fa_u32x2*)(row + 16);
              const fa_u32x4 a = {lo.x, lo.y, hi.x, hi.y};
              acc[cb] = mma16<DT>(a, pf[kb][t], acc[cb]);
            }
      }
    }

    if (has_next) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = (m + log2 l) ln 2 ----------------------
  if constexpr (G::F32) lq_lane = l_lane;  // fp32 products use p unrounded
  const float l_tot = l_lane + __shfl_xor(l_lane, 32);
  const float lq_tot = lq_lane + __shfl_xor(lq_lane, 32);
  const float inv = lq_tot > 0.f ? 1.f / lq_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * FA_LN2 : FA_NEG_INF;
  if (qi < N) {
    unsigned char* Ob = (unsigned char*)p.o + head_off * (OUT_F32 ? 4 : 2);
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = cb * 32 + 8 * g + 4 * half;
        const float o0 = acc[cb][4 * g] * inv, o1 = acc[cb][4 * g + 1] * inv;
        const float o2 = acc[cb][4 * g + 2] * inv, o3 = acc[cb][4 * g + 3] * inv;
        if constexpr (OUT_F32) {
          const fa_f32x4 val = {o0, o1, o2, o3};
          *(fa_f32x4*)(Ob + ((size_t)qi * D + c) * 4) = val;
        } else {
          *(fa_u32x2*)(Ob + ((size_t)qi * D + c) * 2) = pack4<DT>(o0, o1, o2, o3);
        }
      }
    if (half == 0) p.lse[(size_t)bh * N + qi] = lse;
  }
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

template <int DT, int D, bool OUT_F32>
hipError_t launch(const FaFwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.BH * p.n_row_tiles));
  hipLaunchKernelGGL((fa_fwd_kernel<DT, D, OUT_F32>), grid, dim3(256), 0, stream, p);
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
