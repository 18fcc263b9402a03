// Fused exact attention forward pass with 8-bit floating-point inputs, gfx950.
//
// The method is that of the 16-bit kernel in fa_fwd.hip ("FlashAttention
// (NL)": key blocks streamed through on-chip memory, section "Tiling en
// blokgewijze verwerking"; running maximum and exponent sum, section "Online
// berekening van Softmax"; one fused kernel, section "Samensmelting van
// bewerkingen in één CUDA-kernel"), with Q, K and V in FP8, the format the
// section "FlashAttention-3 (2024)" of the same page names for Hopper.  On
// gfx950 that is OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits; largest finite 448, no infinities), and both matrix products run on
// v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3 -> fp32), twice the rate of the
// 16-bit products.
//
// Ping-pong of the two wavefronts of a SIMD, tile classes and the
// persistent work order are those of fa_fwd16_kernel (fa_fwd.hip), without
// its K/V stream across tiles (each tile starts its own); the K/V rings have
// four slots (8 KB blocks), and the leading wavefronts load both K and V at the start of
// their matrix phase: here the softmax phase, not the matrix phase, is the
// longer half of a step, so its wavefronts issue no loads.
// What differs:
//  * S^T = K Q^T contracts 64 head-dim elements per product.  Lane (row
//    l32, half h) of both operands holds elements 64s + 32h .. 64s + 32h + 31
//    of its row: the product pairs byte p of A's lane half h with byte p of
//    B's lane half h, so any split of the contraction that both operands
//    share gives the dot product.
//  * O^T += V^T P^T contracts the 64 keys of a block in one product.  The
//    P^T operand of lane (query row, half h) holds that lane's 32
//    probabilities in accumulator order, byte p = key 32(p/16) + 8((p%16)/4)
//    + 4h + p%4; the V^T operand of lane (head-dim column, half h) holds the
//    same 32 keys of its column, gathered from the row-major V block by four
//    ds_read_b64_tr_b8 (within each 16-lane group, lane j receives byte j%8
//    of the 8-byte pieces addressed by lanes j/8 + 2t, t = 0..7).
//  * Probabilities are rounded to E4M3 (nearest even) as 2^3 p: the reference
//    is reset to the exact row maximum whenever a lane's scaled sum exceeds
//    2^8, so every scaled value stays <= 2^8 (finite), and values down to
//    2^-9 of the reference keep the format's full 3-bit mantissa (normal
//    range from 2^-6).
//  * O is normalised by the row sum of the unrounded probabilities (fp32,
//    also the lse's sum) and multiplied by the caller's V scale; lse removes
//    the 2^3.
//  * K and V rows are 128 bytes (d = 128): 16-byte chunk swizzles make both
//    the 16-byte K reads and the transposing V reads take the minimum
//    number of LDS cycles.
#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_fwd_common.h"
#include "fa_kernels.h"
#include "tile_class.h"

namespace {

typedef int fa_i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int fa_u32x8 __attribute__((ext_vector_type(8)));
typedef int fa_i32x2 __attribute__((ext_vector_type(2)));

// log2 of the factor the probabilities are scaled by before rounding to E4M3
#define FA8_SHIFT 3.0f
// operands of the matrix phase are read this many products ahead
#define FA8_OPND_AHEAD 2

// E4M3 x E4M3 product, fp32 accumulate.  Scale operands 0 select the
// instruction without block scales.
__device__ __forceinline__ fa_f32x16 mma8(fa_u32x8 a, fa_u32x8 b, fa_f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      __builtin_bit_cast(fa_i32x8, a), __builtin_bit_cast(fa_i32x8, b), c, 0, 0, 0, 0, 0, 0);
}

// 16-byte chunk swizzles of the 128-byte K and V rows (chunk position =
// chunk ^ swizzle of the row).  A 16-lane group of K reads takes one chunk of
// 16 consecutive rows; a 32-lane half of a transposing V read takes two
// chunks of rows {0..3, 8..11} + 16i (lane half 0) or {4..7, 12..15} + 16i.
// Both depend on row bits 0-3 only.
__device__ __forceinline__ int kswz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int vswz8(int r) { return (r & 3) + 4 * ((r >> 3) & 1); }

// Round the 32 scaled probabilities of a lane to E4M3 in operand order
// (byte p = pr[p / 16][p % 16]).
__device__ __forceinline__ fa_u32x8 pack_e4m3(const float (&pr)[2][16]) {
  fa_u32x8 w;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float* x = &pr[i / 4][4 * (i % 4)];
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], v, true);
    w[i] = (unsigned)v;
  }
  return w;
}

// Matrix phase of one wavefront: S^T = K Q^T over the current key block and
// O^T += V^T P^T over the previous one, as one software-pipelined sequence
// whose LDS operands are read FA8_OPND_AHEAD products ahead.  Product order:
// Q K by contraction slice s, then key group kb (sc[kb] starts from sc0);
// then P V by output block cb.  The K operand of (s, kb) is two 16-byte
// reads of row 32kb + l32 (chunks 4s + 2half and 4s + 2half + 1); the V^T
// operand of cb four transposing reads at rows 16i + (lane pattern), i =
// 0..3.
template <int D>
__device__ __forceinline__ void matrix_phase8(fa_f32x16 (&acc)[D / 32], fa_f32x16 (&sc)[2],
                                              const fa_f32x16& sc0, const fa_u32x8& pf,
                                              const fa_u32x8 (&qf)[D / 64],
                                              const FA_AS3 unsigned char* kcur,
                                              const FA_AS3 unsigned char* vcur,
                                              const unsigned (&kread)[D / 64][2],
                                              const unsigned (&vread)[D / 32]) {
  constexpr int NCB = D / 32, NS = D / 64, ROWB = D;
  constexpr int NQK = 2 * NS;
  constexpr int NOPS = NQK + NCB;
  constexpr int R = FA8_OPND_AHEAD;
  constexpr int NSLOT = R + 1;
  fa_u32x8 opnd[NSLOT];
  sc[0] = sc0;
  sc[1] = sc0;
#pragma unroll
  for (int i = 0; i < NOPS + R; ++i) {
    if (i >= R) {  // product i - R
      const int j = i - R;
      if (j < NQK) {
        const int s = j / 2, kb = j % 2;
        sc[kb] = mma8(opnd[j % NSLOT], qf[s], sc[kb]);
      } else {
        const int cb = j - NQK;
        acc[cb] = mma8(opnd[j % NSLOT], pf, acc[cb]);
      }
    }
    if (i < NOPS) {  // operand of product i
      if (i < NQK) {
        const int s = i / 2, kb = i % 2;
        const FA_AS3 unsigned char* kp = kcur + kb * 32 * ROWB;
        const fa_u32x4 lo = *(const FA_AS3 fa_u32x4*)(kp + kread[s][0]);
        const fa_u32x4 hi = *(const FA_AS3 fa_u32x4*)(kp + kread[s][1]);
        opnd[i % NSLOT] = fa_u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      } else {
        const int cb = i - NQK;
        const FA_AS3 unsigned char* vp = vcur + vread[cb];
        fa_u32x8 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const fa_i32x2 t =
              __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_AS3 fa_i32x2*)(vp + 16 * r * ROWB));
          o[2 * r] = (unsigned)t.x;
          o[2 * r + 1] = (unsigned)t.y;
        }
        opnd[i % NSLOT] = o;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O = v_scale O^T / l, lse = (m - 3 + log2 l) ln 2 (l: row sum of the
// unrounded scaled probabilities).
template <int D, int OUT_DT>
__device__ __forceinline__ void store_output8(const FaFwdParams& p, const fa_f32x16 (&acc)[D / 32],
                                              float m_ref, float l_tot, int bh, int qi, int half) {
  const int N = p.N;
  const float inv = l_tot > 0.f ? p.v_scale / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_ref - FA8_SHIFT + __log2f(l_tot)) * FA_LN2 : FA_NEG_INF;
  if (qi >= N) return;
  const size_t row = (size_t)bh * N + qi;
  unsigned char* Orow = (unsigned char*)p.o + row * D * (OUT_DT == 0 ? 4 : 2);
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = cb * 32 + 8 * g + 4 * half;
      const float o0 = acc[cb][4 * g] * inv, o1 = acc[cb][4 * g + 1] * inv;
      const float o2 = acc[cb][4 * g + 2] * inv, o3 = acc[cb][4 * g + 3] * inv;
      if constexpr (OUT_DT == 0) {
        const fa_f32x4 val = {o0, o1, o2, o3};
        *(fa_f32x4*)(Orow + c * 4) = val;
      } else {
        *(fa_u32x2*)(Orow + c * 2) = pack4<OUT_DT>(o0, o1, o2, o3);
      }
    }
  if (half == 0) p.lse[row] = lse;
}

// Eight wavefronts, 32 query rows each, two per SIMD, half a key block apart
// (see fa_fwd16_kernel for the schedule and the ring discipline; here the
// rings have four slots, and K(kt+3) and V(kt+2) are loaded while block kt
// is computed).
template <int D, int OUT_DT>
__global__ void __launch_bounds__(FA_WAVES_16 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd8_kernel(FaFwdParams p) {
  constexpr int NW = FA_WAVES_16;
  constexpr int ROWS_WG = NW * FA_ROW_BLOCK;
  constexpr int BC = FA_KEYS_8;    // keys per block
  constexpr int NKB = BC / 32;     // 32-key groups per block
  constexpr int NCB = D / 32;      // 32-column output blocks
  constexpr int NS = D / 64;       // 64-deep slices of the QK^T contraction
  constexpr int ROWB = D;          // bytes of one K/V row
  constexpr int TILEB = BC * ROWB; // bytes of one K or V block
  constexpr int NL = NW / 2;       // wavefronts loading each matrix
  constexpr int LPW = TILEB / (NL * 1024);  // 1 KB loads per loading wave per block
  static_assert(D == 128 && NKB == 2, "128-byte rows and 64-key blocks below");
  static_assert(LPW * NL * 1024 == TILEB, "loads must cover the block");
  static_assert(NL * 1024 / ROWB % 16 == 0, "pieces must be a multiple of 16 rows apart");
  constexpr int NSL = 4;  // ring slots: blocks are prefetched three steps ahead
  static_assert(NW == 8, "schedule below: 2 x 4 wavefronts");
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILEB], ks1[TILEB], ks2[TILEB], ks3[TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[TILEB], vs1[TILEB], vs2[TILEB], vs3[TILEB];
  auto kbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? ks0 : b == 1 ? ks1 : b == 2 ? ks2 : ks3); };
  auto vbuf = [&](int b) { return (FA_AS3 unsigned char*)(b == 0 ? vs0 : b == 1 ? vs1 : b == 2 ? vs2 : vs3); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave < NW / 2;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int N = p.N;

  // Persistent: this workgroup's row tiles in the order of fa_persist_tile_of
  // (one workgroup per compute unit; under a causal mask or none, the tiles
  // an XCD runs together read one key/value head, and under a sliding window
  // of whole row tiles a team of workgroups reads one key/value block at a
  // time, so the XCD's L2 serves their common key and value blocks).
  int bh, q0;
  for (int tile_k = 0; persist_tile(p, tile_k, bh, q0, ROWS_WG); ++tile_k) {
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

    // Q fragment s holds q[qi][64s + 32half .. +31]; rows past N read row N-1
    // (no branch) and are never stored.
    fa_u32x8 qf[NS];
    {
      const unsigned char* qrow = Qh + (size_t)min(qi, N - 1) * ROWB;
  #pragma unroll
      for (int s = 0; s < NS; ++s) {
        const fa_u32x4 lo = *(const fa_u32x4*)(qrow + 64 * s + 32 * half);
        const fa_u32x4 hi = *(const fa_u32x4*)(qrow + 64 * s + 32 * half + 16);
        qf[s] = fa_u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    }

    // Global byte offset (within a block) of this lane's 16 bytes in a loading
    // wave's first one-kilobyte LDS piece (8 rows), swizzle applied; piece i
    // lies 4 KB (32 rows) further on both sides.
    unsigned koff, voff;
    {
      const int o = (wave % NL) * 1024 + 16 * lane;
      const int r = o / ROWB, pos = (o % ROWB) / 16;
      koff = r * ROWB + 16 * (pos ^ kswz8(r));
      voff = r * ROWB + 16 * (pos ^ vswz8(r));
    }
    // LDS read offsets.  K slice s, piece e: row l32, chunk 4s + 2half + e.
    // V^T for output block cb: lane 16g + a addresses row 8(a/8) + 4half +
    // (a/2)%4 (+16i for read i), columns 32cb + 16(g%2) + 8(a%2) .. +7.
    unsigned kread[NS][2], vread[NCB];
  #pragma unroll
    for (int s = 0; s < NS; ++s)
  #pragma unroll
      for (int e = 0; e < 2; ++e) kread[s][e] = l32 * ROWB + 16 * ((4 * s + 2 * half + e) ^ kswz8(l32));
    {
      const int g = lane >> 4, a = lane & 15;
      const int vr = 8 * (a >> 3) + 4 * half + ((a >> 1) & 3);
  #pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        vread[cb] = vr * ROWB + 16 * ((2 * cb + (g & 1)) ^ vswz8(vr)) + 8 * (a & 1);
    }

    // K or V block kt -> LDS slot (descriptor ends at key N: rows past it read
    // as zeros).
    auto issue = [&](const unsigned char* base, unsigned off, FA_AS3 unsigned char* dst, int kt) {
      const int k0 = kt * BC;
      const int nb = (min(N - k0, BC)) * ROWB;
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)k0 * ROWB), 0, nb, FA_BUF_WORD3);
  #pragma unroll
      for (int i = 0; i < LPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (FA_AS3 void*)(dst + (i * NL + wave % NL) * 1024), 16, (int)off, i * NL * 1024, 0, 0);
    };

    fa_f32x16 acc[NCB];  // O^T: acc[cb] holds columns 32cb.., row qi
  #pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    // reference m (base 2) and this lane's sum of the unrounded scaled
    // probabilities 2^(s c2 - m + 3)
    float m_ref = FA_NEG_INF, l_lane = 0.f;
    const float c2 = p.scale_log2;
    const float inv_c2 = 1.f / p.scale_log2;
    const int n_row_blocks = (N + FA_ROW_BLOCK - 1) / FA_ROW_BLOCK;
    const int n_key_blocks = (N + BC - 1) / BC;

    // Scores of the current block (matrix phase -> softmax phase) and its
    // rounded probabilities (softmax phase -> the next matrix phase).
    // sc[kb][r] is key k0 + 32kb + 8(r/4) + 4half + r%4 of row qi.  The score
    // accumulators start from -(m - 3) / c2 (0 while the row has seen no key),
    // so the matrix core delivers (s c2 - m + 3) / c2.
    fa_f32x16 sc[NKB];
    fa_u32x8 pf = fa_u32x8{0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    fa_f32x16 sc0;
  #pragma unroll
    for (int r = 0; r < 16; ++r) sc0[r] = 0.f;

    auto phase_mfma = [&](int ks, int vs) {
      matrix_phase8<D>(acc, sc, sc0, pf, qf, kbuf(ks), vbuf(vs), kread, vread);
    };
    // Softmax phase of block kt.  Fast path (fully visible block, row already
    // started): p = 2^t straight from the scores, accepted if the lane's sum
    // is at most 2^8 (so is each p).  Exact path: mask, row maximum, new
    // reference, rescale of O and the sum, probabilities again (each then at
    // most 2^3, their sum at most 2^8).
    auto phase_softmax = [&](int kt, int cls) {
      if (cls == FA_TILE_SKIP) {
        pf = fa_u32x8{0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        return;
      }
      float pr[NKB][16];
      float psum = 0.f;
      float ps4[4];  // four independent partial sums (short dependency chains)
      bool exact = cls == FA_TILE_PARTIAL || __ballot(m_ref == FA_NEG_INF);
      if (!exact) {
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            pr[kb][r] = exp2_hw(sc[kb][r] * c2);
            ps4[r & 3] = kb == 0 && r < 4 ? pr[kb][r] : ps4[r & 3] + pr[kb][r];
          }
        psum = (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
        exact = __ballot(!(psum <= 256.f));
      }
      if (exact) {
        if (cls == FA_TILE_PARTIAL) apply_mask<NKB>(sc, kt * BC, qi, half, N, p.mask_kind, p.window);
        // the accumulators hold (s c2 - base) / c2
        const float base = m_ref == FA_NEG_INF ? 0.f : m_ref - FA8_SHIFT;
        float mx = FA_NEG_INF;
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        mx = pair_max(mx) * c2;  // block maximum of s c2 - base (-inf: nothing visible)
        const float m_new = fmaxf(m_ref, mx == FA_NEG_INF ? FA_NEG_INF : base + mx);
        // O and the sum are rescaled only where the reference rises above a
        // finite one (a row that has seen no key holds zeros); the
        // wavefront skips the multiplies when no lane needs them
        const bool rise = m_new > m_ref && m_ref != FA_NEG_INF;
        if (__ballot(rise)) {
          const float alpha = rise ? exp2_hw(m_ref - m_new) : 1.f;
          l_lane *= alpha;
  #pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
  #pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        }
        m_ref = m_new;
        const float shift = m_ref == FA_NEG_INF ? 0.f : base - m_ref + FA8_SHIFT;
        psum = 0.f;
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            pr[kb][r] = exp2_hw(__builtin_fmaf(sc[kb][r], c2, shift));
            ps4[r & 3] = kb == 0 && r < 4 ? pr[kb][r] : ps4[r & 3] + pr[kb][r];
          }
        psum = (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
        const float mn = m_ref == FA_NEG_INF ? 0.f : -(m_ref - FA8_SHIFT) * inv_c2;
  #pragma unroll
        for (int r = 0; r < 16; ++r) sc0[r] = mn;
      }
      pf = pack_e4m3(pr);
      l_lane += psum;
    };

    // The leading wavefronts load both matrices, at the start of their matrix
    // phase: K(kt+3) into K(kt-1)'s slot and V(kt+2) into V(kt-2)'s, both
    // last read in step kt-1.  The trailing wavefronts load nothing.
    auto issue_step = [&](int kt, int s) {
      if (kt + NSL - 1 < kv_hi) issue(Kh, koff, kbuf((s + NSL - 1) % NSL), kt + NSL - 1);
      if (kt + NSL - 2 < kv_hi) issue(Vh, voff, vbuf((s + NSL - 2) % NSL), kt + NSL - 2);
    };
    // At the end of a leading wavefront's softmax phase K(kt+1) and V(kt) must
    // have landed (issued in step kt-2, before every later load); the loads of
    // steps kt-1 (K(kt+2), V(kt+1)) and kt (K(kt+3), V(kt+2)) may stay in
    // flight.
    auto wait_step = [&](int kt) {
      if (kt + 3 < kv_hi)
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(4 * LPW));
      else if (kt + 2 < kv_hi)
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(3 * LPW));
      else if (kt + 1 < kv_hi)
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(LPW));
      else
        __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(0));
    };
    auto step = [&](int kt, int s) {
      int cls_cur = FA_TILE_SKIP;
      if (kt < kv_hi) {
        cls_cur = fa_classify(qb0, qb1, kt * BC, BC, N, p.mask_kind, p.window);
        if (p.tiles && lane == 0 && qb0 < N)
          p.tiles[((size_t)bh * n_row_blocks + qb0 / FA_ROW_BLOCK) * n_key_blocks + kt] =
              (unsigned char)(cls_cur + 1);
      }
      if (lead) issue_step(kt, s);
      phase_mfma(s, (s + NSL - 1) % NSL);
      __builtin_amdgcn_s_waitcnt(FA_WAITCNT_LGKM0);
      barrier_nofence();
      phase_softmax(kt, cls_cur);
      if (lead) wait_step(kt);
      __builtin_amdgcn_s_waitcnt(FA_WAITCNT_LGKM0);
      barrier_nofence();
    };

    // Prologue: K and V of the first two blocks, and zeros in the V slot that
    // the first step's (probability 0) P V product reads.
    if (lead) {
      issue(Kh, koff, kbuf(0), kv_lo);
      if (kv_lo + 1 < kv_hi) issue(Kh, koff, kbuf(1), kv_lo + 1);
      if (kv_lo + 2 < kv_hi) issue(Kh, koff, kbuf(2), kv_lo + 2);
      issue(Vh, voff, vbuf(0), kv_lo);
      if (kv_lo + 1 < kv_hi) issue(Vh, voff, vbuf(1), kv_lo + 1);
    }
    static_assert(TILEB % (NW * 64 * 16) == 0, "zero fill must cover the slot");
  #pragma unroll
    for (int i = 0; i < TILEB / (NW * 64 * 16); ++i)
      *(FA_AS3 fa_u32x4*)(vbuf(NSL - 1) + (i * NW * 64 + tid) * 16) = fa_u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!lead) barrier_nofence();
    for (int kt = kv_lo;;) {
      step(kt, 0);
      if (++kt > kv_hi) break;
      step(kt, 1);
      if (++kt > kv_hi) break;
      step(kt, 2);
      if (++kt > kv_hi) break;
      step(kt, 3);
      if (++kt > kv_hi) break;
    }
    if (lead) barrier_nofence();
    store_output8<D, OUT_DT>(p, acc, m_ref, pair_sum(l_lane), bh, qi, half);
    // every wavefront is done with the slots before the next tile refills them
    __syncthreads();
  }
}

// One wavefront, one E4M3 product (lane-order operands of 32 bytes in,
// lane-order accumulator out), or one transposing byte read of a 512-byte
// LDS block whose lane l addresses byte 8l (8 bytes per lane out, as floats).
template <int WHICH>
__global__ void __launch_bounds__(64) fa_probe8_kernel(const void* a, const void* b, float* d) {
  const int l = threadIdx.x;
  if constexpr (WHICH == 0) {
    fa_f32x16 c;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = 0.f;
    c = mma8(((const fa_u32x8*)a)[l], ((const fa_u32x8*)b)[l], c);
#pragma unroll
    for (int r = 0; r < 16; ++r) d[l * 16 + r] = c[r];
  } else {
    __shared__ __attribute__((aligned(16))) unsigned char blk[512];
    ((FA_AS3 fa_u32x2*)blk)[l] = ((const fa_u32x2*)a)[l];
    __syncthreads();
    const fa_i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_AS3 fa_i32x2*)(blk + 8 * l));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      d[l * 8 + i] = (float)((((unsigned)(i < 4 ? t.x : t.y)) >> (8 * (i & 3))) & 255u);
  }
}

template <int D, int OUT_DT>
hipError_t launch8(const FaFwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n_groups * p.wg_per_group));
  hipLaunchKernelGGL((fa_fwd8_kernel<D, OUT_DT>), grid, dim3(FA_WAVES_16 * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t fa_launch_fwd8(int out_dtype, int d, const FaFwdParams& p, hipStream_t stream) {
  (void)d;  // 128 only (checked by the caller)
  switch (out_dtype) {
    case 0: return launch8<128, 0>(p, stream);
    case 1: return launch8<128, 1>(p, stream);
    default: return launch8<128, 2>(p, stream);
  }
}

hipError_t fa_launch_probe8(int which, const void* a, const void* b, float* d,
                            hipStream_t stream) {
  if (which == 0)
    hipLaunchKernelGGL(fa_probe8_kernel<0>, dim3(1), dim3(64), 0, stream, a, b, d);
  else
    hipLaunchKernelGGL(fa_probe8_kernel<1>, dim3(1), dim3(64), 0, stream, a, b, d);
  return hipGetLastError();
}
