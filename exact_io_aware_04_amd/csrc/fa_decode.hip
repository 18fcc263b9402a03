// Decoding against a key/value cache on gfx950 (MI355X, CDNA4): Nq queries
// per head at the last Nq positions of a cache of Nk keys (query i at
// position Nk - Nq + i), the same attention as the forward pass at those
// positions, with H / H_kv query heads per key/value head.
//
// Few queries meet many keys, so the work is reading K and V once from HBM:
// the key range is split into chunks ("split-KV"), each chunk's partial
// result (o normalised over the chunk, and its lse) goes to a workspace, and
// a second kernel merges the chunks with lse = ln sum_c exp(lse_c),
// o = sum_c exp(lse_c - lse) o_c -- the online-softmax rescale of
// "FlashAttention (NL)", section "Online berekening van Softmax", applied to
// whole chunks.  KV-cache streaming for generation is the workload of the
// specialised engines in section "Gespecialiseerde oplossingen".
//
// gfx950 mapping: one wavefront per (batch, key/value head, chunk); four
// independent wavefronts per workgroup, each with its own LDS (no workgroup
// barrier).  Its 32 lanes of rows are the g = H / H_kv query heads x Nq
// queries that read this key/value head (g Nq <= 32: one 32 x 32 matrix-core
// tile), so every K/V byte is read once per key/value head.  The cache
// streams in 32-key K and V blocks HBM -> LDS (buffer_load_dwordx4 with the
// LDS destination) through rings of three slots per wave, two blocks ahead,
// and is consumed as in the forward kernel: S^T = K Q^T from 16-byte K row
// reads, O^T += V^T P^T with V^T from transposing reads, row statistics
// in-lane plus one lane-half exchange.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_device.h"
#include "fa_kernels.h"
#include "tile_class.h"

namespace {

constexpr int DK = FA_DECODE_KEYS;   // keys per block
constexpr int DW = FA_DECODE_WAVES;  // wavefronts (work items) per workgroup
constexpr float LN2 = 0.69314718055994530942f;

// Descriptor of 32-key block kt of a [Nk][D] matrix: rows past Nk read as
// zeros; a block at or past `kend` (the chunk's end) has size 0, so loads
// of it read nothing and return zeros.  (The size and the block's row offset
// are wave-uniform; readfirstlane states that, so the descriptor stays in
// scalar registers.)
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const unsigned char* base, int kt,
                                                             int kend, int Nk) {
  constexpr int ROWB = 2 * D;
  const int k0 = kt * DK;
  const bool in = kt < kend && k0 < Nk;
  const int nb = __builtin_amdgcn_readfirstlane(in ? min(Nk - k0, DK) * ROWB : 0);
  const int r0 = __builtin_amdgcn_readfirstlane(in ? k0 : 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)r0 * ROWB), 0, nb, FA_BUF_WORD3);
}

// K or V block kt -> LDS (K or V swizzle); the wave loads it alone, one
// kilobyte (1024 / (2D) rows) per instruction
template <int D, bool IS_K>
__device__ __forceinline__ void load_block(const unsigned char* base, int kt, int kend, int Nk,
                                           FA_AS3 unsigned char* dst, int lane) {
  constexpr int ROWB = 2 * D, TILEB = DK * ROWB, RPP = 1024 / ROWB, CPR = ROWB / 16;
  const __amdgpu_buffer_rsrc_t rsrc = block_rsrc<D>(base, kt, kend, Nk);
#pragma unroll
  for (int i = 0; i < TILEB / 1024; ++i) {
    const int r = i * RPP + lane / CPR, pos = lane % CPR;
    const int sw = IS_K ? kswz<D>(r) : vswz<D>(r);
    const int off = r * ROWB + 16 * (pos ^ sw);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_AS3 void*)(dst + i * 1024), 16, off, 0, 0, 0);
  }
}

template <int DT>
__device__ __forceinline__ float rounded(float x) {
  if constexpr (DT == 2)
    return (float)(__bf16)x;
  else
    return (float)(_Float16)x;
}

template <int DT, int D>
__global__ void __launch_bounds__(DW * 64) fa_decode_split_kernel(FaDecodeParams p) {
  constexpr int NCB = D / 32, NQF = D / 16, ROWB = 2 * D, TILEB = DK * ROWB;
  constexpr int LPB = TILEB / 1024;  // loads per block and matrix
  // rings of three K and three V blocks per wave, one object per slot so
  // that the compiler can tell the slot being read from the ones being filled
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[DW][TILEB], ks1[DW][TILEB],
      ks2[DW][TILEB], vs0[DW][TILEB], vs1[DW][TILEB], vs2[DW][TILEB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wi = blockIdx.x * DW + wave;
  if (wi >= p.n_items) return;  // whole wavefront; this kernel has no workgroup barrier
  const int c = wi % p.n_chunks, bhk = wi / p.n_chunks;
  const int b = bhk / p.H_kv, hk = bhk % p.H_kv;
  const int Nq = p.Nq, Nk = p.Nk;
  // this lane's row: query head hk*g + hh, query qi at position Nk - Nq + qi
  const bool row_ok = l32 < p.group * Nq;
  const int hh = row_ok ? l32 / Nq : 0, qi = row_ok ? l32 % Nq : 0;
  const size_t qrow = ((size_t)b * p.H + hk * p.group + hh) * Nq + qi;
  const int pos = Nk - Nq + qi;

  fa_u32x4 qf[NQF];
  {
    const unsigned char* src = (const unsigned char*)p.q + qrow * ROWB;
#pragma unroll
    for (int s = 0; s < NQF; ++s) qf[s] = *(const fa_u32x4*)(src + s * 32 + half * 16);
  }
  const int blo = p.kb_lo + c * p.chunk_blocks;
  const int bhi = min(blo + p.chunk_blocks, p.kb_lo + p.n_blocks);
  const size_t kv = (size_t)bhk * Nk * ROWB;
  const unsigned char* Kh = (const unsigned char*)p.k + kv;
  const unsigned char* Vh = (const unsigned char*)p.v + kv;
  FA_AS3 unsigned char* const kb0 = (FA_AS3 unsigned char*)&ks0[wave][0];
  FA_AS3 unsigned char* const kb1 = (FA_AS3 unsigned char*)&ks1[wave][0];
  FA_AS3 unsigned char* const kb2 = (FA_AS3 unsigned char*)&ks2[wave][0];
  FA_AS3 unsigned char* const vb0 = (FA_AS3 unsigned char*)&vs0[wave][0];
  FA_AS3 unsigned char* const vb1 = (FA_AS3 unsigned char*)&vs1[wave][0];
  FA_AS3 unsigned char* const vb2 = (FA_AS3 unsigned char*)&vs2[wave][0];
  auto kbuf = [&](int sl) { return sl == 0 ? kb0 : sl == 1 ? kb1 : kb2; };
  auto vbuf = [&](int sl) { return sl == 0 ? vb0 : sl == 1 ? vb1 : vb2; };

  unsigned kread[NQF], vread[NCB];
#pragma unroll
  for (int s = 0; s < NQF; ++s) kread[s] = l32 * ROWB + 16 * ((2 * s + half) ^ kswz<D>(l32));
  {
    const int g = lane >> 4, t = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      vread[cb] = (4 * half + t) * ROWB + 64 * (cb ^ (D >= 128 ? t : (t >> 1))) + 32 * (g & 1) + 8 * q;
  }

  fa_f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float m = FA_NEG_INF, l_lane = 0.f, lq_lane = 0.f;  // base-2 reference, unrounded / rounded sums
  const float c2 = p.scale_log2;

  // Block kt in slot sl.  At the top the wave issues K(kt+2) and V(kt+2) into
  // the slots of block kt-1, read in the previous step; past the chunk's end
  // these read nothing.  Every step issues the same loads, so one wait
  // serves all: block kt, issued before block kt+1 and this step's loads,
  // has landed once at most 4 x LPB loads are outstanding (loads complete in
  // issue order).
  auto step = [&](int kt, int sl) {
    const int nx = (sl + 2) % 3;
    load_block<D, true>(Kh, kt + 2, bhi, Nk, kbuf(nx), lane);
    load_block<D, false>(Vh, kt + 2, bhi, Nk, vbuf(nx), lane);
    __builtin_amdgcn_s_waitcnt(FA_WAITCNT_VM_LGKM0(4 * LPB));
    const int cls = fa_classify(Nk - Nq, Nk, kt * DK, DK, Nk, p.mask_kind, p.window);
    if (cls == FA_TILE_SKIP) return;
    const FA_AS3 unsigned char* kc = kbuf(sl);
    const FA_AS3 unsigned char* vc = vbuf(sl);
    // S^T = K Q^T: s[r] is key kt*32 + 8(r/4) + 4half + r%4 of this lane's row
    fa_f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < NQF; ++s)
      sc = mma16<DT>(*(const FA_AS3 fa_u32x4*)(kc + kread[s]), qf[s], sc);
    float t[16];
    float mx = FA_NEG_INF;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kt * DK + 8 * (r >> 2) + 4 * half + (r & 3);
      bool vis = true;
      if (cls == FA_TILE_PARTIAL)
        vis = j < Nk && (p.mask_kind == FA_MASKK_NONE ||
                         (j <= pos && (p.mask_kind == FA_MASKK_CAUSAL || j > pos - p.window)));
      t[r] = vis ? sc[r] * c2 : FA_NEG_INF;
      mx = fmaxf(mx, t[r]);
    }
    mx = pair_max(mx);
    // online softmax, base 2: the reference moves only when the block's
    // maximum exceeds it by more than 8 (probabilities stay below 2^8)
    if (__ballot(mx > m + 8.f)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new > m ? (m == FA_NEG_INF ? 0.f : exp2_hw(m - m_new)) : 1.f;
      m = m_new;
      l_lane *= alpha;
      lq_lane *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
    }
    const float m_use = m == FA_NEG_INF ? 0.f : m;
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = exp2_hw(t[r] - m_use);
      l_lane += pr[r];
      lq_lane += rounded<DT>(pr[r]);  // the weights the matrix core multiplies V with
    }
    fa_u32x4 pf[2];
    pf[0] = pack8<DT>(&pr[0]);
    pf[1] = pack8<DT>(&pr[8]);
    // O^T += V^T P^T
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const FA_AS3 unsigned char* vp = vc + 16 * tt * ROWB + vread[cb];
        const fa_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)vp);
        const fa_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_AS3 fa_i16x4*)(vp + 8 * ROWB));
        const fa_u32x2 l2 = __builtin_bit_cast(fa_u32x2, lo), h2 = __builtin_bit_cast(fa_u32x2, hi);
        acc[cb] = mma16<DT>(fa_u32x4{l2.x, l2.y, h2.x, h2.y}, pf[tt], acc[cb]);
      }
  };

  if (blo < bhi) {
    load_block<D, true>(Kh, blo, bhi, Nk, kb0, lane);
    load_block<D, false>(Vh, blo, bhi, Nk, vb0, lane);
    load_block<D, true>(Kh, blo + 1, bhi, Nk, kb1, lane);
    load_block<D, false>(Vh, blo + 1, bhi, Nk, vb1, lane);
    for (int kt = blo;;) {
      step(kt, 0);
      if (++kt >= bhi) break;
      step(kt, 1);
      if (++kt >= bhi) break;
      step(kt, 2);
      if (++kt >= bhi) break;
    }
  }
  // chunk partial: o normalised by the rounded weights' sum, lse by the
  // unrounded one (as in the forward kernel); no visible key: o = 0, -inf
  const float l_tot = pair_sum(l_lane), lq_tot = pair_sum(lq_lane);
  if (!row_ok) return;
  const float inv = lq_tot > 0.f ? 1.f / lq_tot : 0.f;
  const size_t prow = (size_t)c * p.rows + qrow;
  float* wo = p.ws + prow * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const fa_f32x4 val = {acc[cb][4 * g] * inv, acc[cb][4 * g + 1] * inv,
                            acc[cb][4 * g + 2] * inv, acc[cb][4 * g + 3] * inv};
      *(fa_f32x4*)(wo + cb * 32 + 8 * g + 4 * half) = val;
    }
  if (half == 0)
    p.ws[(size_t)p.n_chunks * p.rows * D + prow] =
        l_tot > 0.f ? (m + __log2f(l_tot)) * LN2 : FA_NEG_INF;
}

// Merge of the chunks: one wavefront per row (batch, head, query).  The
// lanes first split the chunks (maximum and sum of exp(lse_c - max)), then
// the columns (D / 64 each), summing the chunks' partial rows with weight
// exp(lse_c - lse).
template <int DT, int D>
__global__ void __launch_bounds__(256) fa_decode_merge_kernel(FaDecodeParams p) {
  constexpr int CPL = D / 64;  // columns per lane
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.rows) return;  // whole wavefront; no barrier in this kernel
  const float* wl = p.ws + (size_t)p.n_chunks * p.rows * D;
  float m = FA_NEG_INF;
  for (int c = lane; c < p.n_chunks; c += 64) m = fmaxf(m, wl[(size_t)c * p.rows + row]);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  float sum = 0.f;
  if (m != FA_NEG_INF)
    for (int c = lane; c < p.n_chunks; c += 64) sum += __expf(wl[(size_t)c * p.rows + row] - m);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) sum += __shfl_xor(sum, s);
  float o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) o[j] = 0.f;
  if (m != FA_NEG_INF) {
    const float inv = 1.f / sum;
#pragma unroll 4
    for (int c = 0; c < p.n_chunks; ++c) {
      const float w = __expf(wl[(size_t)c * p.rows + row] - m) * inv;
      const float* x = p.ws + ((size_t)c * p.rows + row) * D + lane * CPL;
#pragma unroll
      for (int j = 0; j < CPL; ++j) o[j] += w * x[j];
    }
  }
  unsigned char* dst = (unsigned char*)p.o + ((size_t)row * D + lane * CPL) * 2;
  if constexpr (CPL == 2) {
    *(unsigned*)dst = __builtin_bit_cast(unsigned, pack4<DT>(o[0], o[1], 0.f, 0.f).x);
  } else {
    const fa_u32x2 h = pack4<DT>(o[0], 0.f, 0.f, 0.f);
    *(unsigned short*)dst = (unsigned short)(h.x & 0xffffu);
  }
  if (lane == 0) p.lse[row] = m == FA_NEG_INF ? FA_NEG_INF : m + __logf(sum);
}

template <int DT, int D>
hipError_t launch_decode(const FaDecodeParams& p, hipStream_t stream) {
  const unsigned g1 = (unsigned)((p.n_items + DW - 1) / DW);
  hipLaunchKernelGGL((fa_decode_split_kernel<DT, D>), dim3(g1), dim3(DW * 64), 0, stream, p);
  const unsigned g2 = (unsigned)((p.rows + 3) / 4);
  hipLaunchKernelGGL((fa_decode_merge_kernel<DT, D>), dim3(g2), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Chunk partials of fa_decode_noalloc: a file-scope device array instead of a
// caller's workspace, for callers that cannot allocate.  Every GPU holds its
// own copy at its own address; host code reaches it only through the address
// hipGetSymbolAddress gives with that GPU current (the array's name is a
// host-side stand-in, not a device address).  Calls that overlap on one GPU
// share it and race.
static __device__ __align__(256) float scratch[FA_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // per device; nullptr until looked up
}  // namespace

hipError_t fa_decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t fa_launch_decode(int in_dtype, int d, const FaDecodeParams& p, hipStream_t stream) {
  if (in_dtype == 1) return d == 64 ? launch_decode<1, 64>(p, stream) : launch_decode<1, 128>(p, stream);
  return d == 64 ? launch_decode<2, 64>(p, stream) : launch_decode<2, 128>(p, stream);
}
