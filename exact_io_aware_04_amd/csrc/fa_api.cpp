// Host side of the C ABI declared in include/fa.h: argument checks (pure
// host code, no HIP call before they pass), device check, grid order and
// dispatch to the gfx950 kernels, error reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/fa.h"
#include "../../include/fa_diag.h"
#include "fa_kernels.h"
#include "tile_class.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return FA_OK;
}

size_t elem_bytes(int dtype) {
  return dtype == FA_DTYPE_F32 ? 4 : dtype == FA_DTYPE_E4M3 ? 1 : 2;
}

bool valid_dtype(int t) {
  return t == FA_DTYPE_F32 || t == FA_DTYPE_F16 || t == FA_DTYPE_BF16;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int keys_per_block(int in_dtype, int d) { return fa_keys_per_block(in_dtype, d); }

// Everything that can be decided without the device.
int check_args(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int mask_kind,
               int window, int in_dtype, int out_dtype) {
  if (!q || !k || !v || !o || !lse)
    return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || H < 1 || N < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H and N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "H_kv must divide H = %d (got %d)", H, H_kv);
  if (N >= (1 << 30)) return fail(FA_ERR_INVALID_ARG, "N must be < 2^30 (got %d)", N);
  const bool e4m3 = in_dtype == FA_DTYPE_E4M3;
  if (!valid_dtype(in_dtype) && !e4m3)
    return fail(FA_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (!valid_dtype(out_dtype)) return fail(FA_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  if (!e4m3 && out_dtype != in_dtype && out_dtype != FA_DTYPE_F32)
    return fail(FA_ERR_INVALID_ARG, "out_dtype must equal in_dtype or be F32");
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL && mask_kind != FA_MASK_SLIDING)
    return fail(FA_ERR_INVALID_ARG, "unknown mask_kind %d", mask_kind);
  if (mask_kind == FA_MASK_SLIDING && window < 1)
    return fail(FA_ERR_INVALID_ARG, "sliding window must be >= 1 (got %d)", window);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  const long double total = (long double)B * H * N * d;
  if (total >= 4.611686018427387904e18L)  // 2^62
    return fail(FA_ERR_INVALID_ARG, "B*H*N*d too large");
  const long long bh = (long long)B * H;
  const int rows_wg = fa_rows_per_wg(in_dtype, d);
  const long long tiles = bh * ((N + rows_wg - 1) / rows_wg);
  if (tiles > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "too many row tiles for one grid");
  if (!fa_head_dim_built(in_dtype, d))
    return fail(FA_ERR_UNSUPPORTED, e4m3 ? "E4M3 head dim %d not built (128)"
                                         : "head dim %d not built (64, 128; 256 for f16/bf16)", d);
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u;
  if (mis) return fail(FA_ERR_INVALID_ARG, "q, k, v, o must be 16-byte aligned");
  if (((uintptr_t)lse & 3u) != 0) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t nq = (size_t)bh * N * d * elem_bytes(in_dtype);
  const size_t nkv = (size_t)B * H_kv * N * d * elem_bytes(in_dtype);
  const size_t nout = (size_t)bh * N * d * elem_bytes(out_dtype);
  const size_t nlse = (size_t)bh * N * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t nins[3] = {nq, nkv, nkv};
  for (int t = 0; t < 3; ++t) {
    if (overlaps(o, nout, ins[t], nins[t])) return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
    if (overlaps(lse, nlse, ins[t], nins[t])) return fail(FA_ERR_INVALID_ARG, "lse overlaps an input");
  }
  if (overlaps(o, nout, lse, nlse)) return fail(FA_ERR_INVALID_ARG, "o overlaps lse");
  return FA_OK;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];  // compute units per device (0: not yet read)

// compute units of the current device (check_device has run)
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int n = g_cus[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(FA_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_NO_DEVICE, "device index %d", dev);
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(FA_ERR_NO_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  if (state != 1) return fail(FA_ERR_NO_DEVICE, "device %d is not gfx950", dev);
  return FA_OK;
}

int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
            int H, int H_kv, int N, int d, float scale, float v_scale, int mask_kind,
            int window, int in_dtype, int out_dtype, unsigned char* tiles, void* stream) {
  int st = check_args(q, k, v, o, lse, B, H, H_kv, N, d, scale, mask_kind, window,
                      in_dtype, out_dtype);
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  FaFwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.tiles = tiles;
  p.BH = B * H;
  p.kv_group = H / H_kv;
  p.N = N;
  p.mask_kind = mask_kind;
  // a window of N or more keys is the causal mask; clamping keeps every
  // index computation of the kernels far from int overflow
  p.window = mask_kind == FA_MASK_SLIDING ? (window < N ? window : N) : 0;
  // The kernel needs scale_log2 > 0 (masked scores are -inf and must map to
  // probability 0).  scale = 0 becomes the smallest normal float: every
  // exponent s*scale_log2 is then below 2^-100 in magnitude, so each weight
  // is 1 to fp32 precision -- the uniform weights scale = 0 defines.
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  if (!(p.scale_log2 >= FLT_MIN)) p.scale_log2 = FLT_MIN;
  p.v_scale = v_scale;
  p.n_row_tiles = (N + fa_rows_per_wg(in_dtype, d) - 1) / fa_rows_per_wg(in_dtype, d);
  fa_fwd_plan(p, mask_kind, device_cus(), fa_rows_per_wg(in_dtype, d));
  hipError_t e = in_dtype == FA_DTYPE_E4M3
                     ? fa_launch_fwd8(out_dtype, d, p, (hipStream_t)stream)
                     : fa_launch_fwd(in_dtype, out_dtype, d, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int check_bwd_args(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   float* delta, int B, int H, int H_kv, int N, int d, float scale,
                   int mask_kind, int window, int dtype) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta)
    return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || H < 1 || N < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H and N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "H_kv must divide H = %d (got %d)", H, H_kv);
  if (N >= (1 << 30)) return fail(FA_ERR_INVALID_ARG, "N must be < 2^30 (got %d)", N);
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL && mask_kind != FA_MASK_SLIDING)
    return fail(FA_ERR_INVALID_ARG, "unknown mask_kind %d", mask_kind);
  if (mask_kind == FA_MASK_SLIDING && window < 1)
    return fail(FA_ERR_INVALID_ARG, "sliding window must be >= 1 (got %d)", window);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  const long double total = (long double)B * H * N * d;
  if (total >= 4.611686018427387904e18L)  // 2^62
    return fail(FA_ERR_INVALID_ARG, "B*H*N*d too large");
  const long long bh = (long long)B * H;
  if (bh * ((N + FA_BWD_WAVES * 32 - 1) / (FA_BWD_WAVES * 32)) > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARG, "too many tiles for one grid");
  if (dtype == FA_DTYPE_F32)
    return fail(FA_ERR_UNSUPPORTED, "the backward pass is built for f16/bf16 inputs");
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "backward head dim %d not built (64, 128)", d);
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o |
                         (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u;
  if (mis) return fail(FA_ERR_INVALID_ARG, "q, k, v, o, dout, dq, dk, dv must be 16-byte aligned");
  if ((((uintptr_t)lse | (uintptr_t)delta) & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "lse and delta must be 4-byte aligned");
  const size_t nm = (size_t)bh * N * d * elem_bytes(dtype);
  const size_t nkv = (size_t)B * H_kv * N * d * elem_bytes(dtype);
  const size_t nr = (size_t)bh * N * sizeof(float);
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t nins[6] = {nm, nkv, nkv, nm, nm, nr};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t nouts[4] = {nm, nkv, nkv, nr};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], nouts[a], ins[b], nins[b]))
        return fail(FA_ERR_INVALID_ARG, "an output of the backward pass overlaps an input");
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], nouts[a], outs[b], nouts[b]))
        return fail(FA_ERR_INVALID_ARG, "outputs of the backward pass overlap");
  }
  return FA_OK;
}

// Split of the cache for fa_decode: the 32-key blocks from the first one any
// query sees to the end, in n_chunks chunks of chunk_blocks blocks, about
// 2048 work items (wavefronts) in all and at most 256 chunks.
struct DecodePlan {
  int kb_lo, n_blocks, chunk_blocks, n_chunks;
};
DecodePlan decode_plan(int B, int H_kv, int Nq, int Nk, int mask_kind, int window) {
  DecodePlan pl;
  const int lo_key = mask_kind == FA_MASK_SLIDING ? std::max(0, Nk - Nq - window + 1) : 0;
  pl.kb_lo = lo_key / FA_DECODE_KEYS;
  pl.n_blocks = (Nk + FA_DECODE_KEYS - 1) / FA_DECODE_KEYS - pl.kb_lo;
  const long long pairs = (long long)B * H_kv;
  const long long want =
      std::max(1LL, std::min({(long long)pl.n_blocks, (2048 + pairs - 1) / pairs, 256LL}));
  pl.chunk_blocks = (int)((pl.n_blocks + want - 1) / want);
  pl.n_chunks = (pl.n_blocks + pl.chunk_blocks - 1) / pl.chunk_blocks;
  return pl;
}

// Most chunks any mask can give for these sizes.  decode_plan's chunk count
// is ceil(n / ceil(n / want)) <= want = min(n, cap) for n blocks, and a mask
// only removes blocks, so min(unmasked blocks, cap) bounds every mask and
// window (the count itself is not monotone in n: 33 blocks with cap 32 give
// 17 chunks, 32 blocks give 32).
int decode_max_chunks(int B, int H_kv, int Nk) {
  const long long n = (Nk + FA_DECODE_KEYS - 1) / FA_DECODE_KEYS;
  const long long pairs = (long long)B * H_kv;
  return (int)std::max(1LL, std::min({n, (2048 + pairs - 1) / pairs, 256LL}));
}

long long decode_ws_bytes(int B, int H, int Nq, int d, int n_chunks) {
  return (long long)n_chunks * B * H * Nq * (d + 1) * (long long)sizeof(float);
}

int check_decode_args(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int H_kv, int Nq, int Nk, int d, float scale, int mask_kind,
                      int window, int dtype) {
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H, Nq and Nk must be >= 1");
  if (Nq > Nk) return fail(FA_ERR_INVALID_ARG, "Nq (%d) must not exceed Nk (%d)", Nq, Nk);
  if (Nk >= (1 << 30)) return fail(FA_ERR_INVALID_ARG, "Nk must be < 2^30");
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "H_kv must divide H = %d (got %d)", H, H_kv);
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL && mask_kind != FA_MASK_SLIDING)
    return fail(FA_ERR_INVALID_ARG, "unknown mask_kind %d", mask_kind);
  if (mask_kind == FA_MASK_SLIDING && window < 1)
    return fail(FA_ERR_INVALID_ARG, "sliding window must be >= 1 (got %d)", window);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  const long double big = (long double)B * H_kv * Nk * d + (long double)B * H * Nq * d;
  if (big >= 4.611686018427387904e18L) return fail(FA_ERR_INVALID_ARG, "sizes too large");
  if (dtype == FA_DTYPE_F32) return fail(FA_ERR_UNSUPPORTED, "decoding is built for f16/bf16");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "decode head dim %d not built (64, 128)", d);
  if ((H / H_kv) * Nq > 32)
    return fail(FA_ERR_UNSUPPORTED, "(H / H_kv) * Nq = %d rows per key/value head exceeds 32",
                (H / H_kv) * Nq);
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o must be 16-byte aligned");
  if (((uintptr_t)lse & 3u) != 0) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t nq = (size_t)B * H * Nq * d * elem_bytes(dtype);
  const size_t nkv = (size_t)B * H_kv * Nk * d * elem_bytes(dtype);
  const size_t nl = (size_t)B * H * Nq * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t nins[3] = {nq, nkv, nkv};
  for (int t = 0; t < 3; ++t) {
    if (overlaps(o, nq, ins[t], nins[t])) return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
    if (overlaps(lse, nl, ins[t], nins[t])) return fail(FA_ERR_INVALID_ARG, "lse overlaps an input");
  }
  if (overlaps(o, nq, lse, nl)) return fail(FA_ERR_INVALID_ARG, "o overlaps lse");
  return FA_OK;
}

}  // namespace

extern "C" {

long long fa_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || Nq > Nk || H_kv < 1 || H_kv > H || H % H_kv != 0 ||
      d < 1 || Nk >= (1 << 30)) {
    fail(FA_ERR_INVALID_ARG, "invalid sizes");
    return -1;
  }
  ok();
  return decode_ws_bytes(B, H, Nq, d, decode_max_chunks(B, H_kv, Nk));
}

}  // extern "C"

namespace {

// fa_decode after its argument check: workspace check, device check, launch.
int run_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int H_kv, int Nq, int Nk, int d, float scale, int mask_kind, int window,
               int dtype, void* workspace, long long workspace_bytes, void* stream) {
  int st;
  const int win = mask_kind == FA_MASK_SLIDING ? (window < Nk ? window : Nk) : 0;
  const DecodePlan pl = decode_plan(B, H_kv, Nq, Nk, mask_kind, win);
  const long long need = decode_ws_bytes(B, H, Nq, d, pl.n_chunks);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "workspace of %lld bytes needed (got %lld)", need,
                workspace ? workspace_bytes : 0LL);
  if (((uintptr_t)workspace & 15u) != 0)
    return fail(FA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const size_t nq = (size_t)B * H * Nq * d * elem_bytes(dtype);
  const size_t nkv = (size_t)B * H_kv * Nk * d * elem_bytes(dtype);
  const size_t nl = (size_t)B * H * Nq * sizeof(float);
  const void* all[5] = {q, k, v, o, lse};
  const size_t nall[5] = {nq, nkv, nkv, nq, nl};
  for (int t = 0; t < 5; ++t)
    if (overlaps(workspace, (size_t)need, all[t], nall[t]))
      return fail(FA_ERR_INVALID_ARG, "workspace overlaps an argument");
  if ((long long)B * H_kv * pl.n_chunks > 0x7fffffffLL ||
      (long long)B * H * Nq / 4 + 1 > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARG, "too many work items for one grid");
  st = check_device();
  if (st != FA_OK) return st;
  FaDecodeParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.ws = (float*)workspace;
  p.H = H;
  p.H_kv = H_kv;
  p.group = H / H_kv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.mask_kind = mask_kind;
  p.window = win;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  if (!(p.scale_log2 >= FLT_MIN)) p.scale_log2 = FLT_MIN;
  p.kb_lo = pl.kb_lo;
  p.n_blocks = pl.n_blocks;
  p.chunk_blocks = pl.chunk_blocks;
  p.n_chunks = pl.n_chunks;
  p.n_items = B * H_kv * pl.n_chunks;
  p.rows = (long long)B * H * Nq;
  hipError_t e = fa_launch_decode(dtype, d, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int H_kv, int Nq, int Nk, int d, float scale, int mask_kind, int window, int dtype,
              void* workspace, long long workspace_bytes, void* stream) {
  const int st = check_decode_args(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind,
                                   window, dtype);
  if (st != FA_OK) return st;
  return run_decode(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind, window, dtype,
                    workspace, workspace_bytes, stream);
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int H_kv, int Nq, int Nk, int d, float scale, int mask_kind,
                      int window, int dtype, void* stream) {
  int st = check_decode_args(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind, window,
                             dtype);
  if (st != FA_OK) return st;
  const int win = mask_kind == FA_MASK_SLIDING ? (window < Nk ? window : Nk) : 0;
  const long long need = decode_ws_bytes(B, H, Nq, d, decode_plan(B, H_kv, Nq, Nk, mask_kind, win).n_chunks);
  if (need > FA_DECODE_SCRATCH_BYTES)
    return fail(FA_ERR_INVALID_ARG,
                "these sizes need %lld bytes of chunk partials; the static scratch holds %lld",
                need, (long long)FA_DECODE_SCRATCH_BYTES);
  st = check_device();
  if (st != FA_OK) return st;
  void* scratch = nullptr;
  const hipError_t e = fa_decode_scratch(&scratch);
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "address of the decode scratch: %s", hipGetErrorString(e));
  return run_decode(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind, window, dtype,
                    scratch, FA_DECODE_SCRATCH_BYTES, stream);
}

// Few key/value heads leave the dk/dv pass with few workgroups (one per
// key/value head and 128-key tile), each running all g = H / H_kv query
// heads.  Then the query heads are split over kv_parts workgroups per tile
// (aiming at four workgroups per compute unit), whose fp32 partial sums go
// to dq's memory -- free until the dq pass, which runs last -- and are added
// by a small kernel.  The partials take 8 kv_parts B H_kv N d bytes of dq's
// 2 B H N d, hence kv_parts <= g / 4.  (Arguments already validated.)
static int bwd_kv_parts(int B, int H, int H_kv, int N, int cus) {
  const long long tiles =
      (long long)B * H_kv * (((long long)N + FA_BWD_WAVES * 32 - 1) / (FA_BWD_WAVES * 32));
  const long long want = 4LL * cus;
  const int cap = (H / H_kv) / 4;
  if (cap < 2 || tiles >= want) return 1;
  return (int)std::min<long long>(cap, (want + tiles - 1) / tiles);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
               int H_kv, int N, int d, float scale, int mask_kind, int window, int dtype,
               void* stream) {
  int st = check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, scale,
                          mask_kind, window, dtype);
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  FaBwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.BH = B * H;
  p.kv_group = H / H_kv;
  p.N = N;
  p.mask_kind = mask_kind;
  p.window = mask_kind == FA_MASK_SLIDING ? (window < N ? window : N) : 0;
  p.scale = scale;
  // as in the forward call: scale = 0 becomes the smallest normal float,
  // whose weights are uniform to fp32 precision
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  if (!(p.scale_log2 >= FLT_MIN)) p.scale_log2 = FLT_MIN;
  p.n_q_tiles = (N + FA_BWD_DQ_WAVES * 32 - 1) / (FA_BWD_DQ_WAVES * 32);
  p.n_k_tiles = (N + FA_BWD_WAVES * 32 - 1) / (FA_BWD_WAVES * 32);
  p.heavy_first = mask_kind != FA_MASK_NONE ? 1 : 0;
  p.kv_parts = bwd_kv_parts(B, H, H_kv, N, device_cus());
  p.part_scratch = p.kv_parts > 1 ? (float*)dq : nullptr;
  hipError_t e = fa_launch_bwd(dtype, d, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
           int d, float scale, int mask_kind, int window, int dtype, void* stream) {
  return fa_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H, N, d, scale, mask_kind,
                    window, dtype, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int d, float scale, int mask_kind, int window, int in_dtype, int out_dtype,
           void* stream) {
  if (in_dtype == FA_DTYPE_E4M3)
    return fail(FA_ERR_INVALID_ARG, "E4M3 inputs go through fa_fwd_fp8");
  return run_fwd(q, k, v, o, lse, B, H, H, N, d, scale, 1.f, mask_kind, window, in_dtype,
                 out_dtype, nullptr, stream);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int H, int H_kv, int N, int d, float scale, int mask_kind, int window,
               int in_dtype, int out_dtype, void* stream) {
  if (in_dtype == FA_DTYPE_E4M3)
    return fail(FA_ERR_INVALID_ARG, "E4M3 inputs go through fa_fwd_fp8");
  return run_fwd(q, k, v, o, lse, B, H, H_kv, N, d, scale, 1.f, mask_kind, window, in_dtype,
                 out_dtype, nullptr, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int H, int H_kv, int N, int d, float scale, float v_scale, int mask_kind,
               int window, int out_dtype, void* stream) {
  if (!std::isfinite(v_scale))
    return fail(FA_ERR_INVALID_ARG, "v_scale must be finite");
  return run_fwd(q, k, v, o, lse, B, H, H_kv, N, d, scale, v_scale, mask_kind, window,
                 FA_DTYPE_E4M3, out_dtype, nullptr, stream);
}

int fa_fwd_record_tiles(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, float scale, int mask_kind, int window,
                        int in_dtype, int out_dtype, unsigned char* tiles, void* stream) {
  if (!tiles) return fail(FA_ERR_INVALID_ARG, "null tiles buffer");
  if (in_dtype == FA_DTYPE_E4M3)
    return fail(FA_ERR_INVALID_ARG, "E4M3 inputs go through fa_fwd_fp8");
  return run_fwd(q, k, v, o, lse, B, H, H, N, d, scale, 1.f, mask_kind, window, in_dtype,
                 out_dtype, tiles, stream);
}

int fa_bwd_kv_parts(int B, int H, int H_kv, int N, int compute_units, int* parts) {
  if (!parts) return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || H < 1 || N < 1 || compute_units < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H, N and compute_units must be >= 1");
  if (N >= (1 << 30)) return fail(FA_ERR_INVALID_ARG, "N must be < 2^30");
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "H_kv must divide H = %d (got %d)", H, H_kv);
  *parts = bwd_kv_parts(B, H, H_kv, N, compute_units);
  return ok();
}

int fa_tile_shape(int d, int in_dtype, int* rows_per_workgroup, int* rows_per_wave,
                  int* keys_per_block_out) {
  if (!rows_per_workgroup || !rows_per_wave || !keys_per_block_out)
    return fail(FA_ERR_INVALID_ARG, "null output pointer");
  if (!valid_dtype(in_dtype)) return fail(FA_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (!fa_head_dim_built(in_dtype, d))
    return fail(FA_ERR_UNSUPPORTED, "head dim %d not built (64, 128; 256 for f16/bf16)", d);
  *rows_per_workgroup = fa_rows_per_wg(in_dtype, d);
  *rows_per_wave = FA_ROW_BLOCK;
  *keys_per_block_out = keys_per_block(in_dtype, d);
  return ok();
}

int fa_tile_map(int N, int d, int in_dtype, int mask_kind, int window, unsigned char* out) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "null output pointer");
  if (N < 1 || N >= (1 << 30)) return fail(FA_ERR_INVALID_ARG, "bad N %d", N);
  if (!valid_dtype(in_dtype)) return fail(FA_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL && mask_kind != FA_MASK_SLIDING)
    return fail(FA_ERR_INVALID_ARG, "unknown mask_kind %d", mask_kind);
  if (mask_kind == FA_MASK_SLIDING && window < 1)
    return fail(FA_ERR_INVALID_ARG, "sliding window must be >= 1 (got %d)", window);
  if (!fa_head_dim_built(in_dtype, d))
    return fail(FA_ERR_UNSUPPORTED, "head dim %d not built (64, 128; 256 for f16/bf16)", d);
  const int bc = keys_per_block(in_dtype, d);
  const int R = (N + FA_ROW_BLOCK - 1) / FA_ROW_BLOCK;
  const int C = (N + bc - 1) / bc;
  for (int rb = 0; rb < R; ++rb) {
    const int r0 = rb * FA_ROW_BLOCK;
    const int r1 = r0 + FA_ROW_BLOCK < N ? r0 + FA_ROW_BLOCK : N;
    for (int kb = 0; kb < C; ++kb)
      out[(size_t)rb * C + kb] =
          (unsigned char)fa_classify(r0, r1, kb * bc, bc, N, mask_kind, window);
  }
  return ok();
}

int fa_fwd_schedule(int B, int H, int H_kv, int N, int d, int in_dtype, int mask_kind,
                    int window, int compute_units, int* n_workgroups, int* max_tiles, int* out,
                    long long out_len) {
  if (!n_workgroups || !max_tiles) return fail(FA_ERR_INVALID_ARG, "null output pointer");
  if (B < 1 || H < 1 || N < 1 || N >= (1 << 30) || compute_units < 1)
    return fail(FA_ERR_INVALID_ARG, "bad sizes B=%d H=%d N=%d compute_units=%d", B, H, N,
                compute_units);
  if (H_kv < 1 || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "H=%d is not a multiple of H_kv=%d", H, H_kv);
  if (!valid_dtype(in_dtype) && in_dtype != FA_DTYPE_E4M3)
    return fail(FA_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL && mask_kind != FA_MASK_SLIDING)
    return fail(FA_ERR_INVALID_ARG, "unknown mask_kind %d", mask_kind);
  if (mask_kind == FA_MASK_SLIDING && window < 1)
    return fail(FA_ERR_INVALID_ARG, "sliding window must be >= 1 (got %d)", window);
  if (!fa_head_dim_built(in_dtype, d))
    return fail(FA_ERR_UNSUPPORTED, "head dim %d not built for in_dtype %d", d, in_dtype);
  const int rows = fa_rows_per_wg(in_dtype, d);
  const long long T = (N + rows - 1) / rows;
  if ((long long)B * H * T >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARG, "B*H*row tiles beyond int range");
  FaFwdParams p{};
  p.BH = B * H;
  p.kv_group = H / H_kv;
  p.N = N;
  p.window = mask_kind == FA_MASK_SLIDING ? (window < N ? window : N) : 0;
  p.n_row_tiles = (int)T;
  fa_fwd_plan(p, mask_kind, compute_units, rows);
  const bool persistent = fa_fwd_persistent(in_dtype, d);
  const long long G = persistent ? (long long)p.n_groups * p.wg_per_group : (long long)p.BH * T;
  const long long R = persistent ? (p.tiles_per_group + p.wg_per_group - 1) / p.wg_per_group : 1;
  *n_workgroups = (int)G;
  *max_tiles = (int)R;
  if (!out) return ok();
  if (out_len < 2 * G * R)
    return fail(FA_ERR_INVALID_ARG, "out holds %lld ints, the schedule needs %lld", out_len,
                2 * G * R);
  for (long long g = 0; g < G; ++g)
    for (long long k = 0; k < R; ++k) {
      int bh = -1, qt = -1;
      if (persistent) {
        if (!fa_persist_tile_of(p, (int)g, (int)k, &bh, &qt)) bh = qt = -1;
      } else {
        fa_plain_tile_of(p, (int)g, &bh, &qt);
      }
      out[2 * (g * R + k)] = bh;
      out[2 * (g * R + k) + 1] = qt;
    }
  return ok();
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_NO_DEVICE: return "FA_ERR_NO_DEVICE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_ERR_UNKNOWN";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_probe_mfma(int which, const void* a, const void* b, float* d, void* stream) {
  if (which < 0 || which > 4) return fail(FA_ERR_INVALID_ARG, "which must be 0 .. 4");
  if (!a || !b || !d) return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if ((((uintptr_t)a | (uintptr_t)b) & 15u) != 0 || ((uintptr_t)d & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "misaligned operand");
  int st = check_device();
  if (st != FA_OK) return st;
  hipError_t e = which <= 2 ? fa_launch_probe(which, a, b, d, (hipStream_t)stream)
                            : fa_launch_probe8(which - 3, a, b, d, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return ok();
}

int fa_mfma_ceiling(int n_blocks, int iters, unsigned long long* clocks, float* sink,
                    void* stream) {
  if (n_blocks < 1 || iters < 1) return fail(FA_ERR_INVALID_ARG, "n_blocks and iters must be >= 1");
  if (!clocks || !sink) return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if (((uintptr_t)clocks & 7u) != 0 || ((uintptr_t)sink & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "misaligned buffer");
  int st = check_device();
  if (st != FA_OK) return st;
  hipError_t e = fa_launch_mfma_ceiling(n_blocks, iters, clocks, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "ceiling launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
