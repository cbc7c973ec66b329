// C ABI of the library: argument validation, launch configuration, dispatch.
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect on the device or the stream.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/prope.h"
#include "internal.hpp"

namespace prope {

void fill_rope_freq(RopeFreq& f, int d, double base, long double s) {
  // F_i = round(theta_i / (2 pi s) * 2^64), theta_i = base^(-2i/d) (P-RoPE page, Eq. (1));
  // s > 1 gives the interpolated frequencies theta_i / s. theta_i is the running
  // product of base^(-2/d) in long double (one powl per call instead of one per
  // pair, which cost ~20 us of host time per call): after 63 steps its relative
  // error is ~2^-58, a phase error of ~2^-43 turn at ids near 2^17, far below the
  // 2^-32 turn the kernels resolve.
  const long double two_pi = 2.0L * acosl(-1.0L);
  const long double ratio = powl(static_cast<long double>(base), -2.0L / d);
  const long double scale = 18446744073709551616.0L / (two_pi * s);  // 2^64 / (2 pi s)
  long double theta = 1.0L;
  for (int i = 0; i < kMaxPairs; ++i) {
    uint64_t F = 0;
    if (i < d / 2) {
      F = static_cast<uint64_t>(theta * scale + 0.5L);
      theta *= ratio;
    }
    f.lo[i] = static_cast<uint32_t>(F);
    f.hi[i] = static_cast<uint32_t>(F >> 32);
  }
}

}  // namespace prope

using namespace prope;

namespace {

bool valid_base(double b) { return isfinite(b) && b > 1.0; }

// Common checks of the mode parameters. `decode` forbids a period (the
// cache already carries the layer's rotation).
int check_params(const prope_params* p, bool decode) {
  if (!p) return PROPE_ERR_INVALID_ARG;
  if (p->reserved != 0) return PROPE_ERR_INVALID_ARG;
  if (p->w_pretrained < 0) return PROPE_ERR_INVALID_ARG;
  if (p->remote_map != PROPE_REMOTE_ALIAS && p->remote_map != PROPE_REMOTE_INTERP) return PROPE_ERR_INVALID_ARG;
  if (p->remote_map == PROPE_REMOTE_INTERP && p->mode != PROPE_BIFOCAL) return PROPE_ERR_INVALID_ARG;
  if (p->w_pretrained > 0 && (p->mode != PROPE_BIFOCAL || p->remap_scale != 1)) return PROPE_ERR_INVALID_ARG;
  // a real interpolation scale: finite, >= 1, and the only source of s
  if (!(p->interp_scale == 0.0 || (isfinite(p->interp_scale) && p->interp_scale >= 1.0))) return PROPE_ERR_INVALID_ARG;
  if (p->interp_scale != 0.0 &&
      (p->remote_map != PROPE_REMOTE_INTERP || p->remap_scale != 1 || p->w_pretrained != 0))
    return PROPE_ERR_INVALID_ARG;
  // ALiBi biases belong to the nope/rope layers (P-RoPE page, section 1)
  if (p->alibi_slopes && p->mode == PROPE_BIFOCAL) return PROPE_ERR_INVALID_ARG;
  if (p->mode != PROPE_NOPE && p->mode != PROPE_ROPE && p->mode != PROPE_BIFOCAL)
    return PROPE_ERR_INVALID_ARG;
  if (p->period < 0 || p->remap_scale < 1 || p->window_left < -1) return PROPE_ERR_INVALID_ARG;
  if (!(p->softmax_scale >= 0.0f) || !isfinite(p->softmax_scale)) return PROPE_ERR_INVALID_ARG;
  if (p->period != 0 && (p->mode != PROPE_ROPE || decode)) return PROPE_ERR_INVALID_ARG;
  if (p->remap_scale != 1 && p->mode != PROPE_BIFOCAL) return PROPE_ERR_INVALID_ARG;
  if (p->mode != PROPE_NOPE && !valid_base(p->rope_base)) return PROPE_ERR_INVALID_ARG;
  return PROPE_OK;
}

// The aliasing scale s for a sequence of length L: remap_scale, or the dynamic
// group size of Jet-Long Eq. (2) when w_pretrained > 0.
int remote_scale(const prope_params& p, int64_t L) {
  if (p.w_pretrained <= 0) return p.remap_scale;
  const int64_t g = L / p.w_pretrained + (L % p.w_pretrained != 0);
  return g < 1 ? 1 : static_cast<int>(g);
}

// The interpolation scale s for a sequence of length L: interp_scale, else the
// continuous-style factor max(1, L / w_pretrained) of Jet-Long section 3.1 when
// w_pretrained > 0, else the integer remap_scale.
long double interp_scale(const prope_params& p, int64_t L) {
  if (p.interp_scale > 0.0) return p.interp_scale;
  if (p.w_pretrained > 0) {
    const long double s = static_cast<long double>(L) / p.w_pretrained;
    return s > 1.0L ? s : 1.0L;
  }
  return p.remap_scale;
}

float scale_log2(const prope_params* p, int d) {
  const double s = p->softmax_scale > 0.0f ? p->softmax_scale : 1.0 / sqrt(static_cast<double>(d));
  return static_cast<float>(s * 1.4426950408889634);  // * log2(e)
}

int check_prefill(const void* q, const void* k, const void* v, const void* o, const int32_t* pos, int B, int S,
                  int Hq, int Hkv, int d, int dt, const prope_params* params) {
  const int pc = check_params(params, false);
  if (pc != PROPE_OK) return pc;
  if (!q || !k || !v || !o) return PROPE_ERR_INVALID_ARG;
  if (!pos && params->mode != PROPE_NOPE) return PROPE_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || (Hq % Hkv)) return PROPE_ERR_INVALID_ARG;
  if (dt != PROPE_BF16 && dt != PROPE_FP32) return PROPE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return PROPE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o)) % 16)
    return PROPE_ERR_INVALID_ARG;
  // one sequence's q/k/v/o slices are addressed with 32-bit byte offsets
  if (int64_t(S) * Hq * d * 4 >= (int64_t(1) << 32)) return PROPE_ERR_UNSUPPORTED;
  return PROPE_OK;
}

// Decode split policy: a workgroup takes a chunk of keys for hpw KV heads.
//  - 4 heads x 1024 keys (one wave per head) when Hkv % 4 == 0 and that grid
//    has at most one workgroup per compute unit (batch 1 at 128K): the 4 heads'
//    slices of a row are contiguous, which measured 5% faster than one head
//    per workgroup, the combine aside;
//  - else 1 head x 4096 keys when that grid fits in one round, else 2048;
//  - short caches, whose grid would have fewer than kDecodeMinGrid workgroups,
//    halve the chunk until it does or a wave is down to kDecodeMinWaveKeys keys.
constexpr int kDecodeChunkRows = 1024;
constexpr int kDecodeChunk = 2048;
constexpr int kDecodeChunkLarge = 4096;
constexpr int kDecodeMinGrid = 256;
constexpr int kDecodeMinWaveKeys = 128;

// Upper bound of the chunks per sequence that prope_attn_decode uses for a
// cache of Lmax keys (its workspace holds one partial per chunk and head):
// without shrinking a chunk has at least 1024 keys; a shrunk one at least
// kDecodeMinWaveKeys, and the last halving happened with fewer than
// kDecodeMinGrid workgroups, so there are fewer than 2 * kDecodeMinGrid chunks.
size_t decode_max_chunks(int Lmax) {
  const size_t L = static_cast<size_t>(Lmax);
  const size_t base = (L + kDecodeChunkRows - 1) / kDecodeChunkRows;
  const size_t shrunk = std::min<size_t>(2 * kDecodeMinGrid, (L + kDecodeMinWaveKeys - 1) / kDecodeMinWaveKeys);
  return std::max(base, shrunk);
}

// compute units of the current device (256 if it cannot be read)
int device_cus() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    n_cu = 256;
  return n_cu;
}

// `freq_scale` divides the base frequencies (theta_i / freq_scale): the remote
// calls of the unfused composition with the interpolation map.
PrefillArgs prefill_args(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* pos,
                         int B, int S, int Hq, int Hkv, int d, const prope_params& p, uint32_t* queue = nullptr,
                         long double freq_scale = 1.0L) {
  PrefillArgs a{};
  a.queue = queue;
  a.n_cu = queue ? device_cus() : 0;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.pos = pos;
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.D = d;
  a.G = Hq / Hkv;
  a.HG = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0) ? 2 : 1;
  a.BMp = 256 / a.HG;
  a.n_pblocks = (S + a.BMp - 1) / a.BMp;
  a.n_hsub = a.G / a.HG;
  a.mode = p.mode;
  a.period = p.period;
  a.window_left = p.window_left;
  a.period_div = make_fastdiv(p.period > 0 ? static_cast<uint32_t>(p.period) : 1u);
  const bool interp = p.remote_map == PROPE_REMOTE_INTERP;
  a.scale_div = make_fastdiv(static_cast<uint32_t>(interp ? 1 : remote_scale(p, S)));
  a.scale_log2 = scale_log2(&p, d);
  a.alibi = p.alibi_slopes;
  fill_rope_freq(a.f, d, p.mode == PROPE_NOPE ? 10000.0 : p.rope_base, freq_scale);
  if (interp)
    fill_rope_freq(a.fr, d, p.rope_base, interp_scale(p, S));
  else
    a.fr = a.f;
  return a;
}

// Whether the launch grid of a prefill call fits the device's launch limits.
bool prefill_fits(const PrefillArgs& a, int dt) {
  return dt == PROPE_BF16 ? prefill_bf16_fits(a) : prefill_fp32_fits(a);
}

int run_prefill(const PrefillArgs& a, int dt, void* stream) {
  const hipError_t e = dt == PROPE_BF16 ? launch_prefill_bf16(a, static_cast<hipStream_t>(stream))
                                        : launch_prefill_fp32(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PROPE_OK : PROPE_ERR_HIP;
}

// Workspace of the unfused composition: O_A and O_C in the input dtype, the
// three LSE vectors, the remote ids and the work queue of the three calls,
// each region 256-byte aligned. O_B is written into the caller's output.
struct UnfusedLayout {
  size_t oa, oc, la, lb, lc, ids, queue, total;
};
UnfusedLayout unfused_layout(int B, int S, int Hq, int d, int dt) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t obytes = up(size_t(B) * S * Hq * d * (dt == PROPE_BF16 ? 2 : 4));
  const size_t lbytes = up(size_t(B) * Hq * S * sizeof(float));
  UnfusedLayout l;
  l.oa = 0;
  l.oc = l.oa + obytes;
  l.la = l.oc + obytes;
  l.lb = l.la + lbytes;
  l.lc = l.lb + lbytes;
  l.ids = l.lc + lbytes;
  l.queue = l.ids + up(size_t(B) * S * sizeof(int32_t));
  l.total = l.queue + up(kQueueWords * sizeof(uint32_t));
  return l;
}

// Validation and launch set-up shared by the decode entry points (everything
// but the workspace). The chunk policy is described above kDecodeChunkRows.
int decode_setup(DecodeArgs& a, const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                 const int32_t* kv_len, int B, int Lmax, int Hq, int Hkv, int d, int dt,
                 const prope_params* params) {
  const int pc = check_params(params, true);
  if (pc != PROPE_OK) return pc;
  if (!q || !k_cache || !v_cache || !o || !kv_len) return PROPE_ERR_INVALID_ARG;
  if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || (Hq % Hkv)) return PROPE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return PROPE_ERR_INVALID_ARG;
  if (dt != PROPE_BF16 && dt != PROPE_FP32) return PROPE_ERR_INVALID_ARG;
  if (dt != PROPE_BF16) return PROPE_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return PROPE_ERR_UNSUPPORTED;  // query heads of a group fill one 16-wide MFMA tile
  if (B > 65535 || Hkv > 65535) return PROPE_ERR_UNSUPPORTED;  // grid y and z limits
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(o)) % 16)
    return PROPE_ERR_INVALID_ARG;
  // one sequence's cache slice is addressed with 32-bit byte offsets
  if (int64_t(Lmax) * Hkv * d * 2 >= (int64_t(1) << 32)) return PROPE_ERR_UNSUPPORTED;
  const bool interp = params->remote_map == PROPE_REMOTE_INTERP;

  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse; a.kv_len = kv_len;
  a.ws = nullptr;
  a.B = B; a.Lmax = Lmax; a.Hq = Hq; a.Hkv = Hkv; a.D = d; a.G = Hq / Hkv;
  const int n_cu = device_cus();
  const int64_t wg_rows = int64_t(B) * (Hkv / 4) * ((Lmax + kDecodeChunkRows - 1) / kDecodeChunkRows);
  const int64_t wg_large = int64_t(B) * Hkv * ((Lmax + kDecodeChunkLarge - 1) / kDecodeChunkLarge);
  if (Hkv % 4 == 0 && wg_rows <= n_cu) {
    a.hpw = 4;
    a.chunk = kDecodeChunkRows;
  } else {
    a.hpw = 1;
    a.chunk = wg_large <= n_cu ? kDecodeChunkLarge : kDecodeChunk;
  }
  // Short caches: halve the chunk while the grid has fewer than kDecodeMinGrid
  // workgroups, down to kDecodeMinWaveKeys keys per wave, so that the waves'
  // serial key loops get shorter instead of most of the chip idling.
  const int kw = 4 / a.hpw;
  auto grid = [&](int c) { return int64_t(B) * (Hkv / a.hpw) * ((Lmax + c - 1) / c); };
  while (grid(a.chunk) < kDecodeMinGrid && a.chunk / 2 >= kDecodeMinWaveKeys * kw) a.chunk /= 2;
  a.n_chunks = (Lmax + a.chunk - 1) / a.chunk;
  a.mode = params->mode;
  a.window_left = params->window_left;
  a.scale_div = make_fastdiv(static_cast<uint32_t>(interp ? 1 : params->remap_scale));
  a.w_pre = params->w_pretrained;
  a.scale_log2 = scale_log2(params, d);
  a.alibi = params->alibi_slopes;
  fill_rope_freq(a.f, d, params->mode == PROPE_NOPE ? 10000.0 : params->rope_base);
  a.interp = interp;
  if (interp && a.w_pre > 0) {
    a.fr = a.f;  // per sequence: the kernel forms theta_i / s - theta_i from f and kv_len
  } else if (interp) {  // correction frequencies theta_i / s - theta_i, modulo one turn
    RopeFreq fs;
    fill_rope_freq(fs, d, params->rope_base, interp_scale(*params, Lmax));
    for (int i = 0; i < kMaxPairs; ++i) {
      const uint64_t c = ((uint64_t(fs.hi[i]) << 32) | fs.lo[i]) - ((uint64_t(a.f.hi[i]) << 32) | a.f.lo[i]);
      a.fr.lo[i] = static_cast<uint32_t>(c);
      a.fr.hi[i] = static_cast<uint32_t>(c >> 32);
    }
  } else {
    a.fr = a.f;
  }
  return PROPE_OK;
}

}  // namespace

extern "C" {

int prope_version(void) { return PROPE_VERSION; }

const char* prope_status_string(int status) {
  switch (status) {
    case PROPE_OK: return "PROPE_OK";
    case PROPE_ERR_INVALID_ARG: return "PROPE_ERR_INVALID_ARG: invalid argument";
    case PROPE_ERR_UNSUPPORTED: return "PROPE_ERR_UNSUPPORTED: valid but unsupported combination";
    case PROPE_ERR_WORKSPACE: return "PROPE_ERR_WORKSPACE: workspace too small";
    case PROPE_ERR_HIP: return "PROPE_ERR_HIP: HIP launch failed";
    default: return "unknown prope status";
  }
}

int prope_group_size(int64_t L, int64_t w_pretrained) {
  // Jet-Long section 3.1, Eq. (2).
  if (L < 0 || w_pretrained < 1) return -1;
  const int64_t g = L / w_pretrained + (L % w_pretrained != 0);  // ceil without overflow at L near 2^63
  if (g > INT32_MAX) return -1;
  return g < 1 ? 1 : static_cast<int>(g);
}

int prope_rope_apply(const void* x, void* y, const int32_t* pos, int B, int S, int H, int d,
                     int dt, double rope_base, void* stream) {
  if (!x || !y || !pos) return PROPE_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || H < 1 || d < 2 || d > 2 * kMaxPairs || (d % 2)) return PROPE_ERR_INVALID_ARG;
  if (dt != PROPE_BF16 && dt != PROPE_FP32) return PROPE_ERR_INVALID_ARG;
  if (!valid_base(rope_base)) return PROPE_ERR_INVALID_ARG;
  const size_t esz = dt == PROPE_BF16 ? 2 : 4;
  // exact aliasing is fine; partial overlap is not
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(y);
  const size_t bytes = size_t(B) * S * H * d * esz;
  if (xa != ya && xa < ya + bytes && ya < xa + bytes) return PROPE_ERR_INVALID_ARG;
  if ((d % 8) == 0 ? (xa % 16 || ya % 16) : (xa % (2 * esz) || ya % (2 * esz)))
    return PROPE_ERR_INVALID_ARG;
  RopeFreq f;
  fill_rope_freq(f, d, rope_base);
  const hipError_t e = launch_rope_apply(x, y, pos, B, S, H, d, dt, f, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PROPE_OK : PROPE_ERR_HIP;
}

int prope_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int dt,
                       const prope_params* params, void* stream) {
  const int pc = check_prefill(q, k, v, o, pos, B, S, Hq, Hkv, d, dt, params);
  if (pc != PROPE_OK) return pc;
  const PrefillArgs a = prefill_args(q, k, v, o, lse, pos, B, S, Hq, Hkv, d, *params);
  if (!prefill_fits(a, dt)) return PROPE_ERR_UNSUPPORTED;
  return run_prefill(a, dt, stream);
}

size_t prope_prefill_queue_size(void) { return kQueueWords * sizeof(uint32_t); }

int prope_attn_prefill_queued(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int dt,
                              const prope_params* params, void* queue, void* stream) {
  const int pc = check_prefill(q, k, v, o, pos, B, S, Hq, Hkv, d, dt, params);
  if (pc != PROPE_OK) return pc;
  if (!queue || reinterpret_cast<uintptr_t>(queue) % 128) return PROPE_ERR_INVALID_ARG;
  // the fp32 kernel has no queue: it runs its static schedule and leaves the buffer as it is
  uint32_t* wq = dt == PROPE_BF16 ? static_cast<uint32_t*>(queue) : nullptr;
  const PrefillArgs a = prefill_args(q, k, v, o, lse, pos, B, S, Hq, Hkv, d, *params, wq);
  if (!prefill_fits(a, dt)) return PROPE_ERR_UNSUPPORTED;
  return run_prefill(a, dt, stream);
}

size_t prope_bifocal_unfused_workspace_size(int B, int S, int Hq, int d, int dt) {
  if (B < 1 || S < 1 || Hq < 1 || d < 1 || (dt != PROPE_BF16 && dt != PROPE_FP32)) return 0;
  return unfused_layout(B, S, Hq, d, dt).total;
}

int prope_attn_prefill_bifocal_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                                       const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int dt,
                                       const prope_params* params, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  const int pc = check_prefill(q, k, v, o, pos, B, S, Hq, Hkv, d, dt, params);
  if (pc != PROPE_OK) return pc;
  if (params->mode != PROPE_BIFOCAL || !pos || !workspace) return PROPE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return PROPE_ERR_INVALID_ARG;
  const UnfusedLayout ly = unfused_layout(B, S, Hq, d, dt);
  if (workspace_bytes < ly.total) return PROPE_ERR_WORKSPACE;
  // every launch is checked against the grid limits before the first is enqueued
  // (the three calls share one grid; the merge takes a thread per 8 elements)
  if (!prefill_fits(prefill_args(q, k, v, o, lse, pos, B, S, Hq, Hkv, d, *params), dt) ||
      int64_t(B) * S * Hq * (d / 8) > kMaxWorkItems)
    return PROPE_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  void* oa = ws + ly.oa;
  void* oc = ws + ly.oc;
  float* la = reinterpret_cast<float*>(ws + ly.la);
  float* lb = reinterpret_cast<float*>(ws + ly.lb);
  float* lc = reinterpret_cast<float*>(ws + ly.lc);
  int32_t* rid = reinterpret_cast<int32_t*>(ws + ly.ids);
  // the work queue of the three calls: cleared once here, each call leaves it clear
  uint32_t* wq = dt == PROPE_BF16 ? reinterpret_cast<uint32_t*>(ws + ly.queue) : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int w0 = params->window_left;

  // The three calls are plain RoPE attention (no period). The remote view
  // (B, C) is RoPE at the ids floor(pos / s) (aliasing), or at the ids pos
  // with the frequencies theta_i / s (interpolation).
  prope_params call = *params;
  call.mode = PROPE_ROPE;
  call.remap_scale = 1;
  call.period = 0;
  call.w_pretrained = 0;
  call.remote_map = PROPE_REMOTE_ALIAS;
  call.interp_scale = 0.0;
  const bool interp = params->remote_map == PROPE_REMOTE_INTERP;
  const long double rscale = interp ? interp_scale(*params, S) : 1.0L;
  const int32_t* rpos = interp ? pos : rid;
  if (!interp && launch_remap_ids(pos, rid, int64_t(B) * S,
                                  make_fastdiv(static_cast<uint32_t>(remote_scale(*params, S))), st) != hipSuccess)
    return PROPE_ERR_HIP;
  if (wq && launch_zero_words(wq, kQueueWords, st) != hipSuccess) return PROPE_ERR_HIP;
  // B: full causal attention in the remote view, written straight into o
  call.window_left = -1;
  int rc = run_prefill(prefill_args(q, k, v, o, lb, rpos, B, S, Hq, Hkv, d, call, wq, rscale), dt, stream);
  if (rc != PROPE_OK) return rc;
  const bool windows = w0 >= 0;  // w0 = -1: no local window, the result is B alone
  if (windows) {
    // A: the local window at the ids themselves; C: the local window in the remote view
    call.window_left = w0;
    rc = run_prefill(prefill_args(q, k, v, oa, la, pos, B, S, Hq, Hkv, d, call, wq), dt, stream);
    if (rc != PROPE_OK) return rc;
    rc = run_prefill(prefill_args(q, k, v, oc, lc, rpos, B, S, Hq, Hkv, d, call, wq, rscale), dt, stream);
    if (rc != PROPE_OK) return rc;
  }
  return launch_eq7_merge(oa, la, o, lb, oc, lc, lse, B, S, Hq, d, dt, windows, st) == hipSuccess ? PROPE_OK
                                                                                               : PROPE_ERR_HIP;
}

size_t prope_decode_workspace_size(int B, int Lmax, int Hq, int d) {
  if (B < 1 || Lmax < 1 || Hq < 1 || d < 1) return 0;
  return size_t(B) * Hq * decode_max_chunks(Lmax) * (size_t(d) + 2) * sizeof(float);
}

int prope_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int32_t* kv_len, int B, int Lmax, int Hq, int Hkv, int d, int dt,
                      const prope_params* params, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 16) return PROPE_ERR_INVALID_ARG;
  DecodeArgs a{};
  const int rc = decode_setup(a, q, k_cache, v_cache, o, lse, kv_len, B, Lmax, Hq, Hkv, d, dt, params);
  if (rc != PROPE_OK) return rc;
  if (workspace_bytes < prope_decode_workspace_size(B, Lmax, Hq, d)) return PROPE_ERR_WORKSPACE;
  a.ws = static_cast<float*>(workspace);
  const hipError_t e = launch_decode_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PROPE_OK : PROPE_ERR_HIP;
}

int prope_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                              const int32_t* kv_len, int B, int Lmax, int Hq, int Hkv, int d, int dt,
                              const prope_params* params, void* stream) {
  DecodeArgs a{};
  const int rc = decode_setup(a, q, k_cache, v_cache, o, lse, kv_len, B, Lmax, Hq, Hkv, d, dt, params);
  if (rc != PROPE_OK) return rc;
  // the partials of this launch's chunk choice must fit the fixed array
  if (size_t(B) * Hq * a.n_chunks * (size_t(d) + 2) * sizeof(float) > kDecodeScratchBytes)
    return PROPE_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (decode_scratch(&scratch) != hipSuccess) return PROPE_ERR_HIP;
  a.ws = static_cast<float*>(scratch);
  const hipError_t e = launch_decode_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PROPE_OK : PROPE_ERR_HIP;
}

}  // extern "C"
