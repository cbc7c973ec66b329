// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace prope {

enum Mode : int { kNope = 0, kRope = 1, kBifocal = 2 };

// Everything a prefill launch needs; built and validated by the ABI layer.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* pos;
  int B, S, Hq, Hkv, D;
  int G;          // Hq / Hkv
  int HG;         // query heads of one KV group handled by one workgroup
  int BMp;        // query positions per workgroup (BMp * HG == rows per workgroup)
  int n_pblocks;  // ceil(S / BMp)
  int n_hsub;     // G / HG
  int mode;
  int period;       // ROPE: P (0 = none)
  int window_left;  // NOPE/ROPE: max kept i-j (-1 none); BIFOCAL: w0
  FastDiv period_div;
  FastDiv scale_div;  // remote ids floor(p / div): s (alias) or 1 (interpolation)
  float scale_log2;   // softmax scale * log2(e)
  RopeFreq f;         // theta_i at the base ids
  RopeFreq fr;        // theta_i at the remote ids: theta_i (alias) or theta_i / s
  const float* alibi; // NOPE/ROPE: Hq ALiBi slopes (device), or nullptr
  uint32_t* queue;    // bf16: work-queue counters (kQueueWords), or nullptr: one item per workgroup
  int n_cu;           // compute units of the device (persistent grid size with a queue)
};

// Prefill work queue: 8 per-XCD item counters, 8 per-XCD done counts and one
// global done count, each in its own 128-byte line (atomics on one line
// serialise).
constexpr int kQueueLine = 32;  // 32-bit words per counter line
constexpr int kQueueWords = 17 * kQueueLine;

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_len;
  float* ws;  // [B][Hq][n_chunks][D + 2]
  int B, Lmax, Hq, Hkv, D, G;
  int chunk;     // keys per workgroup and head (a multiple of 4 * 32); one partial each
  int n_chunks;  // chunks of a sequence's cache: ceil(Lmax / chunk)
  int hpw;       // KV heads per workgroup: 4 (each wave one head, Hkv % 4 == 0) or 1
                 // (the 4 waves split the chunk of one head)
  int mode;
  int window_left;
  FastDiv scale_div;  // remote scale s (alias, w_pre == 0)
  int w_pre;          // > 0: per-sequence scale from kv_len: alias s = max(1, ceil(kv_len / w_pre));
                      // interpolation s = max(1, kv_len / w_pre), whose correction
                      // frequencies the kernel forms from f
  int interp;         // remote angles p * theta_i / s instead of floor(p / s) * theta_i
  float scale_log2;
  const float* alibi; // NOPE/ROPE: Hq ALiBi slopes (device), or nullptr
  RopeFreq f;         // theta_i
  RopeFreq fr;        // correction frequencies: theta_i (alias, index floor(p/s) - p) or
                      // theta_i / s - theta_i (interpolation, index p; unused with w_pre > 0)
};

// Fill F_i = round(theta_i / (2 pi s) * 2^64), theta_i = base^(-2i/d), in long double
// (s >= 1 real: the interpolated frequencies theta_i / s).
void fill_rope_freq(RopeFreq& f, int d, double base, long double s = 1.0L);

hipError_t launch_rope_apply(const void* x, void* y, const int32_t* pos, int B, int S, int H,
                             int d, int dt, const RopeFreq& f, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_fp32(const PrefillArgs& a, hipStream_t stream);

// A 1-D launch covers at most 2^32 - 1 work-items (the dispatch packet holds the
// grid size in work-items in 32 bits). The prefill launchers' grids, as host-side
// checks made before anything is enqueued:
constexpr int64_t kMaxWorkItems = 0xffffffffLL;
bool prefill_bf16_fits(const PrefillArgs& a);
bool prefill_fp32_fits(const PrefillArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// The fixed device array that prope_attn_decode_noalloc uses for its split-K
// partials (decode_scratch.hip): its size, and its address on the current device.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_remap_ids(const int32_t* pos, int32_t* out, int64_t n, const FastDiv& s, hipStream_t stream);
hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t stream);
hipError_t launch_eq7_merge(const void* oa, const float* la, void* o, const float* lb, const void* oc,
                            const float* lc, float* lse, int B, int S, int Hq, int d, int dt, bool windows,
                            hipStream_t stream);

}  // namespace prope
