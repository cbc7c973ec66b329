/*
 * prope.h - C ABI of the remapped-position RoPE attention library (gfx950).
 *
 * Causal attention with rotary position embedding applied on the fly under
 * remapped position ids:
 *   - NoPE global attention ("Periodic RoPE for Infinite Context LLMs",
 *     section 3.3, Eq. (6)): scores q.k / sqrt(d), no rotation;
 *   - RoPE attention on caller ids, optionally periodic (same page, section
 *     3.1 Eq. (1)-(3) and section 3.2 Eq. (4)-(5): rotate by p mod P) and
 *     optionally restricted to a causal sliding window; EndPrompt's
 *     two-segment ids are just an id array in this mode;
 *   - the same on a sliding window with ALiBi biases (P-RoPE page, section 1:
 *     SWA with ALiBi, a linear distance penalty clamped to the window, with a
 *     manually set slope per head);
 *   - Jet-Long bifocal attention ("Jet-Long: Efficient Long-Context Extension
 *     with Dynamic Bifocal RoPE", section 3, Eq. (1)): keys within w0 of the
 *     query score with RoPE at the true ids, farther keys with RoPE at ids
 *     floor(p / s) (section 3.1, Eq. (3)); the two parts are merged through
 *     partial softmax statistics (section 3.3, Eq. (7)); decode applies the
 *     correction rotation of section 3.2, Eq. (5)-(6) to a cache of
 *     base-rotated keys.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent),
 *     contiguous, in the layouts stated below; `params` is a HOST pointer.
 *   - The caller owns every buffer. The library allocates no device memory,
 *     keeps no state between calls and may be called from several threads.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *     and return without synchronising. Device faults surface at the
 *     caller's next synchronisation.
 *   - Arguments are validated on the host before any HIP call; a bad argument
 *     returns PROPE_ERR_INVALID_ARG (or PROPE_ERR_UNSUPPORTED for a valid
 *     but unimplemented combination) and enqueues nothing. A failed launch
 *     returns PROPE_ERR_HIP.
 *   - RoPE pairs adjacent coordinates (2i, 2i+1) and uses frequency
 *     theta_i = rope_base^(-2i/d) for pair i. Angles are formed from an exact
 *     64-bit fixed-point phase of p * theta_i / (2 pi), so ids up to 2^31 - 1
 *     keep full float32 angle accuracy.
 *   - Masks and bifocal routing use token indices (query index i, key index
 *     j); position ids only drive rotations.
 */
#ifndef PROPE_H
#define PROPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PROPE_VERSION 2

typedef enum {
  PROPE_OK = 0,
  PROPE_ERR_INVALID_ARG = -1,
  PROPE_ERR_UNSUPPORTED = -2,
  PROPE_ERR_WORKSPACE = -3,
  PROPE_ERR_HIP = -4
} prope_status;

typedef enum { PROPE_BF16 = 0, PROPE_FP32 = 1 } prope_dtype;

typedef enum {
  PROPE_NOPE = 0,    /* no rotation (P-RoPE page, Eq. (6))                          */
  PROPE_ROPE = 1,    /* rotate by ids, mod `period` if period > 0 (Eq. (4)-(5))     */
  PROPE_BIFOCAL = 2  /* Jet-Long Eq. (1): local iff i - j <= window_left, else the
                        remote view at ids floor(p / remap_scale)                   */
} prope_mode;

typedef enum {
  PROPE_REMOTE_ALIAS = 0,  /* remote ids floor(p / s) (Jet-Long Eq. (3)), integer s = G     */
  PROPE_REMOTE_INTERP = 1  /* remote angle p * theta_i / s: the frequency-interpolation
                              mapping of Jet-Long section 4.5 (Table 6), unfloored; s may
                              be any real number >= 1 (interp_scale)                      */
} prope_remote_map;

typedef struct {
  int32_t mode;          /* prope_mode                                                   */
  int32_t period;        /* P >= 0; 0 = no period. ROPE mode only (else must be 0)       */
  int32_t remap_scale;   /* s >= 1, the integer group size G of Jet-Long Eq. (2)-(3).
                            BIFOCAL only (must be 1 otherwise)                           */
  int32_t window_left;   /* NOPE/ROPE: keys with i - j > window_left are masked; -1 = no
                            window (full causal). The P-RoPE window of W keys is W - 1.
                            BIFOCAL: w0 >= -1, routing only; -1 = every key remote        */
  double rope_base;      /* Theta > 1 (e.g. 1e4, 1e6); ignored by NOPE                    */
  float softmax_scale;   /* > 0, or 0 for 1/sqrt(d)                                      */
  int32_t w_pretrained;  /* 0: the remote scale is remap_scale (or interp_scale). > 0
                            (BIFOCAL only, with remap_scale = 1 and interp_scale = 0): the
                            scale follows the sequence length L (prefill: S; decode:
                            kv_len[b], per sequence, so a batch may straddle a boundary),
                            as Jet-Long section 3.1 gives it:
                              PROPE_REMOTE_ALIAS:  the integer group size of Eq. (2),
                                                   s = G(L) = max(1, ceil(L / w_pretrained));
                              PROPE_REMOTE_INTERP: the continuous-style factor
                                                   s = max(1, L / w_pretrained)          */
  int32_t remote_map;    /* prope_remote_map; PROPE_REMOTE_INTERP is BIFOCAL only        */
  int32_t reserved;      /* must be 0                                                    */
  double interp_scale;   /* PROPE_REMOTE_INTERP only: the real scale s >= 1 (finite), with
                            remap_scale = 1 and w_pretrained = 0; 0 = use remap_scale    */
  const float* alibi_slopes; /* NULL, or a DEVICE array of Hq float32 slopes m_h (NOPE and
                            ROPE modes only): each kept key's scaled score gets
                            - m_h * (i - j) added (decode: - m_h * (kv_len - 1 - j)). With
                            window_left >= 0 the window masks every key beyond it, which
                            clamps the penalty to distances 0 .. window_left as in the
                            P-RoPE page's SWA + ALiBi layer. Read by the kernels, so it
                            must stay valid until the call's work has run.              */
} prope_params;

/*
 * Prefill: O = softmax(mask(scores)) V for every query row, all heads.
 *   q [B,S,Hq,d], k [B,S,Hkv,d], v [B,S,Hkv,d], o [B,S,Hq,d]: dtype `dt`,
 *     q and k UNROTATED (rotation is fused into the kernel's tile loads).
 *   lse [B,Hq,S] float32, natural-log log-sum-exp of each row's kept scaled
 *     scores; may be NULL.
 *   pos [B,S] int32 position ids, any value (NOPE: ignored, may be NULL). A
 *     negative id rotates backwards; the period takes p mod P in [0, P) and the
 *     remote map floor(p / s), both with mathematical (floor) semantics.
 *   Query head h reads KV head h / (Hq / Hkv); Hq % Hkv must be 0.
 *   d in {64, 128}; 1 <= S; 1 <= B; bf16 or fp32. One sequence's q slice
 *   (S * Hq * d elements) must stay under 2^30 elements (32-bit byte offsets),
 *   else PROPE_ERR_UNSUPPORTED. So must the launch grid, at most 2^32 - 1
 *   work-items: bf16 takes 512 threads per 256 (row, head) pairs, so it fits
 *   any problem that fits in memory; fp32 takes 512 threads per 8 pairs at
 *   d = 64 and per 4 at d = 128, so B * Hq * S is limited to about 2^25.
 *   Rows with no kept key (impossible: the key j = i is always kept) would
 *   get O = 0 and lse = -inf.
 */
int prope_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int dt,
                       const prope_params* params, void* stream);

/*
 * Prefill as prope_attn_prefill (same operation, arguments, checks and
 * results, bit for bit), scheduled through a work queue: one workgroup per
 * compute unit takes (row block, head group) items from eight queues, one per
 * XCD, heaviest row block first, and takes items left in the other XCDs'
 * queues when its own is empty. The XCDs of one device can run at different
 * speeds, and a fixed split of the work over them leaves the fast ones idle
 * at the end; the queue removes that tail.
 *   queue: caller-owned device buffer of prope_prefill_queue_size() bytes,
 *     128-byte aligned, all zero before its first use (e.g. a zero-filled
 *     allocation). Every call leaves it zero again, so it can be reused by the
 *     calls that follow on the same stream. Calls that may run at the same
 *     time (other streams, graph replays) need distinct buffers. NULL or
 *     misaligned -> PROPE_ERR_INVALID_ARG.
 *   fp32 (dt = PROPE_FP32) runs the static schedule and does not touch queue.
 */
size_t prope_prefill_queue_size(void);
int prope_attn_prefill_queued(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int dt,
                              const prope_params* params, void* queue, void* stream);

/*
 * Bifocal prefill composed as the pages' unfused construction (Jet-Long
 * "Efficient Long-Context Extension with Dynamic Bifocal RoPE", section 3.3,
 * Eq. (7)): three ordinary attention calls, each returning O_X and its LSE,
 *   A: window i - j <= w0 at the ids pos,
 *   B: full causal attention at the remote ids floor(pos / s),
 *   C: window i - j <= w0 at the remote ids,
 * merged per query row in fp32 as
 *   (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C), W_X = exp(l_X - max l).
 * Same result as prope_attn_prefill in BIFOCAL mode up to rounding (each call
 * rounds its O_X to dt); provided to measure the fused kernel against the
 * construction it replaces and to check Eq. (7) on the device.
 *   Arguments as prope_attn_prefill; params->mode must be PROPE_BIFOCAL and
 *   pos is required. With PROPE_REMOTE_INTERP, B and C rotate at the ids pos
 *   with the interpolated frequencies theta_i / s instead of at floor(pos / s).
 *   workspace: caller-owned device buffer, 256-byte aligned, of at least
 *     prope_bifocal_unfused_workspace_size(B, S, Hq, d, dt) bytes (O_A, O_C,
 *     three LSE vectors, remote ids, and the work queue of the three calls,
 *     as in prope_attn_prefill_queued); too small -> PROPE_ERR_WORKSPACE. Its
 *     contents need no initialisation and are scratch after the call.
 *   Enqueues six kernels on `stream` (five for fp32, which has no queue).
 *   Beyond prope_attn_prefill's limits, the merge takes one thread per 8
 *   output elements: B * S * Hq * d / 8 over 2^32 - 1 -> PROPE_ERR_UNSUPPORTED.
 *   Every check is made before the first kernel is enqueued.
 */
size_t prope_bifocal_unfused_workspace_size(int B, int S, int Hq, int d, int dt);
int prope_attn_prefill_bifocal_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                                       const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int dt,
                                       const prope_params* params, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * Decode: one new query token per sequence against a KV cache.
 *   q [B,Hq,d]: the new token's query ALREADY rotated at its own position
 *     kv_len[b]-1 (the base view, Jet-Long Eq. (6)'s q_local).
 *   k_cache, v_cache [B,Lmax,Hkv,d]: keys rotated at their own index (Jet-Long
 *     Eq. (4)); the cache is never modified.
 *   kv_len [B] int32 device array, 0 <= kv_len[b] <= Lmax, counting the new
 *     token (its key is at index kv_len[b]-1). kv_len[b] = 0 is an empty slot:
 *     its O rows are 0 and its LSE is -inf (no key to attend to). A value
 *     outside [0, Lmax] is clamped to that range, so no read leaves the cache.
 *   o [B,Hq,d] dtype `dt`; lse [B,Hq] float32, may be NULL.
 *   BIFOCAL: keys with (kv_len-1) - j <= w0 score q.k; farther keys score
 *     RoPE(q, dq).RoPE(k_j, dk_j) with dq = floor(p_q/s) - p_q and
 *     dk_j = floor(j/s) - j (Jet-Long Eq. (5)-(6)), computed in registers.
 *   With PROPE_REMOTE_INTERP the corrections are p_q * (theta_i / s - theta_i)
 *     and j * (theta_i / s - theta_i); with w_pretrained > 0, s = max(1,
 *     kv_len[b] / w_pretrained) per sequence.
 *   NOPE/ROPE: scores q.k_j (q and cache already carry the layer's rotation),
 *     keys beyond window_left masked, optional ALiBi biases. `period` must be 0.
 *   workspace: caller-owned device buffer of at least
 *     prope_decode_workspace_size(B, Lmax, Hq, d) bytes (split-K partials);
 *     too small -> PROPE_ERR_WORKSPACE. bf16 only; Hq / Hkv <= 16, B and
 *     Hkv <= 65535 (launch grid limits) and one sequence's cache slice
 *     (Lmax * Hkv * d * 2 bytes) under 4 GiB, else PROPE_ERR_UNSUPPORTED.
 */
size_t prope_decode_workspace_size(int B, int Lmax, int Hq, int d);
int prope_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int32_t* kv_len, int B, int Lmax, int Hq, int Hkv, int d, int dt,
                      const prope_params* params, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Decode as prope_attn_decode (same arguments, checks and results, bit for bit)
 * for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The split-K partials go
 * to a fixed device array inside the library instead of a caller workspace:
 * PROPE_DECODE_SCRATCH_BYTES per device, held from when the library's code is
 * loaded on the device until the process ends. The array's device address is
 * looked up on the first call on each device (a HIP call, no allocation).
 *   A call fits when its partials, B * Hq * chunks * (d + 2) * 4 bytes for the
 *   launch's chunk choice, fit the array; any call with
 *   prope_decode_workspace_size(B, Lmax, Hq, d) <= PROPE_DECODE_SCRATCH_BYTES
 *   does (the 128K-key batch-8 decode with 32 query heads needs 8.5 MB).
 *   Otherwise PROPE_ERR_WORKSPACE, before any HIP call.
 *   Every call on a device shares its one array, which keeps the last call's
 *   contents (none of it needs to start at zero): calls that may overlap on
 *   one device (other streams, concurrent graph replays) race and must be
 *   ordered by the caller.
 */
#define PROPE_DECODE_SCRATCH_BYTES (16u << 20)
int prope_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                              const int32_t* kv_len, int B, int Lmax, int Hq, int Hkv, int d, int dt,
                              const prope_params* params, void* stream);

/*
 * y = R_pos x per token and head (P-RoPE page, Eq. (2)): x, y [B,S,H,d] of
 * dtype `dt`, pos [B,S] int32 (any sign: a negative id rotates backwards, which
 * applies Jet-Long's Eq. (6) corrections). y may alias x exactly. d even,
 * 2 <= d <= 256. Builds the base-rotated cache of Jet-Long Eq. (4).
 */
int prope_rope_apply(const void* x, void* y, const int32_t* pos, int B, int S, int H, int d,
                     int dt, double rope_base, void* stream);

/* Jet-Long Eq. (2): G = max(1, ceil(L / w_pretrained)); returns -1 on bad input. */
int prope_group_size(int64_t L, int64_t w_pretrained);

/* Static string for a status code (never NULL). */
const char* prope_status_string(int status);

int prope_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PROPE_H */
