// Flash-style causal attention prefill with RoPE fused into the tile loads,
// bf16 operands, fp32 accumulation, gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Scores per mode (token indices i, j; ids p):
//   NOPE     q_i . k_j                                  (P-RoPE page, Eq. (6))
//   ROPE     (R_r q_i) . (R_r k_j), r = p mod P or p    (P-RoPE page, Eq. (3)-(5))
//   BIFOCAL  local  (i - j <= w0): RoPE at p
//            remote (i - j >  w0): RoPE at floor(p / s) (Jet-Long page, Eq. (1), (3)),
//            or with interpolated frequencies theta_i / s at p (same page,
//            section 4.5): the remote pass reads ids floor(p / div) with the
//            frequency table fr, div = s or 1
// scaled by softmax_scale; causal, plus the window for NOPE/ROPE.
//
// Work decomposition. A workgroup (8 wavefronts, two per SIMD) owns 256 query
// rows: HG query heads of one KV group times BMp = 256/HG consecutive
// positions. Each wave owns 32 rows = 32 positions of one head. All query
// heads that read the same KV head sit in one workgroup when possible (HG = 4,
// 2 or 1), so each K tile rotated into LDS is shared by all of them. Such a
// set of rows is one work item: a launch either runs one item per workgroup,
// or (with a work queue) a persistent workgroup per compute unit takes items
// from per-XCD queues until they are empty.
//
// Bifocal merge. The workgroup walks the remote keys first (queries and keys
// rotated at floor(p/s)), then the local window (rotated at p), carrying one
// set of softmax statistics (row max m, row sum l, unnormalised O) across both
// passes. That is the partial-statistics merge of Jet-Long section 3.3,
// Eq. (7), done in registers, with each key routed to exactly one side, so
// call C of Eq. (7) (which only cancels B's local part) is never computed.
// Tiles whose distance range misses a pass are skipped; tiles straddling a
// pass boundary (i - j = w0) are masked per element.
//
// MFMA layout (32x32x16, bf16): S^T = K Q^T, so a lane's output column is a
// query row: lane l holds row m = l % 32 and keys n = 8*(r/4) + 4*(l/32) + r%4
// of accumulator register r. The same register order serves directly as the
// B operand of O^T += V^T P^T. V stays row-major in LDS; its transposed A
// operand comes from ds_read_b64_tr_b16.
//
// Schedule (two wave groups in antiphase). Waves 0-3 (group 0) and 4-7
// (group 1) put one wave of each group on every SIMD. Every wave alternates a
// matrix phase (O += P V for tile t, then S = K Q^T for tile t+1: 32 MFMAs,
// with its share of the K/V LDS stores between them) and a vector phase (mask,
// online softmax and P packing for tile t+1, interleaved with the RoPE of the
// K rows it stores next). Group 1 runs one phase behind group 0, and a
// workgroup barrier separates phases, so on each SIMD one wave's MFMAs overlap
// the other wave's vector work. K and V tiles are double-buffered in LDS; each
// group stages half of every tile's rows, with the global loads issued one
// phase pair ahead.
#include <limits.h>

#include "internal.hpp"

namespace prope {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 512;  // 8 wavefronts, 2 per SIMD
constexpr int kGroupThreads = kThreads / 2;

__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Buffer resource over one batch element of a tensor: loads past `bytes`
// return zero, which pads ragged tiles without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ int bload_i32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// The same with a wave-uniform part of the offset in the instruction's scalar
// offset field: per-lane offsets stay loop-invariant, so the main loop forms
// no vector addresses.
__device__ __forceinline__ u32x4_t bload16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ int bload_i32s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Workgroup barrier that orders LDS accesses only. Unlike __syncthreads() it
// does not wait for outstanding global loads, so prefetches stay in flight
// across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group,
// lane j names row j/4 and columns 4*(j%4) .. +3 of a 4 x 16 block of 16-bit
// values; lane i receives column i of the block, rows 0..3 in order.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// Sum of the two bf16 halves of a packed word, added to c (v_dot2c_f32_bf16).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float c) {
  const bf16x2_t one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, c, false);
}

template <int MODE>
__device__ __forceinline__ int rot_index(int p, int rot, const PrefillArgs& a) {
  if (rot == 2) return static_cast<int>(fastdiv(static_cast<uint32_t>(p), a.scale_div));
  if (MODE == kRope) return a.period > 0 ? static_cast<int>(fastmod(static_cast<uint32_t>(p), a.period_div)) : p;
  return p;
}

// Rotate the 4 pairs of a 16-byte bf16 chunk by id r (pairs pair0 .. pair0+3).
__device__ __forceinline__ u32x4_t rotate_chunk(u32x4_t x, int r, const uint32_t* flo,
                                                const uint32_t* fhi) {
  u32x4_t y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float s, c;
    rope_sincos(r, flo[e], fhi[e], s, c);
    float y0, y1;
    rot_pair(bf16_lo(x[e]), bf16_hi(x[e]), c, s, y0, y1);
    y[e] = pack_bf16(y0, y1);
  }
  return y;
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(const PrefillArgs a) {
  constexpr int KS = D / 16;                  // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;                  // 32-row blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int HR = kBN / 2;                 // tile rows staged by one group
  constexpr int RPS = kGroupThreads / CPR;    // rows covered by one staging sweep of a group
  constexpr int NU = HR / RPS;                // K (and V) chunks per thread per tile
  constexpr int KRow = D + 8;                 // K tile row stride: 16-byte reads of 8 rows hit distinct banks
  constexpr int VRow = D + 32;                // V tile row stride: the 4 rows of a transposing read hit distinct banks
  static_assert(NU >= 1 && NU <= 2 && NU * RPS == HR, "staging layout");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * KRow];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBN * VRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
  const int lr = lane & 31, lg = lane >> 5;
  const int group = wave >> 2;  // waves w and w + 4 share a SIMD

  // ---- work items ---------------------------------------------------------
  // An item is (sequence, KV head, head subgroup, row block). Without a queue
  // every workgroup runs the one item blockIdx names. With a queue the grid is
  // persistent and items come from 8 queues, one per XCD (blockIdx % 8 is the
  // XCD a workgroup runs on): queue x holds the x-th contiguous eighth of the
  // items (whole head groups when possible, so its K/V tiles stay in that XCD's
  // L2), handed out heaviest row block first. A workgroup whose own queue is
  // empty takes items from the others. The XCDs run at different speeds, so a
  // fixed split of the items over them leaves the fast ones idle at the end.
  const int n_items = a.B * a.Hkv * a.n_hsub * a.n_pblocks;
  const int q8 = n_items / 8, r8 = n_items % 8;
  auto q_start = [&](int x) { return x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8; };
  auto q_len = [&](int x) { return q8 + (x < r8 ? 1 : 0); };
  // item of the k-th claim on queue x: a queue made of whole head groups goes
  // row block major across its groups, heaviest (last) row block first
  auto q_item = [&](int x, int k) {
    const int st = q_start(x), len = q_len(x), npb = a.n_pblocks;
    if (st % npb == 0 && len % npb == 0) {
      const int ng = len / npb;
      return st + (k % ng) * npb + k / ng;
    }
    return st + k;
  };
  const int home = blockIdx.x & 7;
  // each queue's first claims are static (rank blockIdx / 8 among the
  // workgroups of that XCD); its counter counts the claims after those
  auto q_static = [&](int x) { return int(gridDim.x) / 8 + (x < int(gridDim.x) % 8 ? 1 : 0); };
  uint32_t* const wq = a.queue;
  bool first = true;
  auto next_item = [&]() -> int {  // run by wave 0; the result is valid in every lane
    if (first) {
      first = false;
      if (!wq) return xcd_remap(blockIdx.x, gridDim.x);
      const int k0 = int(blockIdx.x) / 8;
      if (k0 < q_len(home)) return q_item(home, k0);
    }
    if (!wq) return -1;
    int r = -1;
    if (lane == 0) {
      const uint32_t k = atomicAdd(&wq[kQueueLine * home], 1u) + q_static(home);
      if (k < uint32_t(q_len(home))) r = q_item(home, int(k));
    }
    r = __shfl(r, 0);
    if (r >= 0) return r;
    // own queue empty: read the other queues' counters in one round, then claim
    // from those that still hold items
    const int x = (home + lane) & 7;
    bool has = false;
    if (lane >= 1 && lane < 8)
      has = __hip_atomic_load(&wq[kQueueLine * x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + q_static(x) <
            uint32_t(q_len(x));
    uint64_t m = __ballot(has);
    while (m) {
      const int xs = (home + __builtin_ctzll(m)) & 7;
      m &= m - 1;
      if (lane == 0) {
        const uint32_t k = atomicAdd(&wq[kQueueLine * xs], 1u) + q_static(xs);
        if (k < uint32_t(q_len(xs))) r = q_item(xs, int(k));
      }
      r = __shfl(r, 0);
      if (r >= 0) return r;
    }
    return -1;
  };
  __shared__ int s_item;
#pragma clang loop unroll(disable)
  for (;;) {
  if (wave == 0) {
    const int r = next_item();
    if (lane == 0) s_item = r;
  }
  __syncthreads();
  int item = s_item;
  if (item < 0) break;
  const int pb = a.n_pblocks - 1 - (item % a.n_pblocks);  // heavy (late) rows first
  item /= a.n_pblocks;
  const int hsub = item % a.n_hsub;
  item /= a.n_hsub;
  const int kvh = item % a.Hkv;
  const int b = item / a.Hkv;

  const int S = a.S;
  const int P0 = pb * a.BMp;
  const int P1 = min(S, P0 + a.BMp) - 1;
  const int hl = (wave * 32) / a.BMp;
  const int i0 = P0 + wave * 32 - hl * a.BMp;  // first position of this wave
  const int i1 = min(i0 + 31, S - 1);         // last valid position (i1 < i0: none)
  const int h = kvh * a.G + hsub * a.HG + hl;

  // byte strides and per-batch buffer resources (loads past the end read 0)
  const uint32_t rowq_b = uint32_t(a.Hq) * D * 2, rowk_b = uint32_t(a.Hkv) * D * 2;
  const __amdgpu_buffer_rsrc_t qres = make_rsrc(static_cast<const uint16_t*>(a.q) + size_t(b) * S * a.Hq * D, uint32_t(S) * rowq_b);
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(static_cast<const uint16_t*>(a.k) + size_t(b) * S * a.Hkv * D, uint32_t(S) * rowk_b);
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(static_cast<const uint16_t*>(a.v) + size_t(b) * S * a.Hkv * D, uint32_t(S) * rowk_b);
  const __amdgpu_buffer_rsrc_t pres = make_rsrc(MODE == kNope ? a.q : static_cast<const void*>(a.pos + size_t(b) * S),
                                                MODE == kNope ? 0u : uint32_t(S) * 4);

  // ---- passes and tile ranges ---------------------------------------------
  // pass 0 (remote keys in BIFOCAL, the only pass otherwise) and pass 1 (the
  // local window), as plain scalars: keep a key iff dlo <= i - j <= dhi; rot is
  // 0 (none), 1 (base ids, mod period if any) or 2 (remote ids floor(p/s))
  int dlo0, dhi0, rot0, dlo1 = 0, dhi1 = -1, rot1 = 0, npass;
  if (MODE == kBifocal) {
    const int w0 = a.window_left;
    dlo0 = w0 + 1; dhi0 = INT_MAX; rot0 = 2;
    dlo1 = 0; dhi1 = w0; rot1 = 1;
    npass = w0 >= 0 ? 2 : 1;
  } else {
    dlo0 = 0; dhi0 = a.window_left < 0 ? INT_MAX : a.window_left; rot0 = MODE == kNope ? 0 : 1;
    npass = 1;
  }
  auto tile_range = [&](int dlo, int dhi, int& tb, int& tc) {
    const int64_t jlo = max<int64_t>(0, int64_t(P0) - dhi);
    const int64_t jhi = min<int64_t>(S - 1, int64_t(P1) - dlo);
    tb = 0;
    tc = 0;
    if (jhi >= jlo) {
      tb = static_cast<int>(jlo / kBN);
      tc = static_cast<int>(jhi / kBN) - tb + 1;
    }
  };
  int tb0, tc0, tb1 = 0, tc1 = 0;
  tile_range(dlo0, dhi0, tb0, tc0);
  if (npass > 1) tile_range(dlo1, dhi1, tb1, tc1);
  const int T = tc0 + tc1;

  auto tile_of = [&](int t, int& p, int& kt) {
    p = t < tc0 ? 0 : 1;
    kt = p ? tb1 + (t - tc0) : tb0 + t;
  };

  // ---- per-thread staging coordinates --------------------------------------
  // group g stages rows [HR*g, HR*g + HR) of every K and V tile
  const int gtid = tid & (kGroupThreads - 1);
  const int sc = gtid % CPR;                 // 16-byte column chunk this thread stages
  const int sr = group * HR + gtid / CPR;    // first row this thread stages (then sr + RPS)
  const uint32_t kcol_b = uint32_t(kvh) * D * 2 + sc * 16;
  const uint32_t srow_kv = uint32_t(sr) * rowk_b + kcol_b;  // this thread's first staged row, byte offset in K/V
  const uint32_t srow_id = uint32_t(sr) * 4;                // and in the ids

  // Per-chunk constants kept in LDS rather than registers: the 4 pair
  // frequencies of each 16-byte column chunk, and for each rotation kind the
  // cos/sin of the affine id step between the two K rows a thread stages. The
  // second K row a thread stages is RPS keys after the first; when their
  // rotation ids differ by that step (RPS for base ids, RPS / s for remote ids
  // when s divides RPS) its cos/sin are the first row's times the step's.
  __shared__ uint2 kfreq[2][CPR * 4];  // [0]: base frequencies, [1]: remote frequencies
  __shared__ float2 kstep[2][CPR * 4];
  const int id_step1 = NU > 1 ? RPS : -1;
  const int sdiv = static_cast<int>(a.scale_div.div);
  const int id_step2 = (NU > 1 && RPS % sdiv == 0) ? RPS / sdiv : -1;
  if (MODE != kNope && tid < CPR * 4) {
    const uint32_t flo = a.f.lo[tid], fhi = a.f.hi[tid];
    const uint32_t rlo = a.fr.lo[tid], rhi = a.fr.hi[tid];
    kfreq[0][tid] = make_uint2(flo, fhi);
    kfreq[1][tid] = make_uint2(rlo, rhi);
    float s1 = 0.f, c1 = 1.f, s2 = 0.f, c2 = 1.f;
    if (id_step1 >= 0) rope_sincos(id_step1, flo, fhi, s1, c1);
    if (id_step2 >= 0) rope_sincos(id_step2, rlo, rhi, s2, c2);
    kstep[0][tid] = make_float2(c1, s1);
    kstep[1][tid] = make_float2(c2, s2);
  }
  __syncthreads();

  u32x4_t kraw[NU], vraw[NU];
  int kid[NU];

  // global -> registers: this thread's K rows of tile tk and V rows of tile tv
  // (a tile index outside [0, T) is skipped)
  auto stage_load = [&](int tk, int tv) __attribute__((always_inline)) {
    if (tk >= 0 && tk < T) {
      int p, kt;
      tile_of(tk, p, kt);
      const int rot = p ? rot1 : rot0;
      const uint32_t j0 = uint32_t(kt) * kBN;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t j = j0 + sr + RPS * u;
        kraw[u] = bload16(kres, j * rowk_b + kcol_b);
        kid[u] = (MODE != kNope && rot) ? bload_i32(pres, j * 4) : 0;
      }
    }
    if (tv >= 0 && tv < T) {
      int p, kt;
      tile_of(tv, p, kt);
      const uint32_t j0 = uint32_t(kt) * kBN;
#pragma unroll
      for (int u = 0; u < NU; ++u) vraw[u] = bload16(vres, (j0 + sr + RPS * u) * rowk_b + kcol_b);
    }
  };

  // registers -> LDS: K of tile tk (rotated for its pass) and V of tile tv
  auto stage_store = [&](int tk, int tv) __attribute__((always_inline)) {
    if (tk >= 0 && tk < T) {
      int p, kt;
      tile_of(tk, p, kt);
      uint16_t* dst = Ks[tk & 1];
      const int rot = p ? rot1 : rot0;
      if (MODE != kNope && rot) {
        const int id_step = rot == 2 ? id_step2 : id_step1;
        uint32_t kflo[4], kfhi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint2 f = kfreq[rot - 1][sc * 4 + e];
          kflo[e] = f.x;
          kfhi[e] = f.y;
        }
        float cs[4], sn[4];
        const int r0 = rot_index<MODE>(kid[0], rot, a);
#pragma unroll
        for (int e = 0; e < 4; ++e) rope_sincos(r0, kflo[e], kfhi[e], sn[e], cs[e]);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          if (u > 0) {
            const int ru = rot_index<MODE>(kid[u], rot, a);
            if (id_step >= 0 && ru - r0 == id_step * u) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {  // (cs + i sn) * (step cos + i step sin)
                const float2 es = kstep[rot - 1][sc * 4 + e];
                const float c2 = cs[e] * es.x - sn[e] * es.y;
                const float s2 = sn[e] * es.x + cs[e] * es.y;
                cs[e] = c2;
                sn[e] = s2;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) rope_sincos(ru, kflo[e], kfhi[e], sn[e], cs[e]);
            }
          }
          u32x4_t y;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y0, y1;
            rot_pair(bf16_lo(kraw[u][e]), bf16_hi(kraw[u][e]), cs[e], sn[e], y0, y1);
            y[e] = pack_bf16(y0, y1);
          }
          *reinterpret_cast<u32x4_t*>(&dst[(sr + RPS * u) * KRow + sc * 8]) = y;
        }
      } else {
#pragma unroll
        for (int u = 0; u < NU; ++u) *reinterpret_cast<u32x4_t*>(&dst[(sr + RPS * u) * KRow + sc * 8]) = kraw[u];
      }
    }
    if (tv >= 0 && tv < T) {
      uint16_t* dst = Vs[tv & 1];
#pragma unroll
      for (int u = 0; u < NU; ++u) *reinterpret_cast<u32x4_t*>(&dst[(sr + RPS * u) * VRow + sc * 8]) = vraw[u];
    }
  };

  // Branch-free staging for the main loop (loads here, the rotation in the
  // vector phase, the LDS stores between the MFMAs of the matrix phase). Tile
  // indices past the last tile are harmless there: their loads stay inside the
  // sequence's buffer resources, and the K/V buffers they overwrite are not read
  // again. Row 1's cos/sin always come from the affine step; lanes whose ids
  // break it are redone exactly by fix_row1 after the matrix phase.
  bool need_fix = false;
  // this thread's frequencies and row steps for the rotation kind of the K
  // tiles being staged, in registers (reloaded when that kind changes)
  uint2 kf_reg[4];
  float2 ks_reg[4];
  int kreg_rot = -1;
  auto load_kregs = [&](int rot) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf_reg[e] = kfreq[rot - 1][sc * 4 + e];
      ks_reg[e] = kstep[rot - 1][sc * 4 + e];
    }
    kreg_rot = rot;
  };
  auto stage_load_nb = [&](int tk, int tv) __attribute__((always_inline)) {
    int p, kt;
    tile_of(tk, p, kt);
    const uint32_t j0 = uint32_t(kt) * kBN;  // wave-uniform
    // issue order = use order (ids, K rows, V rows), so each use waits only for
    // its own loads
    if (MODE != kNope) {
#pragma unroll
      for (int u = 0; u < NU; ++u) kid[u] = bload_i32s(pres, srow_id + RPS * 4 * u, j0 * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) kraw[u] = bload16s(kres, srow_kv + RPS * rowk_b * u, j0 * rowk_b);
    __builtin_amdgcn_sched_barrier(0);
    int pv, ktv;
    tile_of(tv, pv, ktv);
    const uint32_t jv = uint32_t(ktv) * kBN;
#pragma unroll
    for (int u = 0; u < NU; ++u) vraw[u] = bload16s(vres, srow_kv + RPS * rowk_b * u, jv * rowk_b);
  };
  auto fix_row1 = [&](int tk) __attribute__((always_inline)) {
    if (MODE != kNope && NU > 1 && need_fix) {
      int p, kt;
      tile_of(tk, p, kt);
      const int rot = p ? rot1 : rot0;
      const int ru = rot_index<MODE>(kid[NU - 1], rot, a);
      u32x4_t y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 f = kfreq[rot - 1][sc * 4 + e];
        float sn, cs, y0, y1;
        rope_sincos(ru, f.x, f.y, sn, cs);
        rot_pair(bf16_lo(kraw[NU - 1][e]), bf16_hi(kraw[NU - 1][e]), cs, sn, y0, y1);
        y[e] = pack_bf16(y0, y1);
      }
      *reinterpret_cast<u32x4_t*>(&Ks[tk & 1][(sr + RPS * (NU - 1)) * KRow + sc * 8]) = y;
    }
  };

  // ---- query operand (B of S^T = K Q^T): lane holds row lr, dims ks*16 + lg*8 .. +7
  u32x4_t qreg[KS];
  auto load_q = [&](int p) __attribute__((always_inline)) {
    const int rot = p ? rot1 : rot0;
    const uint32_t i = uint32_t(i0 + lr);
    const uint32_t qoff = i * rowq_b + uint32_t(h) * D * 2 + lg * 16;
    const int r = (MODE != kNope && rot) ? rot_index<MODE>(bload_i32(pres, i * 4), rot, a) : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = bload16(qres, qoff + ks * 32);  // rows past the sequence read 0
      if (MODE != kNope && rot) {
        uint32_t flo[4], fhi[4];
        const RopeFreq& fq = rot == 2 ? a.fr : a.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          flo[e] = fq.lo[ks * 8 + lg * 4 + e];
          fhi[e] = fq.hi[ks * 8 + lg * 4 + e];
        }
        x = rotate_chunk(x, r, flo, fhi);
      }
      qreg[ks] = x;
    }
  };

  // ---- per-lane LDS addresses of the PV operand (transposing reads of V) ---
  // A operand of O^T += V^T P^T for d-block db and 16-key step kk: lane (lr, lg)
  // needs V[16kk + 4lg + e][32db + lr] for e = 0..3 and V[16kk + 8 + 4lg + e][..].
  const int j15 = lane & 15;
  const int vrow0 = 4 * lg + (j15 >> 2);
  const int vcol0 = 16 * (lr >> 4) + 4 * (j15 & 3);

  // ---- running statistics ---------------------------------------------------
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  f32x16_t sacc[2];    // S^T of the tile in flight (two 32-key blocks)
  u32x4_t pop[4];      // its P, bf16, as four 16-key B operands
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pop[kk] = u32x4_t{0, 0, 0, 0};
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.f;        // this lane's share of the running sum
  const float sl2 = a.scale_log2;

  // does tile t hold any kept (row, key) pair of this wave?
  auto wave_live = [&](int t, bool& need_mask, int& dlo, int& dhi, int& j0) __attribute__((always_inline)) {
    int p, kt;
    tile_of(t, p, kt);
    dlo = p ? dlo1 : dlo0;
    dhi = p ? dhi1 : dhi0;
    j0 = kt * kBN;
    const int dmin = i0 - (j0 + kBN - 1), dmax = i1 - j0;
    need_mask = dmin < dlo || dmax > dhi;
    return i1 >= i0 && dmax >= dlo && dmin <= dhi;
  };
  auto live = [&](int t) __attribute__((always_inline)) {
    bool nm;
    int dlo, dhi, j0;
    return wave_live(t, nm, dlo, dhi, j0);
  };
  auto pass_of = [&](int t) __attribute__((always_inline)) { return t < tc0 ? 0 : 1; };

  auto xhalf_max = [&](float x) __attribute__((always_inline)) {
    // max with the lane 32 apart (same query row, other half of the keys)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };

  // S^T = K Q^T for tile t (prologue only; the main loop uses the matrix phase below)
  auto qk_step = [&](int t) __attribute__((always_inline)) {
    const uint16_t* kbase = &Ks[t & 1][lr * KRow + lg * 8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[nb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const u32x4_t kop = *reinterpret_cast<const u32x4_t*>(kbase + nb * 32 * KRow + ks * 16);
        sacc[nb] = mfma32x32x16(kop, qreg[ks], sacc[nb]);
      }
    }
  };
  auto qk_or_clear = [&](int t) __attribute__((always_inline)) {
    if (t < T && live(t)) {
      qk_step(t);
    } else {  // nothing to score: keeps sacc from living across the whole loop
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[nb][r] = 0.f;
    }
  };

  // RoPE of the K rows a thread stages for tile t + 2, done during the vector
  // phase of tile t: the rotation index, the exact phase (quarter-rate integer
  // multiplies), sin/cos and the pair rotations are independent of the softmax,
  // so they fill its dependency gaps, and the matrix phase is left with the
  // LDS stores. The raw rows were loaded at the end of the previous matrix
  // phase.
  u32x4_t krot[NU];
  auto rotate_k = [&](int t) __attribute__((always_inline)) {
    if (MODE == kNope) return;
    int pk, kt;
    tile_of(t + 2, pk, kt);
    const int rot = pk ? rot1 : rot0;
    const int id_step = rot == 2 ? id_step2 : id_step1;
    const int r0 = rot_index<MODE>(kid[0], rot, a);
    if (NU > 1) need_fix = !(id_step >= 0 && rot_index<MODE>(kid[NU - 1], rot, a) - r0 == id_step);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sn, cs, y0, y1;
      phase_sincos(phase_top_u(static_cast<uint32_t>(r0), kf_reg[e].x, kf_reg[e].y), sn, cs);
      rot_pair(bf16_lo(kraw[0][e]), bf16_hi(kraw[0][e]), cs, sn, y0, y1);
      krot[0][e] = pack_bf16(y0, y1);
      if (NU > 1) {  // the second row: one id step further, (cs + i sn) * (step cos + i step sin)
        const float2 es = ks_reg[e];
        const float c2 = cs * es.x - sn * es.y, s2 = sn * es.x + cs * es.y;
        rot_pair(bf16_lo(kraw[NU - 1][e]), bf16_hi(kraw[NU - 1][e]), c2, s2, y0, y1);
        krot[NU - 1][e] = pack_bf16(y0, y1);
      }
    }
  };
  // Matrix phase of iteration t: PV(t) (16 MFMAs), then QK(t+1) (16 MFMAs),
  // with the LDS stores of this thread's rows of K tile t+2 and V tile t+1 one
  // per MFMA slot, scheduling barriers keeping that order. Operand reads run
  // one PV step / three QK steps ahead of their MFMAs.
  // NoPE: the V operands of the first two PV steps (keys 0-31, which this
  // wave's group staged itself) are read at the start of the vector phase,
  // which has no rotation work to hide and leaves this wave's LDS port idle
  // (one wave reads only about a quarter of the CU's LDS rate, so the matrix
  // phase is bound by its own operand reads). The rotating modes measured
  // slower with it: their vector phase is already full.
  constexpr bool kVpre = MODE == kNope;
  u32x4_t vpre[kVpre ? 2 : 1][DB];
  auto read_vpre = [&](int t) __attribute__((always_inline)) {
    const uint16_t* vbase = &Vs[t & 1][vrow0 * VRow + vcol0];
#pragma unroll
    for (int kk = 0; kk < (kVpre ? 2 : 0); ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2_t va = lds_read_tr16(vbase + kk * 16 * VRow + db * 32);
        const u32x2_t vb = lds_read_tr16(vbase + kk * 16 * VRow + 8 * VRow + db * 32);
        vpre[kk][db] = u32x4_t{va[0], va[1], vb[0], vb[1]};
      }
  };
  auto mphase = [&](int t) __attribute__((always_inline)) {
    const int tk = t + 2, tv = t + 1;
    uint16_t* kdst = &Ks[tk & 1][sr * KRow + sc * 8];
    uint16_t* vdst = &Vs[tv & 1][sr * VRow + sc * 8];
    // staging stores, one per MFMA slot: K rows (rotated in the vector phase,
    // or raw for NoPE), then V rows
    auto piece = [&](int i) __attribute__((always_inline)) {
      if (i < NU)
        *reinterpret_cast<u32x4_t*>(kdst + RPS * i * KRow) = MODE == kNope ? kraw[i] : krot[i];
      else if (i < 2 * NU)
        *reinterpret_cast<u32x4_t*>(vdst + RPS * (i - NU) * VRow) = vraw[i - NU];
    };
    const uint16_t* vbase = &Vs[t & 1][vrow0 * VRow + vcol0];
    const uint16_t* kbase = &Ks[(t + 1) & 1][lr * KRow + lg * 8];
    u32x4_t vop[2][DB];
    auto read_v = [&](int kk, u32x4_t* dst) __attribute__((always_inline)) {
      const uint16_t* vrow = vbase + kk * 16 * VRow;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2_t va = lds_read_tr16(vrow + db * 32);
        const u32x2_t vb = lds_read_tr16(vrow + 8 * VRow + db * 32);
        dst[db] = u32x4_t{va[0], va[1], vb[0], vb[1]};
      }
    };
    constexpr int KA = 3;  // K steps read ahead
    u32x4_t kop[KA + 1][2];
    auto read_k = [&](int ks, u32x4_t* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) dst[nb] = *reinterpret_cast<const u32x4_t*>(kbase + nb * 32 * KRow + ks * 16);
    };
    int pc = 0;  // next staging piece
    read_v(kVpre ? 2 : 0, vop[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kVpre ? kk == 1 : kk + 1 < 4) {
        read_v(kVpre ? 3 : kk + 1, vop[kVpre ? 1 : (kk + 1) & 1]);
      } else if (kk == 3) {
#pragma unroll
        for (int ks = 0; ks < KA; ++ks) read_k(ks, kop[ks]);
      }
      const u32x4_t* vk = (kVpre && kk < 2) ? vpre[kVpre ? kk : 0] : vop[kk & 1];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        oacc[db] = mfma32x32x16(vk[db], pop[kk], oacc[db]);
        piece(pc++);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + KA < KS) read_k(ks + KA, kop[(ks + KA) % (KA + 1)]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        sacc[nb] = mfma32x32x16(kop[ks % (KA + 1)][nb], qreg[ks], ks == 0 ? f32x16_t{} : sacc[nb]);
        piece(pc++);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (; pc < 2 * NU; ++pc) piece(pc);  // whatever is left
  };

  // vector phase of tile t: mask, online softmax, P -> bf16, lazy O rescale
  auto softmax_step = [&](int t) __attribute__((always_inline)) {
    bool need_mask;
    int dlo, dhi, j0;
    if (!wave_live(t, need_mask, dlo, dhi, j0)) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pop[kk] = u32x4_t{0, 0, 0, 0};
      rotate_k(t);
      return false;
    }
    if (need_mask) {
      const int dbase = (i0 + lr) - (j0 + 4 * lg);  // i - j of register 0 of block 0
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dist = dbase - (nb * 32 + 8 * (r >> 2) + (r & 3));
          if (dist < dlo || dist > dhi) sacc[nb][r] = -INFINITY;
        }
    }
    float mx0 = fmaxf(sacc[0][0], sacc[0][1]), mx1 = fmaxf(sacc[1][0], sacc[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      mx0 = fmaxf(mx0, fmaxf(sacc[0][r], sacc[0][r + 1]));
      mx1 = fmaxf(mx1, fmaxf(sacc[1][r], sacc[1][r + 1]));
    }
    const float mx = xhalf_max(fmaxf(mx0, mx1)) * sl2;
    rotate_k(t);
    // The reference max moves only when the tile's max exceeds it by more than
    // 8 (log2 units): P <= 2^8 stays exact in bf16 and fp32, and O and l are
    // rescaled far less often. The final O / l and LSE = m + log2 l are unchanged.
    const float mnew = mx > m_run + 8.f ? mx : m_run;
    const bool grow = mnew > m_run;
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mref);
    m_run = mnew;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int nb = kk >> 1, r0 = (kk & 1) * 8;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r0 + e], sl2, -mref));
      const u32x4_t w = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                         pack_bf16(pv[6], pv[7])};
      pop[kk] = w;
      // the row sum takes the same bf16 P the PV product uses
      rs0 = add_bf16_pair(w[0], rs0);
      rs1 = add_bf16_pair(w[1], rs1);
      rs0 = add_bf16_pair(w[2], rs0);
      rs1 = add_bf16_pair(w[3], rs1);
    }
    l_run = l_run * alpha + (rs0 + rs1);
    if (__any(grow)) {  // rescale O only when some row of the wave raised its max
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    return true;
  };

  // ---- prologue: K tile 0 in LDS; K tile 1 and V tile 0 in registers --------
  stage_load(0, -1);
  stage_store(0, -1);
  stage_load(1, 0);
  load_q(pass_of(0));
  lds_barrier();

  // ---- phases -----------------------------------------------------------------
  // Group 0: QK(0) | soft(0) | PV(0) QK(1) | soft(1) | PV(1) QK(2) | ... | PV(T-1) | -
  // Group 1:  -    | QK(0)   | soft(0)     | PV(0) QK(1) | ...         | PV(T-1)
  // with a workgroup barrier after every phase. The vector phase of tile t
  // also rotates this wave's rows of K tile t+2; the matrix phase after it
  // stores them and its rows of V tile t+1 to LDS between its MFMAs, then
  // issues the loads of K tile t+3 and V tile t+2.
  if (group == 1) lds_barrier();
  qk_or_clear(0);
  stage_store(1, 0);
  stage_load_nb(2, 1);  // same issue order as in the loop, so the loads keep exact wait counts
  lds_barrier();
#pragma clang loop unroll(disable)
  for (int t = 0; t < T; ++t) {
    if (MODE != kNope) {
      const int srot = pass_of(t + 2) ? rot1 : rot0;
      if (srot != kreg_rot) load_kregs(srot);
    }
    if (kVpre) read_vpre(t);
    softmax_step(t);  // P of a tile with no kept key is zero
    if (MODE == kBifocal && t + 1 < T && pass_of(t + 1) != pass_of(t)) load_q(pass_of(t + 1));
    lds_barrier();
    // one region: PV(t), QK(t+1) (the scores of tile T, if any, are never used)
    // and the LDS stores of K tile t+2 / V tile t+1 between the MFMAs. It runs
    // at raised wave priority: the SIMD's arbiter gives the MFMA stream its
    // issue slots first and the other wave's vector work fills the gaps.
    __builtin_amdgcn_s_setprio(1);
    mphase(t);
    fix_row1(t + 2);
    stage_load_nb(t + 3, t + 2);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
  }
  if (group == 0) lds_barrier();

  // ---- finalize ---------------------------------------------------------------
  uint16_t* og = static_cast<uint16_t*>(a.o) + size_t(b) * S * a.Hq * D + size_t(h) * D;
  const size_t rowq = size_t(a.Hq) * D;
  const float l = l_run + __shfl_xor(l_run, 32);
  const int i = i0 + lr;
  if (i <= i1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * lg;
        u32x2_t w;
        w[0] = pack_bf16(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
        w[1] = pack_bf16(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(og + size_t(i) * rowq + d) = w;
      }
    if (a.lse && lg == 0) {
      const float lse = l > 0.f ? (m_run + log2f(l)) * 0.6931471805599453f : -INFINITY;
      a.lse[(size_t(b) * a.Hq + h) * S + i] = lse;
    }
  }
  __syncthreads();  // LDS and s_item are reused by the next item
  }  // items

  // Queue clean-up: each workgroup counts itself done on its XCD's counter, the
  // last of each XCD on the global one, and the very last puts every counter
  // back to 0, so the buffer is ready for the next launch.
  if (wq && wave == 0) {
    uint32_t last = 0;
    if (lane == 0) {
      const uint32_t dn = atomicAdd(&wq[kQueueLine * (8 + home)], 1u);
      if (dn == uint32_t(q_static(home)) - 1)
        last = atomicAdd(&wq[kQueueLine * 16], 1u) == uint32_t(min(8, int(gridDim.x))) - 1;
    }
    last = __shfl(last, 0);
    if (last && lane < 17) atomicExch(&wq[kQueueLine * lane], 0u);
  }
}

int64_t n_items(const PrefillArgs& a) { return int64_t(a.B) * a.Hkv * a.n_hsub * a.n_pblocks; }

template <int D, int MODE>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  // one workgroup per item, or with a queue one per compute unit (a workgroup
  // fills a CU: 8 waves at 2 per SIMD)
  const int64_t n = n_items(a);
  const int64_t grid = a.queue ? (n < a.n_cu ? n : a.n_cu) : n;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

// Bounded by the static schedule's grid, one workgroup per item; the queued
// schedule launches fewer but numbers the same items.
bool prefill_bf16_fits(const PrefillArgs& a) { return n_items(a) * kThreads <= kMaxWorkItems; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  if (a.D == 128) {
    switch (a.mode) {
      case kNope: return launch_t<128, kNope>(a, stream);
      case kRope: return launch_t<128, kRope>(a, stream);
      default: return launch_t<128, kBifocal>(a, stream);
    }
  }
  switch (a.mode) {
    case kNope: return launch_t<64, kNope>(a, stream);
    case kRope: return launch_t<64, kRope>(a, stream);
    default: return launch_t<64, kBifocal>(a, stream);
  }
}

}  // namespace prope
