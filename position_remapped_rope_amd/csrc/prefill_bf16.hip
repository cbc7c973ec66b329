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
// scaled by softmax_scale; causal, plus the window for NOPE/ROPE. Ids may be
// negative: the period and the remote map use floor semantics. NOPE/ROPE may add
// ALiBi biases - m_h (i - j) to the scaled scores (P-RoPE page, section 1: SWA
// with ALiBi; the window clamps the penalty to the kept distances).
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
#include <float.h>
#include <limits.h>

#include "prefill_common.hpp"

// Item-phase tracing, compiled in only by the trace build (PROPE_ITEM_TRACE=1):
// thread 0 of each of the first kTraceWGs workgroups records the 100 MHz
// real-time counter at entry (slot 0), at five points of each of its first
// kTraceItems items (slots 1 + 5k ...: start after the claim, end of the load
// and rotation setup, start of the tile loop, end of the loop, end of the
// item) and at exit (slot 63).
#ifndef PROPE_ITEM_TRACE
#define PROPE_ITEM_TRACE 0
#endif

namespace prope {
constexpr int kTraceWGs = 1024, kTraceSlots = 64, kTraceItems = 12;
#if PROPE_ITEM_TRACE
__device__ unsigned long long item_trace[kTraceWGs * kTraceSlots];
#endif
namespace {

__device__ __forceinline__ void trace_point(int slot) {
#if PROPE_ITEM_TRACE
  if (threadIdx.x == 0 && blockIdx.x < kTraceWGs && slot < kTraceSlots)
    item_trace[blockIdx.x * kTraceSlots + slot] = __builtin_amdgcn_s_memrealtime();
#else
  (void)slot;
#endif
}

using namespace pf;

constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 512;  // 8 wavefronts, 2 per SIMD
constexpr int kGroupThreads = kThreads / 2;

template <int D, int MODE, bool ALIBI>
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

  // Per-chunk constants kept in LDS rather than registers: the 4 pair
  // frequencies of each 16-byte column chunk, and for each rotation kind the
  // cos/sin of the affine id step between the two K rows a thread stages. The
  // second K row a thread stages is RPS keys after the first; when their
  // rotation ids differ by that step (RPS for base ids, RPS / s for remote ids
  // when s divides RPS) its cos/sin are the first row's times the step's.
  // The frequencies are held in the signed split of phase_split (one
  // instruction less per phase); the ALiBi kernels, which read them from LDS in
  // the loop and have fewer registers to spare, keep the plain split.
  __shared__ uint2 kfreq[2][CPR * 4];  // [0]: base frequencies, [1]: remote frequencies
  __shared__ float2 kstep[2][CPR * 4];
  constexpr bool kSplit = !ALIBI;
  auto kphase = [](int r, uint2 f) __attribute__((always_inline)) {
    return kSplit ? phase_top_split(r, f.x, f.y) : phase_top(r, f.x, f.y);
  };
  auto ksincos = [](int r, uint2 f, float& sn, float& cs) __attribute__((always_inline)) {
    if (kSplit) rope_sincos_split(r, f.x, f.y, sn, cs);
    else rope_sincos(r, f.x, f.y, sn, cs);
  };
  const int id_step1 = NU > 1 ? RPS : -1;
  const int sdiv = static_cast<int>(a.scale_div.div);
  const int id_step2 = (NU > 1 && RPS % sdiv == 0) ? RPS / sdiv : -1;
  if (MODE != kNope && tid < CPR * 4) {
    const uint32_t flo = a.f.lo[tid], fhi = a.f.hi[tid];
    const uint32_t rlo = a.fr.lo[tid], rhi = a.fr.hi[tid];
    const PhaseSplit sb = phase_split(flo, fhi), sm = phase_split(rlo, rhi);
    kfreq[0][tid] = kSplit ? make_uint2(sb.fls, sb.fhs) : make_uint2(flo, fhi);
    kfreq[1][tid] = kSplit ? make_uint2(sm.fls, sm.fhs) : make_uint2(rlo, rhi);
    float s1 = 0.f, c1 = 1.f, s2 = 0.f, c2 = 1.f;
    if (id_step1 >= 0) rope_sincos(id_step1, flo, fhi, s1, c1);
    if (id_step2 >= 0) rope_sincos(id_step2, rlo, rhi, s2, c2);
    kstep[0][tid] = make_float2(c1, s1);
    kstep[1][tid] = make_float2(c2, s2);
  }
  // ---- work items (one per workgroup, or from the per-XCD queues) --------------
  // (the barrier after each claim also publishes the tables above)
  ItemQueue iq(a);
  __shared__ int s_item;
  trace_point(0);
  int n_traced = 0;  // items of this workgroup so far (trace build)
  auto trace_item = [&](int k) __attribute__((always_inline)) {
    if (n_traced < kTraceItems) trace_point(1 + 5 * n_traced + k);
  };
#pragma clang loop unroll(disable)
  for (;;) {
  if (wave == 0) {
    const int r = iq.next(lane);
    if (lane == 0) s_item = r;
  }
  lds_barrier();
  int item = s_item;
  if (item < 0) break;
  trace_item(0);
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

  // pass of tile t. Tiles past the last (t >= T, staged but never read) get a
  // valid rotation kind too: NOPE/ROPE have pass 0 only, and bifocal's pass 1
  // (base ids) is valid even without a local window.
  auto pass_of = [&](int t) __attribute__((always_inline)) { return (MODE == kBifocal && t >= tc0) ? 1 : 0; };
  auto tile_of = [&](int t, int& p, int& kt) {
    p = pass_of(t);
    kt = p ? tb1 + (t - tc0) : tb0 + t;
  };
  // Are the rotation indices of a thread's two staged K rows (ids k0 and k1,
  // RPS keys apart, k0's index r0) one id step apart? It is enough that the ids
  // are RPS apart without wrapping around the int32 range: for remote ids
  // floor(p/s), s divides RPS wherever id_step >= 0; with a period P the index
  // r0 = k0 mod P must also stay below P - RPS, so that k1 mod P = r0 + RPS.
  auto rows_affine = [&](int k0, int k1, int r0, int rot, int id_step) __attribute__((always_inline)) {
    if (id_step < 0) return false;
    const bool ids = k1 > k0 && uint32_t(k1) - uint32_t(k0) == uint32_t(RPS);
    if (MODE == kRope && a.period > 0)  // (the ALiBi kernels, short of registers, compare the indices)
      return ALIBI ? rot_index<MODE>(k1, rot, a) - r0 == id_step : ids && r0 < a.period - RPS;
    return ids;
  };

  // ---- per-thread staging coordinates --------------------------------------
  // group g stages rows [HR*g, HR*g + HR) of every K and V tile
  const int gtid = tid & (kGroupThreads - 1);
  const int sc = gtid % CPR;                 // 16-byte column chunk this thread stages
  const int sr = group * HR + gtid / CPR;    // first row this thread stages (then sr + RPS)
  const uint32_t kcol_b = uint32_t(kvh) * D * 2 + sc * 16;
  const uint32_t srow_kv = uint32_t(sr) * rowk_b + kcol_b;  // this thread's first staged row, byte offset in K/V
  const uint32_t srow_id = uint32_t(sr) * 4;                // and in the ids

  u32x4_t kraw[NU], vraw[NU];
  int kid[NU];

  // Prologue staging, global -> registers: this thread's K rows (and ids) of
  // tile tk and V rows of tile tv into the given registers (a tile index
  // outside [0, T) is skipped)
  auto stage_load = [&](int tk, int tv, u32x4_t(&kr)[NU], int(&ki)[NU], u32x4_t(&vr)[NU])
                        __attribute__((always_inline)) {
    if (tk >= 0 && tk < T) {
      int p, kt;
      tile_of(tk, p, kt);
      const int rot = p ? rot1 : rot0;
      const uint32_t j0 = uint32_t(kt) * kBN;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t j = j0 + sr + RPS * u;
        kr[u] = bload16(kres, j * rowk_b + kcol_b);
        ki[u] = (MODE != kNope && rot) ? bload_i32(pres, j * 4) : 0;
      }
    }
    if (tv >= 0 && tv < T) {
      int p, kt;
      tile_of(tv, p, kt);
      const uint32_t j0 = uint32_t(kt) * kBN;
#pragma unroll
      for (int u = 0; u < NU; ++u) vr[u] = bload16(vres, (j0 + sr + RPS * u) * rowk_b + kcol_b);
    }
  };

  // registers -> LDS: K of tile tk (rotated for its pass) and V of tile tv
  auto stage_store = [&](int tk, int tv, const u32x4_t(&kr)[NU], const int(&ki)[NU],
                         const u32x4_t(&vr)[NU]) __attribute__((always_inline)) {
    if (tk >= 0 && tk < T) {
      int p, kt;
      tile_of(tk, p, kt);
      uint16_t* dst = Ks[tk & 1];
      const int rot = p ? rot1 : rot0;
      if (MODE != kNope && rot) {
        const int id_step = rot == 2 ? id_step2 : id_step1;
        uint2 kf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) kf[e] = kfreq[rot - 1][sc * 4 + e];
        float cs[4], sn[4];
        const int r0 = rot_index<MODE>(ki[0], rot, a);
#pragma unroll
        for (int e = 0; e < 4; ++e) ksincos(r0, kf[e], sn[e], cs[e]);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          if (u > 0) {
            if (rows_affine(ki[0], ki[u], r0, rot, id_step)) {  // (NU = 2: u = 1)
#pragma unroll
              for (int e = 0; e < 4; ++e) {  // (cs + i sn) * (step cos + i step sin)
                const float2 es = kstep[rot - 1][sc * 4 + e];
                const float c2 = cs[e] * es.x - sn[e] * es.y;
                const float s2 = sn[e] * es.x + cs[e] * es.y;
                cs[e] = c2;
                sn[e] = s2;
              }
            } else {
              const int ru = rot_index<MODE>(ki[u], rot, a);
#pragma unroll
              for (int e = 0; e < 4; ++e) ksincos(ru, kf[e], sn[e], cs[e]);
            }
          }
          u32x4_t y;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y0, y1;
            rot_pair(bf16_lo(kr[u][e]), bf16_hi(kr[u][e]), cs[e], sn[e], y0, y1);
            y[e] = pack_bf16(y0, y1);
          }
          *reinterpret_cast<u32x4_t*>(&dst[(sr + RPS * u) * KRow + sc * 8]) = y;
        }
      } else {
#pragma unroll
        for (int u = 0; u < NU; ++u) *reinterpret_cast<u32x4_t*>(&dst[(sr + RPS * u) * KRow + sc * 8]) = kr[u];
      }
    }
    if (tv >= 0 && tv < T) {
      uint16_t* dst = Vs[tv & 1];
#pragma unroll
      for (int u = 0; u < NU; ++u) *reinterpret_cast<u32x4_t*>(&dst[(sr + RPS * u) * VRow + sc * 8]) = vr[u];
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
  // tiles being staged, in registers (reloaded when that kind changes); the
  // ALiBi kernels, short of registers, read them from the LDS tables instead
  uint2 kf_reg[4];
  float2 ks_reg[4];
  auto load_kregs = [&](int rot) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf_reg[e] = kfreq[rot - 1][sc * 4 + e];
      ks_reg[e] = kstep[rot - 1][sc * 4 + e];
    }
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
        float sn, cs, y0, y1;
        ksincos(ru, kfreq[rot - 1][sc * 4 + e], sn, cs);
        rot_pair(bf16_lo(kraw[NU - 1][e]), bf16_hi(kraw[NU - 1][e]), cs, sn, y0, y1);
        y[e] = pack_bf16(y0, y1);
      }
      *reinterpret_cast<u32x4_t*>(&Ks[tk & 1][(sr + RPS * (NU - 1)) * KRow + sc * 8]) = y;
    }
  };

  // ---- query operand (B of S^T = K Q^T): lane holds row lr, dims ks*16 + lg*8 .. +7
  u32x4_t qreg[KS];
  // issue the loads of this lane's query chunks and id (rows past the sequence read 0) ...
  auto issue_q = [&](u32x4_t(&qraw)[KS], int& qid) __attribute__((always_inline)) {
    const uint32_t i = uint32_t(i0 + lr);
    const uint32_t qoff = i * rowq_b + uint32_t(h) * D * 2 + lg * 16;
    qid = MODE != kNope ? bload_i32(pres, i * 4) : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = bload16(qres, qoff + ks * 32);
  };
  // ... and rotate them for pass p into qreg
  auto rotate_q = [&](int p, const u32x4_t(&qraw)[KS], int qid) __attribute__((always_inline)) {
    const int rot = p ? rot1 : rot0;
    const int r = (MODE != kNope && rot) ? rot_index<MODE>(qid, rot, a) : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = qraw[ks];
      if (MODE != kNope && rot) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // pair frequencies from the LDS copy of the table
          float sn, cs, y0, y1;
          ksincos(r, kfreq[rot - 1][ks * 8 + lg * 4 + e], sn, cs);
          rot_pair(bf16_lo(x[e]), bf16_hi(x[e]), cs, sn, y0, y1);
          x[e] = pack_bf16(y0, y1);
        }
      }
      qreg[ks] = x;
    }
  };
  auto load_q = [&](int p) __attribute__((always_inline)) {
    u32x4_t qraw[KS];
    int qid;
    issue_q(qraw, qid);
    rotate_q(p, qraw, qid);
  };

  // ---- per-lane LDS addresses of the PV operand (transposing reads of V) ---
  // A operand of O^T += V^T P^T for d-block db and 16-key step kk: lane (lr, lg)
  // needs V[16kk + 4lg + e][32db + lr] for e = 0..3 and V[16kk + 8 + 4lg + e][..].
  const int lane_d = lr - 4 * lg;  // i - j offset of this lane's first score register within a wave's tile
  const int j15 = lane & 15;
  const int vrow0 = 4 * lg + (j15 >> 2);
  const int vcol0 = 16 * (lr >> 4) + 4 * (j15 & 3);

  // ---- running statistics ---------------------------------------------------
  f32x16_t oacc[DB];   // set to zero after the prologue, which does not need them
  f32x16_t sacc[2];    // S^T of the tile in flight (two 32-key blocks)
  u32x4_t pop[4];      // its P, bf16, as four 16-key B operands
  // Reference max of the scaled scores (log2 units) that P is taken against.
  // It starts at -FLT_MAX rather than -inf, so that it is always a finite
  // reference: the first kept key of a row raises it to that tile's max (and the
  // rescale of the empty O and l by 2^(-FLT_MAX - max) is a multiply by 0), and a
  // row with no kept key yet takes P = 2^-inf = 0.
  float m_run = -FLT_MAX;
  float l_run = 0.f;        // this lane's share of the running sum
  const float sl2 = a.scale_log2;
  // ALiBi slope of this wave's head in log2 units (the scores are kept in log2 units)
  const float slope2 = ALIBI ? a.alibi[h] * 1.4426950408889634f : 0.f;

  // does tile t hold any kept (row, key) pair of this wave? Also: do some of
  // its pairs fall below the pass's distance range (need_lo) or above it
  // (need_hi)?
  auto wave_live = [&](int t, bool& need_lo, bool& need_hi, int& dlo, int& dhi, int& j0)
                       __attribute__((always_inline)) {
    int p, kt;
    tile_of(t, p, kt);
    dlo = p ? dlo1 : dlo0;
    dhi = p ? dhi1 : dhi0;
    j0 = kt * kBN;
    const int dmin = i0 - (j0 + kBN - 1), dmax = i1 - j0;
    need_lo = dmin < dlo;
    need_hi = dmax > dhi;
    return i1 >= i0 && dmax >= dlo && dmin <= dhi;
  };
  auto live = [&](int t) __attribute__((always_inline)) {
    bool nl, nh;
    int dlo, dhi, j0;
    return wave_live(t, nl, nh, dlo, dhi, j0);
  };

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
    if (NU > 1) need_fix = !rows_affine(kid[0], kid[NU - 1], r0, rot, id_step);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sn, cs, y0, y1;
      const uint2 kf = ALIBI ? kfreq[rot - 1][sc * 4 + e] : kf_reg[e];
      {  // The phase's top 23 bits as the mantissa of a float x in [1, 2): the
         // sine and cosine take revolutions, so x is the same angle (one
         // instruction instead of a conversion and a scaling; the truncation
         // moves the angle by under 2^-23 turn, far below the bf16 rounding of
         // the rotated key)
        const float x = __uint_as_float(__builtin_amdgcn_alignbit(0x7fu, kphase(r0, kf), 9));
        sn = __builtin_amdgcn_sinf(x);
        cs = __builtin_amdgcn_cosf(x);
      }
      rot_pair(bf16_lo(kraw[0][e]), bf16_hi(kraw[0][e]), cs, sn, y0, y1);
      krot[0][e] = pack_bf16(y0, y1);
      if (NU > 1) {  // the second row: one id step further, (cs + i sn) * (step cos + i step sin)
        const float2 es = ALIBI ? kstep[rot - 1][sc * 4 + e] : ks_reg[e];
        const float c2 = cs * es.x - sn * es.y, s2 = sn * es.x + cs * es.y;
        rot_pair(bf16_lo(kraw[NU - 1][e]), bf16_hi(kraw[NU - 1][e]), c2, s2, y0, y1);
        krot[NU - 1][e] = pack_bf16(y0, y1);
      }
    }
  };
  // Matrix phase of iteration t: PV(t) (16 MFMAs), then QK(t+1) (16 MFMAs),
  // with the LDS stores of this thread's rows of K tile t+2 and V tile t+1 one
  // per MFMA slot, scheduling barriers keeping that order. Operand reads run
  // one PV step / two QK steps ahead of their MFMAs.
  // NoPE: the V operands of the first two PV steps (keys 0-31, which this
  // wave's group staged itself) are read at the start of the vector phase,
  // which has no rotation work to hide and leaves this wave's LDS port idle
  // (one wave reads only about a quarter of the CU's LDS rate, so the matrix
  // phase is bound by its own operand reads). The rotating modes measured
  // slower with it: their vector phase is already full.
  constexpr bool kVpre = MODE == kNope && !ALIBI;
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
    constexpr int KA = 2;  // K steps read ahead
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

  // The bifocal kernel forms P against the current reference before any row
  // max, and takes the max only when a lane's sum of P exceeds 2^8 (P >= 0, so
  // a smaller sum bounds every P by 2^8): 17 instructions fewer per tile of its
  // long items, and the same references, P and results as the max-first order
  // wherever no P lies within a bf16 rounding of 2^8. The other modes keep the
  // max first: in their short items the first kept tile of every row would
  // form P twice, and keeping the scores live through P spills around the
  // item set-up.
  constexpr bool kSumCheck = MODE == kBifocal && !ALIBI;
  // vector phase of tile t: mask, online softmax, P -> bf16, lazy O rescale
  auto softmax_step = [&](int t) __attribute__((always_inline)) {
    bool need_lo, need_hi;
    int dlo, dhi, j0;
    if (!wave_live(t, need_lo, need_hi, dlo, dhi, j0)) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pop[kk] = u32x4_t{0, 0, 0, 0};
      rotate_k(t);
      return false;
    }
    // i - j of register 0 of block 0 is (i0 - j0) + (lr - 4 lg): a wave-uniform
    // part (scalar) and a per-lane constant, folded with the bounds below
    if (ALIBI) {  // logits in log2 units: s * scale - slope * (i - j)
      const float b0 = -slope2 * static_cast<float>(lane_d + (i0 - j0));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float c = static_cast<float>(nb * 32 + 8 * (r >> 2) + (r & 3));
          sacc[nb][r] = fmaf(sacc[nb][r], sl2, fmaf(slope2, c, b0));
        }
    }
    // Keep dlo <= i - j <= dhi, i.e. dbase - dhi <= c <= dbase - dlo for the key
    // offset c = j - j0 - 4 lg of a register, a constant, with dbase the i - j
    // of register 0 of block 0: each bound that cuts the tile costs one compare
    // and one select per score. (A live tile has dlo <= S and dhi >= -S, so
    // neither difference overflows.)
    if (need_lo) {
      const int chi = lane_d + (i0 - j0 - dlo);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (nb * 32 + 8 * (r >> 2) + (r & 3) > chi) sacc[nb][r] = -INFINITY;
    }
    if (need_hi) {
      const int clo = lane_d + (i0 - j0 - dhi);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (nb * 32 + 8 * (r >> 2) + (r & 3) < clo) sacc[nb][r] = -INFINITY;
    }
    const float smul = ALIBI ? 1.f : sl2;  // ALiBi scores are scaled already
    // the row max of this lane's 32 scores in 16 three-input maxima, and across
    // the two lanes that hold the row; smul > 0, so scaling after the max is
    // the max of the scaled scores
    auto row_max = [&]() __attribute__((always_inline)) {
      auto max3 = [](float x, float y, float z) __attribute__((always_inline)) { return fmaxf(fmaxf(x, y), z); };
      float m1[10];
#pragma unroll
      for (int g = 0; g < 10; ++g) {
        const int v = 3 * g;
        m1[g] = max3(sacc[v >> 4][v & 15], sacc[(v + 1) >> 4][(v + 1) & 15], sacc[(v + 2) >> 4][(v + 2) & 15]);
      }
      const float m2 = max3(max3(m1[0], m1[1], m1[2]), max3(m1[3], m1[4], m1[5]), max3(m1[6], m1[7], m1[8]));
      return xhalf_max(fmaxf(m2, max3(m1[9], sacc[1][14], sacc[1][15]))) * smul;
    };
    // The reference max moves only when the tile's max exceeds it by more than
    // 8 (log2 units): P <= 2^8 stays exact in bf16 and fp32, and O and l are
    // rescaled far less often. The final O / l and LSE = m + log2 l are unchanged.
    auto raise_ref = [&](float mx) __attribute__((always_inline)) {
      if (__any(mx > m_run + 8.f)) {  // some row of the wave raises its reference
        const float mnew = mx > m_run + 8.f ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
        m_run = mnew;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        return true;
      }
      return false;
    };
    // P of the tile against the current reference, and this lane's sum of it
    // (from the same bf16 P the PV product uses)
    auto exps = [&]() __attribute__((always_inline)) {
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int nb = kk >> 1, r0 = (kk & 1) * 8;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r0 + e], smul, -m_run));
        const u32x4_t w = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                           pack_bf16(pv[6], pv[7])};
        pop[kk] = w;
        rs0 = add_bf16_pair(w[0], rs0);
        rs1 = add_bf16_pair(w[1], rs1);
        rs0 = add_bf16_pair(w[2], rs0);
        rs1 = add_bf16_pair(w[3], rs1);
      }
      return rs0 + rs1;
    };
    float ts;
    if (kSumCheck) {
      // P first, against the current reference: a lane's P values are >= 0,
      // so a sum of at most 2^8 bounds each of them, and only a larger sum (an
      // infinite one while a row's reference is still -FLT_MAX) needs the max
      rotate_k(t);
      ts = exps();
#pragma unroll
      for (int u = 0; u < NU; ++u)  // the rotation stays ahead of the branch, among the exps
#pragma unroll
        for (int e = 0; e < 4; ++e) asm volatile("" ::"v"(krot[u][e]));
      if (__any(!(ts <= 256.f)) && raise_ref(row_max())) ts = exps();
    } else {
      const float mx = row_max();
      rotate_k(t);
      raise_ref(mx);
      ts = exps();
    }
    l_run += ts;
    return true;
  };

  // ---- prologue: one round of global loads (K tiles 0 and 1 with their ids,
  // V tile 0, the queries, then K tile 2 and V tile 1 into the loop's staging
  // registers, in the loop's issue order so its waits stay exact), then K
  // tiles 0 and 1 and V tile 0 to LDS and the query rotation
  {
    u32x4_t kraw0[NU], kraw1[NU], vraw0[NU], qraw[KS];
    int kid0[NU], kid1[NU], qid;
    stage_load(0, 0, kraw0, kid0, vraw0);
    stage_load(1, -1, kraw1, kid1, vraw0);
    issue_q(qraw, qid);
    stage_load_nb(2, 1);
    stage_store(0, 0, kraw0, kid0, vraw0);
    stage_store(1, -1, kraw1, kid1, vraw0);
    rotate_q(pass_of(0), qraw, qid);
  }
  lds_barrier();

  // ---- phases -----------------------------------------------------------------
  // Group 0: QK(0) | soft(0) | PV(0) QK(1) | soft(1) | PV(1) QK(2) | ... | PV(T-1) | -
  // Group 1:  -    | QK(0)   | soft(0)     | PV(0) QK(1) | ...         | PV(T-1)
  // with a workgroup barrier after every phase. The vector phase of tile t
  // also rotates this wave's rows of K tile t+2; the matrix phase after it
  // stores them and its rows of V tile t+1 to LDS between its MFMAs, then
  // issues the loads of K tile t+3 and V tile t+2.
  trace_item(1);
  if (group == 1) lds_barrier();
  qk_or_clear(0);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pop[kk] = u32x4_t{0, 0, 0, 0};
  lds_barrier();
  trace_item(2);
  if (MODE != kNope && !ALIBI) load_kregs(pass_of(2) ? rot1 : rot0);  // the kind of the first K tile the loop stages
  // the one iteration after which the query switches to the local pass (none
  // when either pass has no tile)
  const int tq_switch = (MODE == kBifocal && tc0 >= 1 && tc0 < T) ? tc0 - 1 : -1;
  // Wave priority of the matrix phase: when both waves of a SIMD want an issue
  // slot, the SIMD's arbiter serves the higher one first. NOPE and ROPE raise
  // the matrix phase, so the MFMA stream gets its slots first and the other
  // wave's vector work fills the gaps. The bifocal kernel, whose vector phase
  // (softmax plus the K rotation of its long items) is the longer one, leaves
  // both phases at the default: 64K and 128K 0.5-0.8% faster in alternating
  // runs on two machines.
  constexpr int kMatPrio = MODE == kBifocal ? 0 : 1;
#pragma clang loop unroll(disable)
  for (int t = 0; t < T; ++t) {
    // the K tiles staged from here on (t + 2 onwards) are all local ones
    if (MODE == kBifocal && !ALIBI && t + 2 == tc0) load_kregs(rot1);
    if (kVpre) read_vpre(t);
    softmax_step(t);  // P of a tile with no kept key is zero
    if (MODE == kBifocal && t == tq_switch) load_q(1);
    lds_barrier();
    // one region: PV(t), QK(t+1) (the scores of tile T, if any, are never used)
    // and the LDS stores of K tile t+2 / V tile t+1 between the MFMAs
    if (kMatPrio != 0) __builtin_amdgcn_s_setprio(kMatPrio);
    mphase(t);
    fix_row1(t + 2);
    stage_load_nb(t + 3, t + 2);
    if (kMatPrio != 0) __builtin_amdgcn_s_setprio(0);
    lds_barrier();
  }
  if (group == 0) lds_barrier();
  trace_item(3);

  // ---- finalize ---------------------------------------------------------------
  // O / l goes through LDS so that each global store writes whole rows: a
  // lane's accumulators hold 4 dims of one row, which stored directly would
  // touch 32 rows per instruction. Both groups have passed their last loop
  // barrier, so the K and V tiles are free: waves 0-3 use the K buffers, waves
  // 4-7 the V buffers, 32 rows of D + 8 elements each (16-byte aligned rows).
  const float l = l_run + __shfl_xor(l_run, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  constexpr int ORow = D + 8;
  static_assert(4 * 32 * ORow <= 2 * kBN * KRow && 4 * 32 * ORow <= 2 * kBN * VRow, "output staging fits");
  uint16_t* ob = (group == 0 ? &Ks[0][0] : &Vs[0][0]) + (wave & 3) * 32 * ORow;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2_t w;
      w[0] = pack_bf16(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
      w[1] = pack_bf16(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
      *reinterpret_cast<u32x2_t*>(ob + lr * ORow + db * 32 + 8 * g4 + 4 * lg) = w;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's rows are in LDS
  uint16_t* og = static_cast<uint16_t*>(a.o) + size_t(b) * S * a.Hq * D + size_t(h) * D;
  const size_t rowq = size_t(a.Hq) * D;
  constexpr int RPI = 64 / CPR;  // rows per read / store instruction
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rr = it * RPI + lane / CPR, ch = lane % CPR;
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(ob + rr * ORow + ch * 8);
    if (i0 + rr <= i1) *reinterpret_cast<u32x4_t*>(og + size_t(i0 + rr) * rowq + ch * 8) = x;
  }
  const int i = i0 + lr;
  if (a.lse && lg == 0 && i <= i1) {
    const float lse = l > 0.f ? (m_run + log2f(l)) * 0.6931471805599453f : -INFINITY;
    a.lse[(size_t(b) * a.Hq + h) * S + i] = lse;
  }
  lds_barrier();  // LDS and s_item are reused by the next item (the output stores need no wait)
  trace_item(4);
  ++n_traced;
  }  // items

  if (wave == 0) iq.finish(lane);
  trace_point(kTraceSlots - 1);
}

int64_t n_items(const PrefillArgs& a) { return int64_t(a.B) * a.Hkv * a.n_hsub * a.n_pblocks; }

template <int D, int MODE, bool ALIBI = false>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  // one workgroup per item, or with a queue one per compute unit (a workgroup
  // fills a CU: 8 waves at 2 per SIMD)
  const int64_t n = n_items(a);
  const int64_t grid = a.queue ? (n < a.n_cu ? n : a.n_cu) : n;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE, ALIBI>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  if (a.alibi) return a.mode == kNope ? launch_t<D, kNope, true>(a, stream) : launch_t<D, kRope, true>(a, stream);
  switch (a.mode) {
    case kNope: return launch_t<D, kNope>(a, stream);
    case kRope: return launch_t<D, kRope>(a, stream);
    default: return launch_t<D, kBifocal>(a, stream);
  }
}

}  // namespace

// Bounded by the static schedule's grid, one workgroup per item; the queued
// schedule launches fewer but numbers the same items.
bool prefill_bf16_fits(const PrefillArgs& a) { return n_items(a) * kThreads <= kMaxWorkItems; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  return a.D == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace prope

#if PROPE_ITEM_TRACE
// Trace build only (not part of the library's ABI): copy the item-phase table
// (kTraceWGs x kTraceSlots 64-bit counters, zero where nothing was recorded)
// to host memory and clear it. dst must hold sizeof the table; returns 0, or
// the HIP error of the copy.
extern "C" int prope_item_trace_read(void* dst, size_t bytes) {
  if (bytes < sizeof(prope::item_trace)) return hipErrorInvalidValue;
  hipError_t e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(prope::item_trace), sizeof(prope::item_trace));
  if (e != hipSuccess) return e;
  static unsigned long long zero[prope::kTraceWGs * prope::kTraceSlots];
  return hipMemcpyToSymbol(HIP_SYMBOL(prope::item_trace), zero, sizeof(zero));
}
#endif
