// Flash-style causal attention prefill with RoPE fused into the tile loads,
// bf16 operands, fp32 accumulation, gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Scores per mode (token indices i, j; ids p):
//   NOPE     q_i . k_j                                  (P-RoPE page, Eq. (6))
//   ROPE     (R_r q_i) . (R_r k_j), r = p mod P or p    (P-RoPE page, Eq. (3)-(5))
//   BIFOCAL  local  (i - j <= w0): RoPE at p
//            remote (i - j >  w0): RoPE at floor(p / s) (Jet-Long page, Eq. (1), (3))
// scaled by softmax_scale; causal, plus the window for NOPE/ROPE.
//
// Work decomposition. A workgroup (8 wavefronts, two per SIMD) owns 256 query
// rows: HG query heads of one KV group times BMp = 256/HG consecutive
// positions. Each wave owns 32 rows = 32 positions of one head. All query heads that read the same KV
// head sit in one workgroup when possible (HG = 4, 2 or 1), so each K tile
// rotated into LDS is shared by all of them.
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
// of accumulator register r. The same
// register order serves directly as the B operand of O^T += V^T P^T, with the
// A operand V^T read from an LDS copy of V stored transposed.
#include <limits.h>

#include "internal.hpp"

namespace prope {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 512;  // 8 wavefronts, 2 per SIMD
constexpr int kVRow = 68;      // transposed-V row stride (elements): 64 keys + pad

__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Element (d, n) of the transposed V tile. The row stride of 34 dwords puts
// consecutive d two banks apart: 8-byte operand reads by 16 lanes (consecutive
// d) and 4-byte transposing writes by 32 lanes (consecutive key pairs n/2) both
// hit distinct banks.
__device__ __forceinline__ int vt_index(int d, int n) { return d * kVRow + n; }

struct Pass {
  int dlo, dhi;  // keep a key iff dlo <= i - j <= dhi
  int rot;       // 0: none, 1: base ids (mod period if any), 2: remote ids floor(p/s)
};

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
  constexpr int KS = D / 16;            // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;            // 32-row blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;   // K rows covered by one staging sweep
  constexpr int NU = kBN / RPP;         // K chunks per thread per tile
  constexpr int VPW = kThreads / 32;    // V column chunks covered per sweep
  constexpr int NV = (CPR + VPW - 1) / VPW;  // V chunks (row pairs) per thread per tile
  constexpr int KRow = D + 8;           // K tile row stride (elements)
  static_assert(NU >= 1 && NU <= 2 && NV >= 1, "staging layout");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * KRow];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * kVRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;

  // ---- work item --------------------------------------------------------
  int item = xcd_remap(blockIdx.x, gridDim.x);
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

  const size_t rowq = size_t(a.Hq) * D, rowk = size_t(a.Hkv) * D;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + size_t(b) * S * rowq + size_t(h) * D;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + size_t(b) * S * rowk + size_t(kvh) * D;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + size_t(b) * S * rowk + size_t(kvh) * D;
  const int32_t* posb = MODE == kNope ? nullptr : a.pos + size_t(b) * S;

  // ---- passes and tile ranges ---------------------------------------------
  Pass pass0, pass1;
  int npass;
  if (MODE == kBifocal) {
    const int w0 = a.window_left;
    pass0 = {w0 + 1, INT_MAX, 2};
    pass1 = {0, w0, 1};
    npass = w0 >= 0 ? 2 : 1;
  } else {
    pass0 = {0, a.window_left < 0 ? INT_MAX : a.window_left, MODE == kNope ? 0 : 1};
    pass1 = pass0;
    npass = 1;
  }
  auto tile_range = [&](const Pass& ps, int& tb, int& tc) {
    const int64_t jlo = max<int64_t>(0, int64_t(P0) - ps.dhi);
    const int64_t jhi = min<int64_t>(S - 1, int64_t(P1) - ps.dlo);
    tb = 0;
    tc = 0;
    if (jhi >= jlo) {
      tb = static_cast<int>(jlo / kBN);
      tc = static_cast<int>(jhi / kBN) - tb + 1;
    }
  };
  int tb0, tc0, tb1 = 0, tc1 = 0;
  tile_range(pass0, tb0, tc0);
  if (npass > 1) tile_range(pass1, tb1, tc1);
  const int T = tc0 + tc1;

  // ---- per-thread staging coordinates --------------------------------------
  const int sc = tid % CPR;   // 16-byte column chunk of K this thread stages
  const int sr = tid / CPR;   // first K row this thread stages (second: sr + RPP)
  const int vp = tid & 31;    // V key pair (rows 2vp, 2vp+1) this thread stages
  const int vc = tid >> 5;    // first V column chunk this thread stages
  uint32_t kflo[4], kfhi[4];  // frequencies of the K chunk's 4 pairs
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kflo[e] = a.f.lo[sc * 4 + e];
    kfhi[e] = a.f.hi[sc * 4 + e];
  }
  // The second K row a thread stages is RPP keys after the first. When the
  // rotation ids of the two rows differ by the pass's affine step (RPP for base
  // ids; RPP / s for remote ids when s divides RPP), the second row's cos/sin
  // are the first row's times the fixed rotation by that step.
  float estep_c[4], estep_s[4];
  int id_step = -1;

  u32x4_t kraw[NU], vraw[2 * NV];
  int kid[NU];

  auto tile_of = [&](int t, int& p, int& kt) {
    p = t < tc0 ? 0 : 1;
    kt = p ? tb1 + (t - tc0) : tb0 + t;
  };

  auto set_pass_step = [&](int rot) {
    id_step = -1;
    if (MODE == kNope || rot == 0 || NU < 2) return;
    if (rot == 2) {
      const uint32_t sdiv = a.scale_div.div;
      if (RPP % sdiv == 0) id_step = RPP / static_cast<int>(sdiv);
    } else {
      id_step = RPP;  // (a period wrap inside the pair of rows is caught by the check below)
    }
    if (id_step >= 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) rope_sincos(id_step, kflo[e], kfhi[e], estep_s[e], estep_c[e]);
    }
  };

  auto stage_load = [&](int t) {
    int p, kt;
    tile_of(t, p, kt);
    const int j0 = kt * kBN;
    const int rot = p ? pass1.rot : pass0.rot;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int j = j0 + sr + RPP * u;
      const bool ok = j < S;
      kraw[u] = ok ? *reinterpret_cast<const u32x4_t*>(kg + size_t(j) * rowk + sc * 8) : u32x4_t{0, 0, 0, 0};
      kid[u] = (ok && rot) ? posb[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int j = j0 + 2 * vp;
      const int c = vc + VPW * u;
      if (c >= CPR) continue;  // d = 64: half the threads stage no V
      vraw[2 * u] = j < S ? *reinterpret_cast<const u32x4_t*>(vg + size_t(j) * rowk + c * 8) : u32x4_t{0, 0, 0, 0};
      vraw[2 * u + 1] = j + 1 < S ? *reinterpret_cast<const u32x4_t*>(vg + size_t(j + 1) * rowk + c * 8) : u32x4_t{0, 0, 0, 0};
    }
  };

  auto stage_store = [&](int t, int buf) {
    int p, kt;
    tile_of(t, p, kt);
    const int rot = p ? pass1.rot : pass0.rot;
    if (MODE != kNope && rot) {
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
            for (int e = 0; e < 4; ++e) {  // (cs + i sn) * (estep_c + i estep_s)
              const float c2 = cs[e] * estep_c[e] - sn[e] * estep_s[e];
              const float s2 = sn[e] * estep_c[e] + cs[e] * estep_s[e];
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
        *reinterpret_cast<u32x4_t*>(&Ks[buf][(sr + RPP * u) * KRow + sc * 8]) = y;
      }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u)
        *reinterpret_cast<u32x4_t*>(&Ks[buf][(sr + RPP * u) * KRow + sc * 8]) = kraw[u];
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      if (vc + VPW * u >= CPR) continue;
      const int n = 2 * vp;
      const u32x4_t r0 = vraw[2 * u], r1 = vraw[2 * u + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = (vc + VPW * u) * 8 + 2 * e;
        // column d (low halves) and d+1 (high halves) of rows n, n+1
        const uint32_t lo = (r0[e] & 0xffffu) | (r1[e] << 16);
        const uint32_t hi = (r0[e] >> 16) | (r1[e] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&Vt[buf][vt_index(d, n)]) = lo;
        *reinterpret_cast<uint32_t*>(&Vt[buf][vt_index(d + 1, n)]) = hi;
      }
    }
  };

  // ---- query operand (B of S^T = K Q^T): lane holds row lr, dims ks*16 + lg*8 .. +7
  u32x4_t qreg[KS];
  auto load_q = [&](int p) {
    const int rot = p ? pass1.rot : pass0.rot;
    const int i = i0 + lr;
    const bool ok = i <= i1;
    const int r = (ok && MODE != kNope && rot) ? rot_index<MODE>(posb[i], rot, a) : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = ok ? *reinterpret_cast<const u32x4_t*>(qg + size_t(i) * rowq + ks * 16 + lg * 8)
                     : u32x4_t{0, 0, 0, 0};
      if (MODE != kNope && rot) {
        uint32_t flo[4], fhi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          flo[e] = a.f.lo[ks * 8 + lg * 4 + e];
          fhi[e] = a.f.hi[ks * 8 + lg * 4 + e];
        }
        x = rotate_chunk(x, r, flo, fhi);
      }
      qreg[ks] = x;
    }
  };

  // ---- running statistics ---------------------------------------------------
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.f;        // this lane's share of the running sum
  const float sl2 = a.scale_log2;

  // ---- main loop ------------------------------------------------------------
  int cur_pass = 0;
  set_pass_step(pass0.rot);
  stage_load(0);
  stage_store(0, 0);
  load_q(0);
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    int p, kt;
    tile_of(t, p, kt);
    if (p != cur_pass) {  // entering the local pass: re-rotate queries and the K step
      cur_pass = p;
      load_q(p);
      set_pass_step(pass1.rot);
    }
    if (t + 1 < T) {
      int pn, ktn;
      tile_of(t + 1, pn, ktn);
      if (pn != cur_pass) set_pass_step(pass1.rot);
      stage_load(t + 1);
    }
    const int j0 = kt * kBN;
    const int dlo = p ? pass1.dlo : pass0.dlo, dhi = p ? pass1.dhi : pass0.dhi;
    const int dmin = i0 - (j0 + kBN - 1), dmax = i1 - j0;
    const bool live = i1 >= i0 && dmax >= dlo && dmin <= dhi;
    if (live) {
      const bool need_mask = dmin < dlo || dmax > dhi;
      // S^T = K Q^T for the 64 keys (two 32-key blocks nb) and the wave's 32 rows
      f32x16_t sacc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[nb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4_t kop = *reinterpret_cast<const u32x4_t*>(&Ks[buf][(nb * 32 + lr) * KRow + ks * 16 + lg * 8]);
          sacc[nb] = mfma32x32x16(kop, qreg[ks], sacc[nb]);
        }
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
      // online softmax; a lane's column is one query row
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[nb][r], sacc[nb][r + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m_run, mx * sl2);
      const bool grow = mnew > m_run;
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mref);
      m_run = mnew;
      float rs = 0.f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r], sl2, -mref));
          sacc[nb][r] = pv;
          rs += pv;
        }
      l_run = l_run * alpha + rs;
      // rescale O only when some row of the wave raised its max
      if (__any(grow)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      // O^T += V^T P^T over the 64 keys (four k-steps of 16)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int nb = kk >> 1, r0 = (kk & 1) * 8;
        const u32x4_t pop = {pack_bf16(sacc[nb][r0 + 0], sacc[nb][r0 + 1]),
                             pack_bf16(sacc[nb][r0 + 2], sacc[nb][r0 + 3]),
                             pack_bf16(sacc[nb][r0 + 4], sacc[nb][r0 + 5]),
                             pack_bf16(sacc[nb][r0 + 6], sacc[nb][r0 + 7])};
        const int n = kk * 16 + 4 * lg;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + lr;
          const u32x2_t va = *reinterpret_cast<const u32x2_t*>(&Vt[buf][vt_index(d, n)]);
          const u32x2_t vb = *reinterpret_cast<const u32x2_t*>(&Vt[buf][vt_index(d, n + 8)]);
          const u32x4_t vop = {va[0], va[1], vb[0], vb[1]};
          oacc[db] = mfma32x32x16(vop, pop, oacc[db]);
        }
      }
    }
    if (t + 1 < T) stage_store(t + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- finalize ---------------------------------------------------------------
  uint16_t* og = static_cast<uint16_t*>(a.o) + size_t(b) * S * rowq + size_t(h) * D;
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
}

template <int D, int MODE>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int64_t n = int64_t(a.B) * a.Hkv * a.n_hsub * a.n_pblocks;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE>), dim3(static_cast<unsigned>(n)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

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
