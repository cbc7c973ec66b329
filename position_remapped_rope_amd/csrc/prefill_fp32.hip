// float32 prefill: same scores, masks and bifocal routing as the bf16 kernel,
// computed with fp32 vector ALU (no operand rounding). D / 8 adjacent lanes
// share one query row of one head, 8 dims each, and reduce each score with
// lane shuffles; K (rotated in fp32) and V tiles of 32 keys are staged in LDS,
// the next tile's loads in flight while the current one is processed.
// Meant for small fp32 problems such as the EndPrompt two-segment check: the
// narrow row split gives a 256-token problem enough workgroups to spread over
// the chip. The bf16 MFMA kernel is the throughput path.
#include <limits.h>

#include "internal.hpp"

namespace prope {
namespace {

constexpr int kBNf = 32;
constexpr int kThreadsF = 256;

// Sum over the N = 8 or 16 adjacent lanes that share a query row, with DPP
// lane permutations inside the VALU (no LDS round trip): swap with lane ^ 1,
// then ^ 2 (each lane now holds its quad's sum), then lane i with 7 - i of its
// group of 8 (the two quads), then, for 16, lane i with 15 - i of its row.
template <int N>
__device__ __forceinline__ float row_group_sum(float x) {
  static_assert(N == 8 || N == 16, "lanes per row");
  auto dpp = [](float v, int ctrl) {
    switch (ctrl) {  // the control must be a constant expression
      case 0: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
      case 1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
      case 2: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
    }
  };
  x += dpp(x, 0);  // quad_perm [1,0,3,2]
  x += dpp(x, 1);  // quad_perm [2,3,0,1]
  x += dpp(x, 2);  // row_half_mirror
  if (N == 16) x += dpp(x, 3);  // row_mirror
  return x;
}

template <int MODE>
__device__ __forceinline__ int rot_index_f(int p, int rot, const PrefillArgs& a) {
  if (rot == 2) return static_cast<int>(fastdiv(static_cast<uint32_t>(p), a.scale_div));
  if (MODE == kRope) return a.period > 0 ? static_cast<int>(fastmod(static_cast<uint32_t>(p), a.period_div)) : p;
  return p;
}

// TPR = D / 8 lanes share one query row, each owning 8 of its dims; a
// workgroup covers 256 / TPR rows (HG heads x BMp positions, set by the launcher).
template <int D, int MODE>
__global__ __launch_bounds__(kThreadsF) void prefill_fp32_kernel(const PrefillArgs a) {
  constexpr int DH = 8;                            // dims per lane
  constexpr int TPR = D / DH;                      // lanes per query row
  constexpr int NPR = D / 2;                       // pairs per row
  constexpr int PAIRS = kBNf * NPR / kThreadsF;    // pairs staged per thread
  constexpr int RPS = kThreadsF / NPR;             // rows per staging sweep
  __shared__ __attribute__((aligned(16))) float Ks[kBNf][D];
  __shared__ __attribute__((aligned(16))) float Vs[kBNf][D];

  const int tid = threadIdx.x;
  const int row = tid / TPR, part = tid % TPR;
  int item = xcd_remap(blockIdx.x, gridDim.x);
  const int pb = a.n_pblocks - 1 - (item % a.n_pblocks);
  item /= a.n_pblocks;
  const int hsub = item % a.n_hsub;
  item /= a.n_hsub;
  const int kvh = item % a.Hkv;
  const int b = item / a.Hkv;
  const int S = a.S;
  const int P0 = pb * a.BMp;
  const int P1 = min(S, P0 + a.BMp) - 1;
  const int hl = row / a.BMp;
  const int i = P0 + row - hl * a.BMp;
  const bool valid = i < S;
  const int h = kvh * a.G + hsub * a.HG + hl;

  const size_t rowq = size_t(a.Hq) * D, rowk = size_t(a.Hkv) * D;
  const float* qg = static_cast<const float*>(a.q) + size_t(b) * S * rowq + size_t(h) * D;
  const float* kg = static_cast<const float*>(a.k) + size_t(b) * S * rowk + size_t(kvh) * D;
  const float* vg = static_cast<const float*>(a.v) + size_t(b) * S * rowk + size_t(kvh) * D;
  const int32_t* posb = MODE == kNope ? nullptr : a.pos + size_t(b) * S;

  int dlo[2], dhi[2], rot[2], npass;
  if (MODE == kBifocal) {
    dlo[0] = a.window_left + 1; dhi[0] = INT_MAX; rot[0] = 2;
    dlo[1] = 0; dhi[1] = a.window_left; rot[1] = 1;
    npass = a.window_left >= 0 ? 2 : 1;
  } else {
    dlo[0] = 0; dhi[0] = a.window_left < 0 ? INT_MAX : a.window_left; rot[0] = MODE == kNope ? 0 : 1;
    dlo[1] = dlo[0]; dhi[1] = dhi[0]; rot[1] = rot[0];
    npass = 1;
  }

  const int spair = tid % NPR;  // pair this thread stages (same for every row it stages)

  float o[DH], q[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) o[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (p >= npass) break;
    const RopeFreq& fp = rot[p] == 2 ? a.fr : a.f;  // the remote pass may use interpolated frequencies
    const uint32_t sflo = fp.lo[spair], sfhi = fp.hi[spair];
    // this lane's slice of the rotated query row for this pass
    const int rq = (valid && MODE != kNope && rot[p]) ? rot_index_f<MODE>(posb[i], rot[p], a) : 0;
#pragma unroll
    for (int e = 0; e < DH / 2; ++e) {
      const int pe = part * (DH / 2) + e;
      float x0 = valid ? qg[size_t(i) * rowq + 2 * pe] : 0.f;
      float x1 = valid ? qg[size_t(i) * rowq + 2 * pe + 1] : 0.f;
      if (MODE != kNope && rot[p]) {
        float s, c;
        rope_sincos(rq, fp.lo[pe], fp.hi[pe], s, c);
        float y0, y1;
        rot_pair(x0, x1, c, s, y0, y1);
        x0 = y0;
        x1 = y1;
      }
      q[2 * e] = x0;
      q[2 * e + 1] = x1;
    }
    const int64_t jlo = max<int64_t>(0, int64_t(P0) - dhi[p]);
    const int64_t jhi = min<int64_t>(S - 1, int64_t(P1) - dlo[p]);
    if (jhi < jlo) continue;
    // this thread's K/V pairs and ids of one tile, loaded a tile ahead
    float2 kr[PAIRS], vr[PAIRS];
    int jid[PAIRS];
    auto load_tile = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int j = j0 + tid / NPR + RPS * u;
        kr[u] = vr[u] = make_float2(0.f, 0.f);
        jid[u] = 0;
        if (j < S) {
          kr[u] = *reinterpret_cast<const float2*>(kg + size_t(j) * rowk + 2 * spair);
          vr[u] = *reinterpret_cast<const float2*>(vg + size_t(j) * rowk + 2 * spair);
          if (MODE != kNope && rot[p]) jid[u] = posb[j];
        }
      }
    };
    const int jfirst = static_cast<int>(jlo / kBNf) * kBNf;
    load_tile(jfirst);
    for (int j0 = jfirst; j0 <= jhi; j0 += kBNf) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int n = tid / NPR + RPS * u;
        float x0 = kr[u].x, x1 = kr[u].y;
        if (MODE != kNope && rot[p] && j0 + n < S) {
          float s, c;
          rope_sincos(rot_index_f<MODE>(jid[u], rot[p], a), sflo, sfhi, s, c);
          float y0, y1;
          rot_pair(x0, x1, c, s, y0, y1);
          x0 = y0;
          x1 = y1;
        }
        Ks[n][2 * spair] = x0;
        Ks[n][2 * spair + 1] = x1;
        Vs[n][2 * spair] = vr[u].x;
        Vs[n][2 * spair + 1] = vr[u].y;
      }
      __syncthreads();
      if (j0 + kBNf <= jhi) load_tile(j0 + kBNf);  // in flight during this tile's math
      float sc[kBNf];
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < kBNf; ++n) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < DH; ++c) acc = fmaf(q[c], Ks[n][part * DH + c], acc);
        acc = row_group_sum<TPR>(acc);
        const int dist = i - (j0 + n);
        const bool keep = dist >= dlo[p] && dist <= dhi[p];
        sc[n] = keep ? acc * sl2 : -INFINITY;
        mx = fmaxf(mx, sc[n]);
      }
      const float mnew = fmaxf(m_run, mx);
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mref);
      m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < DH; ++c) o[c] *= alpha;
#pragma unroll
      for (int n = 0; n < kBNf; ++n) {
        const float pv = __builtin_amdgcn_exp2f(sc[n] - mref);
        l_run += pv;
#pragma unroll
        for (int c = 0; c < DH; ++c) o[c] = fmaf(pv, Vs[n][part * DH + c], o[c]);
      }
    }
  }
  if (!valid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* og = static_cast<float*>(a.o) + size_t(b) * S * rowq + size_t(h) * D + size_t(i) * rowq + part * DH;
#pragma unroll
  for (int c = 0; c < DH; c += 4)
    *reinterpret_cast<float4*>(og + c) = make_float4(o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv);
  if (a.lse && part == 0)
    a.lse[(size_t(b) * a.Hq + h) * S + i] = l_run > 0.f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
}

template <int D, int MODE>
hipError_t launch_f(const PrefillArgs& a0, hipStream_t stream) {
  // rows per workgroup = 256 / (D / 8)
  PrefillArgs a = a0;
  a.BMp = (kThreadsF / (D / 8)) / a.HG;
  a.n_pblocks = (a.S + a.BMp - 1) / a.BMp;
  const int64_t n = int64_t(a.B) * a.Hkv * a.n_hsub * a.n_pblocks;
  hipLaunchKernelGGL((prefill_fp32_kernel<D, MODE>), dim3(static_cast<unsigned>(n)), dim3(kThreadsF), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp32(const PrefillArgs& a, hipStream_t stream) {
  if (a.D == 128) {
    switch (a.mode) {
      case kNope: return launch_f<128, kNope>(a, stream);
      case kRope: return launch_f<128, kRope>(a, stream);
      default: return launch_f<128, kBifocal>(a, stream);
    }
  }
  switch (a.mode) {
    case kNope: return launch_f<64, kNope>(a, stream);
    case kRope: return launch_f<64, kRope>(a, stream);
    default: return launch_f<64, kBifocal>(a, stream);
  }
}

}  // namespace prope
