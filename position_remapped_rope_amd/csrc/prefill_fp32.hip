// float32 prefill: same scores, masks and bifocal routing as the bf16 kernel,
// computed with fp32 vector ALU (no operand rounding). Meant for small fp32
// problems such as the EndPrompt two-segment check; the bf16 MFMA kernel is
// the throughput path.
//
// A workgroup of 8 waves owns a few query rows (64 / (D/8) of them: D/8
// adjacent lanes share a row, 8 dims each) and splits their keys: wave w takes
// every 8th 16-key tile of each pass, stages it (K rotated in fp32) in its own
// LDS slot, and keeps its own softmax statistics (m, l, O) for the rows. The
// 8 partial states are merged once at the end (the log-sum-exp algebra of
// Jet-Long Eq. (7) with disjoint parts). With the keys split this way a
// row's tiles run 8 at a time instead of one after another: a short problem
// is bound by the latency of its longest rows' tile loop, at one wave per SIMD.
// ALiBi slopes (NOPE/ROPE), when given, subtract m_h (i - j) from each scaled
// score (P-RoPE page, section 1).
#include <limits.h>

#include "internal.hpp"

namespace prope {
namespace {

constexpr int kBNf = 16;         // keys per tile
constexpr int kWavesF = 8;       // key groups per workgroup
constexpr int kThreadsF = 64 * kWavesF;

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
  if (rot == 2) return floordiv_s(p, a.scale_div);
  if (MODE == kRope) return a.period > 0 ? floormod_s(p, a.period_div) : p;
  return p;
}

// A workgroup covers RPW = 64 / TPR rows (HG heads x BMp = RPW / HG positions,
// set by the launcher); each of its 8 waves holds all of them.
template <int D, int MODE>
__global__ __launch_bounds__(kThreadsF) void prefill_fp32_kernel(const PrefillArgs a) {
  constexpr int DH = 8;                  // dims per lane
  constexpr int TPR = D / DH;            // lanes per query row
  constexpr int RPW = 64 / TPR;          // rows per workgroup (every wave holds them all)
  constexpr int NPR = D / 2;             // pairs per key row
  constexpr int PAIRS = kBNf * NPR / 64; // pairs a lane stages per tile
  constexpr int KPS = 64 / NPR;          // keys one staging sweep of the wave covers
  __shared__ __attribute__((aligned(16))) float Ks[kWavesF][kBNf][D];
  __shared__ __attribute__((aligned(16))) float Vs[kWavesF][kBNf][D];
  __shared__ float red_m[kWavesF][RPW], red_l[kWavesF][RPW];
  __shared__ __attribute__((aligned(16))) float red_o[kWavesF][RPW][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane / TPR, part = lane % TPR;
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

  const int spair = lane % NPR;  // pair this lane stages (the same in every key it stages)
  float (*ks)[D] = Ks[wave];
  float (*vs)[D] = Vs[wave];

  float o[DH], q[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) o[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;
  // ALiBi slope of this row's head, log2 units (0 without ALiBi: the bias term vanishes)
  const float slope2 = (MODE != kBifocal && a.alibi) ? a.alibi[h] * 1.4426950408889634f : 0.f;

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
    // this wave's tiles of the pass: every kWavesF-th, starting at tile `wave`
    const int t_first = static_cast<int>(jlo / kBNf), t_last = static_cast<int>(jhi / kBNf);
    // this lane's K/V pairs and ids of one tile, loaded a tile ahead
    float2 kr[PAIRS], vr[PAIRS];
    int jid[PAIRS];
    auto load_tile = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int j = j0 + u * KPS + lane / NPR;
        kr[u] = vr[u] = make_float2(0.f, 0.f);
        jid[u] = 0;
        if (j < S) {
          kr[u] = *reinterpret_cast<const float2*>(kg + size_t(j) * rowk + 2 * spair);
          vr[u] = *reinterpret_cast<const float2*>(vg + size_t(j) * rowk + 2 * spair);
          if (MODE != kNope && rot[p]) jid[u] = posb[j];
        }
      }
    };
    int t = t_first + wave;
    if (t <= t_last) load_tile(t * kBNf);
    for (; t <= t_last; t += kWavesF) {
      const int j0 = t * kBNf;
      // stage this tile in the wave's own LDS slot (the wave alone reads it,
      // and its LDS operations complete in order: no workgroup barrier)
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int n = u * KPS + lane / NPR;
        float x0 = kr[u].x, x1 = kr[u].y;
        if (MODE != kNope && rot[p] && j0 + n < S) {
          float s, c;
          rope_sincos(rot_index_f<MODE>(jid[u], rot[p], a), sflo, sfhi, s, c);
          float y0, y1;
          rot_pair(x0, x1, c, s, y0, y1);
          x0 = y0;
          x1 = y1;
        }
        ks[n][2 * spair] = x0;
        ks[n][2 * spair + 1] = x1;
        vs[n][2 * spair] = vr[u].x;
        vs[n][2 * spair + 1] = vr[u].y;
      }
      if (t + kWavesF <= t_last) load_tile((t + kWavesF) * kBNf);  // in flight during this tile's math
      float sc[kBNf];
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < kBNf; ++n) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < DH; ++c) acc = fmaf(q[c], ks[n][part * DH + c], acc);
        acc = row_group_sum<TPR>(acc);
        const int dist = i - (j0 + n);
        const bool keep = dist >= dlo[p] && dist <= dhi[p] && j0 + n < S;
        sc[n] = keep ? fmaf(acc, sl2, -slope2 * static_cast<float>(dist)) : -INFINITY;
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
        for (int c = 0; c < DH; ++c) o[c] = fmaf(pv, vs[n][part * DH + c], o[c]);
      }
    }
  }

  // merge the 8 waves' statistics of each row
  if (part == 0) {
    red_m[wave][row] = m_run;
    red_l[wave][row] = l_run;
  }
#pragma unroll
  for (int c = 0; c < DH; ++c) red_o[wave][row][part * DH + c] = o[c];
  __syncthreads();
  for (int idx = tid; idx < RPW * D; idx += kThreadsF) {
    const int r = idx / D, dd = idx % D;
    const int hr = r / a.BMp;
    const int ir = P0 + r - hr * a.BMp;
    if (ir >= S) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesF; ++w) M = fmaxf(M, red_m[w][r]);
    const float Mref = M == -INFINITY ? 0.f : M;
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesF; ++w) {
      const float wt = __builtin_amdgcn_exp2f(red_m[w][r] - Mref);
      acc = fmaf(wt, red_o[w][r][dd], acc);
      lsum = fmaf(wt, red_l[w][r], lsum);
    }
    const int hr_head = kvh * a.G + hsub * a.HG + hr;
    float* og = static_cast<float*>(a.o) + size_t(b) * S * rowq + size_t(hr_head) * D + size_t(ir) * rowq;
    og[dd] = lsum > 0.f ? acc / lsum : 0.f;
    if (a.lse && dd == 0)
      a.lse[(size_t(b) * a.Hq + hr_head) * S + ir] = lsum > 0.f ? (M + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
  }
}

// rows per workgroup = 64 / (D / 8), split over HG heads
PrefillArgs fp32_args(const PrefillArgs& a0) {
  PrefillArgs a = a0;
  a.BMp = (64 / (a.D / 8)) / a.HG;
  a.n_pblocks = (a.S + a.BMp - 1) / a.BMp;
  return a;
}

int64_t n_blocks(const PrefillArgs& a) { return int64_t(a.B) * a.Hkv * a.n_hsub * a.n_pblocks; }

template <int D, int MODE>
hipError_t launch_f(const PrefillArgs& a0, hipStream_t stream) {
  const PrefillArgs a = fp32_args(a0);
  const int64_t n = n_blocks(a);
  hipLaunchKernelGGL((prefill_fp32_kernel<D, MODE>), dim3(static_cast<unsigned>(n)), dim3(kThreadsF), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

bool prefill_fp32_fits(const PrefillArgs& a) { return n_blocks(fp32_args(a)) * kThreadsF <= kMaxWorkItems; }

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
