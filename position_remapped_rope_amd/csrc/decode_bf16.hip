// Split-K decode against a KV cache of base-rotated keys (bf16), HBM-bound.
//
// Jet-Long page, section 3.2: the cache keeps k_cache[j] = RoPE(x_j, j)
// (Eq. (4)) and is never rewritten. For a query at p_q = kv_len - 1, a key at
// distance p_q - j <= w0 scores with the cached vectors as they are; a farther
// key scores with the remote view RoPE(q, dq) . RoPE(k_j, dk_j), where
// dq = floor(p_q/s) - p_q and dk_j = floor(j/s) - j (Eq. (5)-(6)). Both
// corrections are formed in registers from exact integer phases; nothing is
// written back. NOPE/ROPE caches already carry their rotation, so those modes
// score q . k_j with an optional window.
//
// Kernel 1 (split): one workgroup per (chunk of kDecodeChunk keys, KV head,
// sequence). 16 lanes cover one key's 128 dims (16 B each, coalesced 256-byte
// rows); the workgroup keeps 16 keys in flight per step, 4 steps unrolled so
// each lane has 8 independent 16-byte loads outstanding. Every key is scored
// against all G query heads of its KV group (G-fold reuse of each loaded byte).
// Partial softmax statistics (row max m, row sum l, unnormalised O) are
// merged across lane groups in LDS and written to the workspace.
// Kernel 2 (combine): per (sequence, query head) the chunk partials are
// merged with log-sum-exp weights (Jet-Long Eq. (7)'s merge with only
// disjoint parts) into O and the LSE.
#include "internal.hpp"

namespace prope {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDThreads = 256;
constexpr int kUnroll = 4;

template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = LPK / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <int D, int MODE, int GM>
__global__ __launch_bounds__(kDThreads) void decode_split_kernel(const DecodeArgs a) {
  constexpr int LPK = D / 8;                 // lanes per key
  constexpr int GROUPS = kDThreads / LPK;    // keys in flight per step
  __shared__ float red_m[GROUPS][GM];
  __shared__ float red_l[GROUPS][GM];
  __shared__ float red_o[GROUPS][GM][D];

  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, c = tid % LPK, grp = tid / LPK;
  const int G = a.G;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);  // a length outside [0, Lmax] never reads past the cache
  const int jbeg = chunk * kDecodeChunk;
  const size_t head_stride = size_t(a.n_chunks) * (D + 2);
  float* wsb = a.ws + (size_t(b) * a.Hq + size_t(kvh) * G) * head_stride + size_t(chunk) * (D + 2);

  if (jbeg >= L) {  // chunk past this sequence's length: an empty partial
    if (tid < G) {
      wsb[tid * head_stride] = -INFINITY;
      wsb[tid * head_stride + 1] = 0.f;
    }
    return;
  }
  const int jend = min(L, jbeg + kDecodeChunk);
  const int pq = L - 1;
  const float sl2 = a.scale_log2;

  // query slice (dims c*8 .. c*8+7) of every head in the group, local and remote views
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + (size_t(b) * a.Hq + size_t(kvh) * G) * D + c * 8;
  float ql[GM][8], qr[GM][8];
  uint32_t flo[4], fhi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    flo[e] = a.f.lo[c * 4 + e];
    fhi[e] = a.f.hi[c * 4 + e];
  }
  const int dq = MODE == kBifocal ? static_cast<int>(fastdiv(static_cast<uint32_t>(pq), a.scale_div)) - pq : 0;
  float qs[4], qc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) rope_sincos(dq, flo[e], fhi[e], qs[e], qc[e]);
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    u32x4_t w = {0, 0, 0, 0};
    if (g < G) w = *reinterpret_cast<const u32x4_t*>(qg + size_t(g) * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ql[g][2 * e] = bf16_lo(w[e]);
      ql[g][2 * e + 1] = bf16_hi(w[e]);
      rot_pair(ql[g][2 * e], ql[g][2 * e + 1], qc[e], qs[e], qr[g][2 * e], qr[g][2 * e + 1]);
    }
  }

  float m_run[GM], l_run[GM], o[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }

  const size_t rowk = size_t(a.Hkv) * D;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + size_t(b) * a.Lmax * rowk + size_t(kvh) * D + c * 8;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + size_t(b) * a.Lmax * rowk + size_t(kvh) * D + c * 8;
  const int w0 = a.window_left;

  for (int jb = jbeg + grp; jb < jend; jb += GROUPS * kUnroll) {
    u32x4_t kw[kUnroll], vw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + GROUPS * u;
      const bool ok = j < jend;
      kw[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kg + size_t(j) * rowk)) : u32x4_t{0, 0, 0, 0};
      vw[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vg + size_t(j) * rowk)) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + GROUPS * u;
      if (j >= jend) break;  // uniform within the 16-lane group
      float kx[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kx[2 * e] = bf16_lo(kw[u][e]);
        kx[2 * e + 1] = bf16_hi(kw[u][e]);
      }
      const int dist = pq - j;
      bool remote = false;
      bool keep = true;
      if (MODE == kBifocal) {
        remote = dist > w0;
      } else if (w0 >= 0) {
        keep = dist <= w0;
      }
      if (remote) {
        const int dk = static_cast<int>(fastdiv(static_cast<uint32_t>(j), a.scale_div)) - j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s, cs, y0, y1;
          rope_sincos(dk, flo[e], fhi[e], s, cs);
          rot_pair(kx[2 * e], kx[2 * e + 1], cs, s, y0, y1);
          kx[2 * e] = y0;
          kx[2 * e + 1] = y1;
        }
      }
      float vx[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vx[2 * e] = bf16_lo(vw[u][e]);
        vx[2 * e + 1] = bf16_hi(vw[u][e]);
      }
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        if (g >= G) break;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(remote ? qr[g][e] : ql[g][e], kx[e], part);
        const float sc = keep ? group_sum<LPK>(part) * sl2 : -INFINITY;
        const float mnew = fmaxf(m_run[g], sc);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m_run[g] - mref);
        const float pv = __builtin_amdgcn_exp2f(sc - mref);
        m_run[g] = mnew;
        l_run[g] = fmaf(l_run[g], alpha, pv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = fmaf(o[g][e], alpha, pv * vx[e]);
      }
    }
  }

  // merge the lane groups' partials
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g >= G) break;
    if (c == 0) {
      red_m[grp][g] = m_run[g];
      red_l[grp][g] = l_run[g];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[grp][g][c * 8 + e] = o[g][e];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kDThreads) {
    const int g = idx / D, dd = idx % D;
    float M = -INFINITY;
    for (int r = 0; r < GROUPS; ++r) M = fmaxf(M, red_m[r][g]);
    const float Mref = M == -INFINITY ? 0.f : M;
    float acc = 0.f, lsum = 0.f;
    for (int r = 0; r < GROUPS; ++r) {
      const float w = __builtin_amdgcn_exp2f(red_m[r][g] - Mref);
      acc = fmaf(w, red_o[r][g][dd], acc);
      lsum = fmaf(w, red_l[r][g], lsum);
    }
    float* dst = wsb + size_t(g) * head_stride;
    dst[2 + dd] = acc;
    if (dd == 0) {
      dst[0] = M;
      dst[1] = lsum;
    }
  }
}

// One workgroup per (query head, sequence). Threads split the chunk partials
// (max, sum) and, for O, pairs of (chunk group, 4 dims), then reduce in LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeArgs a) {
  constexpr int NT = 256;
  constexpr int DV = D / 4;       // float4 columns per partial
  constexpr int CG = NT / DV;     // chunk groups for the O reduction
  __shared__ float red[NT];
  __shared__ float4 ored[CG][DV];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);
  const int nc = (L + kDecodeChunk - 1) / kDecodeChunk;
  const size_t stride = D + 2;
  const float* wsb = a.ws + (size_t(b) * a.Hq + h) * size_t(a.n_chunks) * stride;

  float mx = -INFINITY;
  for (int c = tid; c < nc; c += NT) mx = fmaxf(mx, wsb[size_t(c) * stride]);
  red[tid] = mx;
  __syncthreads();
  for (int off = NT / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  const float M = red[0];
  const float Mref = M == -INFINITY ? 0.f : M;
  __syncthreads();

  float ls = 0.f;
  for (int c = tid; c < nc; c += NT)
    ls = fmaf(__builtin_amdgcn_exp2f(wsb[size_t(c) * stride] - Mref), wsb[size_t(c) * stride + 1], ls);
  red[tid] = ls;
  __syncthreads();
  for (int off = NT / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const float lsum = red[0];

  const int dv = tid % DV, cg = tid / DV;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int c = cg; c < nc; c += CG) {
    const float* part = wsb + size_t(c) * stride;
    const float w = __builtin_amdgcn_exp2f(part[0] - Mref);
    // partial O starts at float offset 2: read as two float2 to stay 8-byte aligned
    const float2 x0 = *reinterpret_cast<const float2*>(part + 2 + 4 * dv);
    const float2 x1 = *reinterpret_cast<const float2*>(part + 4 + 4 * dv);
    acc.x = fmaf(w, x0.x, acc.x);
    acc.y = fmaf(w, x0.y, acc.y);
    acc.z = fmaf(w, x1.x, acc.z);
    acc.w = fmaf(w, x1.y, acc.w);
  }
  ored[cg][dv] = acc;
  __syncthreads();
  if (tid < DV) {
    float4 t = ored[0][tid];
    for (int g = 1; g < CG; ++g) {
      t.x += ored[g][tid].x;
      t.y += ored[g][tid].y;
      t.z += ored[g][tid].z;
      t.w += ored[g][tid].w;
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint2 packed;
    packed.x = pack_bf16(t.x * inv, t.y * inv);
    packed.y = pack_bf16(t.z * inv, t.w * inv);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + (size_t(b) * a.Hq + h) * D + 4 * tid) = packed;
  }
  if (a.lse && tid == 0)
    a.lse[size_t(b) * a.Hq + h] = lsum > 0.f ? (M + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
}

template <int D, int MODE, int GM>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, MODE, GM>), dim3(a.n_chunks, a.Hkv, a.B), dim3(kDThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.Hq, a.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t stream) {
  if (a.G <= 1) return launch_d<D, MODE, 1>(a, stream);
  if (a.G <= 2) return launch_d<D, MODE, 2>(a, stream);
  if (a.G <= 4) return launch_d<D, MODE, 4>(a, stream);
  return launch_d<D, MODE, 8>(a, stream);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.D == 128) {
    switch (a.mode) {
      case kNope: return launch_dg<128, kNope>(a, stream);
      case kRope: return launch_dg<128, kRope>(a, stream);
      default: return launch_dg<128, kBifocal>(a, stream);
    }
  }
  switch (a.mode) {
    case kNope: return launch_dg<64, kNope>(a, stream);
    case kRope: return launch_dg<64, kRope>(a, stream);
    default: return launch_dg<64, kBifocal>(a, stream);
  }
}

}  // namespace prope
