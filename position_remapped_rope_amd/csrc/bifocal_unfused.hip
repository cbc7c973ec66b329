// Kernels of the unfused bifocal composition (Jet-Long page, section 3.3):
// three ordinary attention calls merged by Eq. (7).
//
//   A: sliding-window attention (i - j <= w0) at the ids p
//   B: full causal attention at the remote ids floor(p / s)
//   C: sliding-window attention (i - j <= w0) at the remote ids
//
// Each call returns O_X and its row log-sum-exp l_X. Per query row, with
// M = max(l_A, l_B, l_C) and W_X = exp(l_X - M), the result is
// (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C), formed in fp32: B and C
// score the window keys identically, so W_B O_B - W_C O_C keeps only the
// remote keys (the inclusion-exclusion step).
//
// remap_ids_kernel writes floor(p / s) (any sign) for the remote calls of the
// aliasing map; with the interpolation map the remote calls rotate at the ids
// themselves with frequencies theta_i / s. eq7_merge_kernel
// is a streaming pass over the three outputs (HBM-bound: it reads three rows
// of d values and writes one per (token, query head)).
#include "internal.hpp"

namespace prope {
namespace {

__global__ __launch_bounds__(256) void remap_ids_kernel(const int32_t* __restrict__ pos, int32_t* __restrict__ out,
                                                        int64_t n, FastDiv s) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = floordiv_s(pos[i], s);
}

// clears the prefill work queue that the three calls share (vector stores)
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int n) {
  const int i = int(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// 8 output elements per thread (bf16: one 16-byte vector; fp32: two).
template <typename T>
struct Vec8 {
  float v[8];
  __device__ __forceinline__ void load(const T* p);
  __device__ __forceinline__ void store(T* p) const;
};
template <>
__device__ __forceinline__ void Vec8<uint16_t>::load(const uint16_t* p) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16_lo(u[e]);
    v[2 * e + 1] = bf16_hi(u[e]);
  }
}
template <>
__device__ __forceinline__ void Vec8<uint16_t>::store(uint16_t* p) const {
  uint4 w;
  w.x = pack_bf16(v[0], v[1]);
  w.y = pack_bf16(v[2], v[3]);
  w.z = pack_bf16(v[4], v[5]);
  w.w = pack_bf16(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = w;
}
template <>
__device__ __forceinline__ void Vec8<float>::load(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void Vec8<float>::store(float* p) const {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// One thread per (batch, token, query head, 8-element chunk). o holds O_B on
// entry and the merged output on exit. Without a local window (w0 = -1) the
// result is O_B and l_B themselves.
template <typename T>
__global__ __launch_bounds__(256) void eq7_merge_kernel(const T* __restrict__ oa, const float* __restrict__ la,
                                                        T* o, const float* __restrict__ lb,
                                                        const T* __restrict__ oc, const float* __restrict__ lc,
                                                        float* __restrict__ lse, int B, int S, int Hq, int d,
                                                        bool windows) {
  const int cpr = d / 8;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(B) * S * Hq * cpr;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % cpr);
  const int64_t row = idx / cpr;  // (b * S + i) * Hq + h
  const int h = static_cast<int>(row % Hq);
  const int64_t bi = row / Hq;
  const int i = static_cast<int>(bi % S);
  const int b = static_cast<int>(bi / S);
  const int64_t li = (int64_t(b) * Hq + h) * S + i;
  const int64_t off = row * d + 8 * c;
  const float lB = lb[li];
  if (!windows) {
    if (lse && c == 0) lse[li] = lB;
    return;  // o already holds O_B
  }
  const float lA = la[li], lC = lc[li];
  const float M = fmaxf(lA, fmaxf(lB, lC));
  const float wa = expf(lA - M), wb = expf(lB - M), wc = expf(lC - M);
  // B - C first: exactly zero where the remote calls saw the same keys
  const float den = wa + (wb - wc);
  const float inv = 1.f / den;
  Vec8<T> A, Bv, C;
  A.load(oa + off);
  Bv.load(o + off);
  C.load(oc + off);
#pragma unroll
  for (int e = 0; e < 8; ++e) Bv.v[e] = (wa * A.v[e] + (wb * Bv.v[e] - wc * C.v[e])) * inv;
  Bv.store(o + off);
  if (lse && c == 0) lse[li] = M + logf(den);
}

}  // namespace

hipError_t launch_remap_ids(const int32_t* pos, int32_t* out, int64_t n, const FastDiv& s, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(remap_ids_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, pos, out, n, s);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_eq7_merge(const void* oa, const float* la, void* o, const float* lb, const void* oc,
                            const float* lc, float* lse, int B, int S, int Hq, int d, int dt, bool windows,
                            hipStream_t stream) {
  const int64_t total = int64_t(B) * S * Hq * (d / 8);
  const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
  if (dt == 0)
    hipLaunchKernelGGL((eq7_merge_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(oa), la, static_cast<uint16_t*>(o), lb,
                       static_cast<const uint16_t*>(oc), lc, lse, B, S, Hq, d, windows);
  else
    hipLaunchKernelGGL((eq7_merge_kernel<float>), dim3(blocks), dim3(256), 0, stream,
                       static_cast<const float*>(oa), la, static_cast<float*>(o), lb,
                       static_cast<const float*>(oc), lc, lse, B, S, Hq, d, windows);
  return hipGetLastError();
}

}  // namespace prope
