// y = R_pos x (P-RoPE page, section 3.1, Eq. (2)), streaming, HBM-bound.
//
// One thread owns one token and a chunk of VEC adjacent coordinates (VEC/2
// rotation pairs): it forms the pairs' sin/cos once from the token's id and
// reuses them for every head of the token, so the transcendental work is
// amortised H times. Loads and stores are 16-byte vectors; consecutive
// threads walk consecutive chunks of a row, so a wavefront touches whole
// 256-byte rows of each head.
#include "internal.hpp"

namespace prope {

template <typename T, int VEC>
struct VecIO;

template <>
struct VecIO<uint16_t, 8> {  // 8 bf16 = 16 B
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(ws[i]);
      x[2 * i + 1] = bf16_hi(ws[i]);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* y) {
    uint4 w;
    w.x = pack_bf16(y[0], y[1]);
    w.y = pack_bf16(y[2], y[3]);
    w.z = pack_bf16(y[4], y[5]);
    w.w = pack_bf16(y[6], y[7]);
    *reinterpret_cast<uint4*>(p) = w;
  }
};

template <>
struct VecIO<uint16_t, 2> {  // one pair
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    x[0] = bf16_lo(w);
    x[1] = bf16_hi(w);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* y) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16(y[0], y[1]);
  }
};

template <>
struct VecIO<float, 8> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* y) {
    reinterpret_cast<float4*>(p)[0] = make_float4(y[0], y[1], y[2], y[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(y[4], y[5], y[6], y[7]);
  }
};

template <>
struct VecIO<float, 2> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    x[0] = a.x;
    x[1] = a.y;
  }
  static __device__ __forceinline__ void store(float* p, const float* y) {
    *reinterpret_cast<float2*>(p) = make_float2(y[0], y[1]);
  }
};

template <typename T, int VEC>
__global__ __launch_bounds__(256) void rope_apply_kernel(const T* __restrict__ x, T* y,
                                                         const int32_t* __restrict__ pos,
                                                         int64_t n_tokens, int H, int d,
                                                         RopeFreq f) {
  constexpr int NP = VEC / 2;
  constexpr int kHeads = 8;
  const int cpr = d / VEC;  // chunks per row
  const int64_t n_items = n_tokens * cpr;
  for (int64_t item = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; item < n_items;
       item += int64_t(gridDim.x) * blockDim.x) {
    const int64_t tok = item / cpr;
    const int c = static_cast<int>(item - tok * cpr);
    const int32_t p = pos[tok];
    float sn[NP], cs[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) rope_sincos(p, f.lo[c * NP + i], f.hi[c * NP + i], sn[i], cs[i]);
    const int64_t base = tok * H * int64_t(d) + c * VEC;
    auto rotate_store = [&](int h, const float* v) {
      float r[VEC];
#pragma unroll
      for (int i = 0; i < NP; ++i) rot_pair(v[2 * i], v[2 * i + 1], cs[i], sn[i], r[2 * i], r[2 * i + 1]);
      VecIO<T, VEC>::store(y + base + int64_t(h) * d, r);
    };
    // whole groups of kHeads heads: all of a group's loads go out before the
    // first rotation, so a thread keeps kHeads requests in flight
    int h = 0;
    for (; h + kHeads <= H; h += kHeads) {
      float v[kHeads][VEC];
#pragma unroll
      for (int u = 0; u < kHeads; ++u) VecIO<T, VEC>::load(x + base + int64_t(h + u) * d, v[u]);
#pragma unroll
      for (int u = 0; u < kHeads; ++u) rotate_store(h + u, v[u]);
    }
    for (; h < H; ++h) {  // the rest, one head at a time
      float v[VEC];
      VecIO<T, VEC>::load(x + base + int64_t(h) * d, v);
      rotate_store(h, v);
    }
  }
}

template <typename T, int VEC>
static hipError_t launch_rope_t(const void* x, void* y, const int32_t* pos, int64_t n_tokens,
                                int H, int d, const RopeFreq& f, hipStream_t stream) {
  const int64_t items = n_tokens * (d / VEC);
  const int64_t want = (items + 255) / 256;
  const int grid = static_cast<int>(want < 256 * 32 ? want : 256 * 32);
  hipLaunchKernelGGL((rope_apply_kernel<T, VEC>), dim3(grid), dim3(256), 0, stream,
                     static_cast<const T*>(x), static_cast<T*>(y), pos, n_tokens, H, d, f);
  return hipGetLastError();
}

hipError_t launch_rope_apply(const void* x, void* y, const int32_t* pos, int B, int S, int H,
                             int d, int dt, const RopeFreq& f, hipStream_t stream) {
  const int64_t n_tokens = int64_t(B) * S;
  const bool v8 = (d % 8) == 0;
  if (dt == 0) {
    return v8 ? launch_rope_t<uint16_t, 8>(x, y, pos, n_tokens, H, d, f, stream)
              : launch_rope_t<uint16_t, 2>(x, y, pos, n_tokens, H, d, f, stream);
  }
  return v8 ? launch_rope_t<float, 8>(x, y, pos, n_tokens, H, d, f, stream)
            : launch_rope_t<float, 2>(x, y, pos, n_tokens, H, d, f, stream);
}

}  // namespace prope
