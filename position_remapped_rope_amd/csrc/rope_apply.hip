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
  using Raw = uint4;
  static __device__ __forceinline__ Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ void unpack(const Raw& w, float* x) {
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
  using Raw = uint32_t;
  static __device__ __forceinline__ Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
  static __device__ __forceinline__ void unpack(const Raw& w, float* x) {
    x[0] = bf16_lo(w);
    x[1] = bf16_hi(w);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* y) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16(y[0], y[1]);
  }
};

template <>
struct VecIO<float, 8> {
  struct Raw {
    float4 a, b;
  };
  static __device__ __forceinline__ Raw load_raw(const float* p) {
    return Raw{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  static __device__ __forceinline__ void unpack(const Raw& w, float* x) {
    const float4 a = w.a, b = w.b;
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
  using Raw = float2;
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *reinterpret_cast<const float2*>(p); }
  static __device__ __forceinline__ void unpack(const Raw& a, float* x) {
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
    const int64_t base = tok * H * int64_t(d) + c * VEC;
    // the id and the pair frequencies first, then whole groups of kHeads
    // heads: all of a group's loads go out before the first rotation, so a
    // thread keeps kHeads requests in flight, and the first group's loads are
    // issued before the sin/cos, which wait only for the id and frequencies
    // (loads complete in order)
    const int32_t p = pos[tok];
    uint32_t flo[NP], fhi[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      flo[i] = f.lo[c * NP + i];
      fhi[i] = f.hi[c * NP + i];
    }
    typename VecIO<T, VEC>::Raw v[kHeads];
    auto load_group = [&](int h) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kHeads; ++u) v[u] = VecIO<T, VEC>::load_raw(x + base + int64_t(h + u) * d);
    };
    float sn[NP], cs[NP];
    auto angles = [&](int32_t r) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NP; ++i) rope_sincos(r, flo[i], fhi[i], sn[i], cs[i]);
    };
    auto rotate_store = [&](int h, const typename VecIO<T, VEC>::Raw& w) {
      float xv[VEC], r[VEC];
      VecIO<T, VEC>::unpack(w, xv);
#pragma unroll
      for (int i = 0; i < NP; ++i) rot_pair(xv[2 * i], xv[2 * i + 1], cs[i], sn[i], r[2 * i], r[2 * i + 1]);
      VecIO<T, VEC>::store(y + base + int64_t(h) * d, r);
    };
    int h = 0;
    if (H >= kHeads) {  // (one straight block from the loads to the sin/cos, so their wait is exact)
      load_group(0);
      // the id passes through an empty asm after the loads, so that the
      // compiler cannot hoist its phase arithmetic (and the wait for it)
      // above them
      int32_t r = p;
      asm volatile("" : "+v"(r));
      angles(r);
      for (; h + kHeads <= H; h += kHeads) {
        if (h > 0) load_group(h);
#pragma unroll
        for (int u = 0; u < kHeads; ++u) rotate_store(h + u, v[u]);
      }
    } else {
      angles(p);
    }
    for (; h < H; ++h)  // the rest, one head at a time
      rotate_store(h, VecIO<T, VEC>::load_raw(x + base + int64_t(h) * d));
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
