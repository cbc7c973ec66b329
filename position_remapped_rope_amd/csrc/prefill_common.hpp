// Device helpers shared by the bf16 prefill kernels (gfx950): MFMA and
// buffer-load wrappers, the transposing LDS read, rotation indices, and the
// work-item queue of the persistent launch.
#pragma once

#include "internal.hpp"

namespace prope {
namespace pf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

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

// Rotation index of id p for rotation kind rot: 2 = remote ids floor(p / s)
// (Jet-Long Eq. (3)), 1 = base ids (p mod P with a period, P-RoPE Eq. (4)).
template <int MODE>
__device__ __forceinline__ int rot_index(int p, int rot, const PrefillArgs& a) {
  if (rot == 2) return floordiv_s(p, a.scale_div);
  if (MODE == kRope) return a.period > 0 ? floormod_s(p, a.period_div) : p;
  return p;
}

// ---- work items ---------------------------------------------------------
// An item is (sequence, KV head, head subgroup, row block). Without a queue
// every workgroup runs the one item blockIdx names. With a queue the grid is
// persistent and items come from 8 queues, one per XCD (blockIdx % 8 is the
// XCD a workgroup runs on): queue x holds the x-th contiguous eighth of the
// items (whole head groups when possible, so its K/V tiles stay in that XCD's
// L2), handed out heaviest row block first. A workgroup whose own queue is
// empty takes items from the others. The XCDs run at different speeds, so a
// fixed split of the items over them leaves the fast ones idle at the end.
struct ItemQueue {
  uint32_t* wq;
  int n_items, q8, r8, npb, home;
  bool first;

  __device__ __forceinline__ ItemQueue(const PrefillArgs& a)
      : wq(a.queue), n_items(a.B * a.Hkv * a.n_hsub * a.n_pblocks), npb(a.n_pblocks),
        home(int(blockIdx.x) & 7), first(true) {
    q8 = n_items / 8;
    r8 = n_items % 8;
  }
  __device__ __forceinline__ int q_start(int x) const { return x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8; }
  __device__ __forceinline__ int q_len(int x) const { return q8 + (x < r8 ? 1 : 0); }
  // item of the k-th claim on queue x: a queue made of whole head groups goes
  // row block major across its groups, heaviest (last) row block first
  __device__ __forceinline__ int q_item(int x, int k) const {
    const int st = q_start(x), len = q_len(x);
    if (st % npb == 0 && len % npb == 0) {
      const int ng = len / npb;
      return st + (k % ng) * npb + k / ng;
    }
    return st + k;
  }
  // each queue's first claims are static (rank blockIdx / 8 among the
  // workgroups of that XCD); its counter counts the claims after those
  __device__ __forceinline__ int q_static(int x) const {
    return int(gridDim.x) / 8 + (x < int(gridDim.x) % 8 ? 1 : 0);
  }
  // The next item of this workgroup, or -1. Run by one whole wave; the result is
  // valid in every lane.
  __device__ __forceinline__ int next(int lane) {
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
  }
  // Queue clean-up, by one wave after the workgroup's last item: each workgroup
  // counts itself done on its XCD's counter, the last of each XCD on the global
  // one, and the very last puts every counter back to 0, so the buffer is ready
  // for the next launch.
  __device__ __forceinline__ void finish(int lane) {
    if (!wq) return;
    uint32_t last = 0;
    if (lane == 0) {
      const uint32_t dn = atomicAdd(&wq[kQueueLine * (8 + home)], 1u);
      if (dn == uint32_t(q_static(home)) - 1)
        last = atomicAdd(&wq[kQueueLine * 16], 1u) == uint32_t(min(8, int(gridDim.x))) - 1;
    }
    last = __shfl(last, 0);
    if (last && lane < 17) atomicExch(&wq[kQueueLine * lane], 0u);
  }
};

}  // namespace pf
}  // namespace prope
