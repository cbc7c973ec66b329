// Shared device helpers for the remapped-position RoPE kernels (gfx950).
//
// RoPE angle (P-RoPE page, section 3.1, Eq. (1)-(2)): pair i of a vector at
// rotation index r turns by r * theta_i, theta_i = base^(-2i/d). A float32
// product r * theta_i loses ~1e-2 rad at r ~ 1.3e5, so the angle is formed
// from an exact fixed-point phase instead: F_i = round(theta_i / (2 pi) * 2^64)
// (host, long double), and the turn count r * F_i mod 2^64 is computed with
// integer multiplies; its top 32 bits give the angle in turns in [-1/2, 1/2),
// which the hardware sine/cosine (argument in revolutions) consume directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prope {

constexpr int kMaxPairs = 128;  // rope_apply supports d <= 256; attention d <= 128

// Per-pair phase increments, 64-bit fixed-point turns per unit of id, split in
// 32-bit halves. Passed by value as a kernel argument (1 KiB).
struct RopeFreq {
  uint32_t lo[kMaxPairs];
  uint32_t hi[kMaxPairs];
};

// Top 32 bits of (r * F) mod 2^64: the phase in units of 2^-32 turn. Works for
// negative r (two's complement sign extension of r to 64 bits: the unsigned
// product of r + 2^32 carries an extra 2^32 * F, whose top half is flo).
__device__ __forceinline__ uint32_t phase_top(int32_t r, uint32_t flo, uint32_t fhi) {
  const uint32_t ru = static_cast<uint32_t>(r);
  const uint32_t sgn = static_cast<uint32_t>(r >> 31);  // all ones iff r < 0
  return __umulhi(ru, flo) + ru * fhi - (flo & sgn);
}

// The same phase from F split with a SIGNED low half: F = fhs * 2^32 + fls, fls
// in [-2^31, 2^31) (fls = flo - 2^32 and fhs = fhi + 1 when flo >= 2^31). Then
// the signed 64-bit product r * fls carries the sign of r by itself, and the top
// 32 bits of (r * F) mod 2^64 are r * fhs + hi32(r * fls): one signed high
// multiply, one low multiply and an add, no sign correction.
struct PhaseSplit {
  uint32_t fls;  // the signed low half, as bits
  uint32_t fhs;
};
__host__ __device__ inline PhaseSplit phase_split(uint32_t flo, uint32_t fhi) {
  return PhaseSplit{flo, fhi + (flo >> 31)};
}
__host__ __device__ inline uint32_t phase_top_split(int32_t r, uint32_t fls, uint32_t fhs) {
  const int32_t hi = static_cast<int32_t>((int64_t(r) * int64_t(static_cast<int32_t>(fls))) >> 32);
  return static_cast<uint32_t>(hi) + static_cast<uint32_t>(r) * fhs;
}

// sin and cos of 2*pi*t for t in [-1/2, 1/2) (v_sin_f32 / v_cos_f32 take revolutions).
__device__ __forceinline__ void sincos_turns(float t, float& s, float& c) {
  s = __builtin_amdgcn_sinf(t);
  c = __builtin_amdgcn_cosf(t);
}

// The same phase as a signed fraction of a turn in [-1/2, 1/2).
__device__ __forceinline__ float phase_turns(int32_t r, uint32_t flo, uint32_t fhi) {
  return static_cast<float>(static_cast<int32_t>(phase_top(r, flo, fhi))) * 0x1p-32f;
}

// sin/cos of a phase held as 2^-32 turn units
__device__ __forceinline__ void phase_sincos(uint32_t ph, float& s, float& c) {
  sincos_turns(static_cast<float>(static_cast<int32_t>(ph)) * 0x1p-32f, s, c);
}

__device__ __forceinline__ void rope_sincos(int32_t r, uint32_t flo, uint32_t fhi, float& s,
                                            float& c) {
  sincos_turns(phase_turns(r, flo, fhi), s, c);
}

// rope_sincos from the signed split of F (phase_split)
__device__ __forceinline__ void rope_sincos_split(int32_t r, uint32_t fls, uint32_t fhs, float& s, float& c) {
  sincos_turns(static_cast<float>(static_cast<int32_t>(phase_top_split(r, fls, fhs))) * 0x1p-32f, s, c);
}

// ---- bf16 bit helpers ---------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (a in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = static_cast<__bf16>(a);
  v.y = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}

// Rotate one packed bf16 pair word (x_{2i} low, x_{2i+1} high) by (c, s); returns floats.
__device__ __forceinline__ void rot_pair(float x0, float x1, float c, float s, float& y0,
                                         float& y1) {
  y0 = c * x0 - s * x1;
  y1 = s * x0 + c * x1;
}

// ---- division by an invariant integer ---------------------------------
// Round-up multiply-shift division (Granlund and Montgomery, "Division by
// Invariant Integers using Multiplication", PLDI 1994): for 1 <= d < 2^31 and
// 0 <= n < 2^31, n / d == (umulhi(n, magic) + n) >> shift.
struct FastDiv {
  uint32_t magic;
  uint32_t shift;
  uint32_t div;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.div = d;
  f.shift = 0;
  while ((1u << f.shift) < d) ++f.shift;
  f.magic = static_cast<uint32_t>(((uint64_t(1) << 32) * ((uint64_t(1) << f.shift) - d)) / d + 1);
  return f;
}

__host__ __device__ inline uint32_t umulhi32(uint32_t a, uint32_t b) {
  return static_cast<uint32_t>((static_cast<uint64_t>(a) * b) >> 32);
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  return (umulhi32(n, f.magic) + n) >> f.shift;
}

__host__ __device__ inline uint32_t fastmod(uint32_t n, const FastDiv& f) {
  return n - fastdiv(n, f) * f.div;
}

// floor(n / d) for any int32 n: for n < 0 the complement ~n = -n - 1 is in
// [0, 2^31), and floor(n / d) = ~floor(~n / d).
__host__ __device__ inline int32_t floordiv_s(int32_t n, const FastDiv& f) {
  const uint32_t sgn = static_cast<uint32_t>(n >> 31);
  return static_cast<int32_t>(fastdiv(static_cast<uint32_t>(n) ^ sgn, f) ^ sgn);
}

// n mod d in [0, d) for any int32 n (the remainder of the floor division; formed
// modulo 2^32, where n - floor(n/d) * d cannot overflow)
__host__ __device__ inline int32_t floormod_s(int32_t n, const FastDiv& f) {
  return static_cast<int32_t>(static_cast<uint32_t>(n) - static_cast<uint32_t>(floordiv_s(n, f)) * f.div);
}

// floor(F * num / den) for 64-bit F and 0 < num <= den < 2^31 (so the quotient
// fits in 64 bits): schoolbook division of the 96-bit product by 32-bit limbs.
__host__ __device__ inline uint64_t muldiv_u64(uint64_t F, uint32_t num, uint32_t den) {
  const uint64_t lo = (F & 0xffffffffull) * num;
  const uint64_t hi = (F >> 32) * num + (lo >> 32);  // < 2^63 + 2^32
  const uint64_t q1 = hi / den, r1 = hi % den;
  const uint64_t q0 = ((r1 << 32) | (lo & 0xffffffffull)) / den;
  return (q1 << 32) + q0;
}

// ---- XCD-aware work order ---------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin (block b -> XCD b % 8).
// Remap so that each XCD walks one contiguous range of work items: items that
// share K/V (same batch and KV head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int xcd = bid % kXcd, slot = bid / kXcd;
  const int start = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return start + slot;
}

}  // namespace prope
