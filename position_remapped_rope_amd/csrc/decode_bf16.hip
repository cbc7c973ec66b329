// Split-K decode against a KV cache of base-rotated keys (bf16), HBM-bound.
//
// Jet-Long page, section 3.2: the cache keeps k_cache[j] = RoPE(x_j, j)
// (Eq. (4)) and is never rewritten. For a query at p_q = kv_len - 1, a key at
// distance p_q - j <= w0 scores with the cached vectors as they are; a farther
// key scores with the remote view RoPE(q, dq) . RoPE(k_j, dk_j), where
// dq = floor(p_q/s) - p_q and dk_j = floor(j/s) - j (Eq. (5)-(6)); with the
// frequency-interpolation mapping (same page, section 4.5) the corrections are
// p_q * (theta_i/s - theta_i) and j * (theta_i/s - theta_i). Both are formed in
// registers from exact integer phases; nothing is written back. With the
// interpolation map and a per-sequence scale s = max(1, kv_len / w_pre) (the
// continuous-style factor of Jet-Long section 3.1), each workgroup forms the
// correction frequencies theta_i * w_pre / kv_len - theta_i from the exact
// 64-bit phases. NOPE/ROPE caches already carry their rotation, so those modes
// score q . k_j with an optional window and optional ALiBi biases
// - m_h (p_q - j) (P-RoPE page, section 1).
//
// Kernel 1 (split): one workgroup per (chunk of a.chunk keys, group of a.hpw
// KV heads, sequence). With hpw = 4 each of its 4 waves streams the whole chunk
// of one head (the 4 heads' slices of a key row are contiguous); with hpw = 1
// the 4 waves stream a quarter of the chunk of one head each and merge their
// partials in LDS at the end. Waves step through their keys 32 at a time with
// no workgroup barrier. Per step and wave:
//   - K rows are loaded straight into the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 (lane l: key l%16, dims 8*(l/16) + 32*ks ..+7;
//     16-byte loads, each key's 256 bytes read by 16 lanes), remote keys are
//     rotated by dk_j in registers and rounded to bf16;
//   - S^T = K Q^T on MFMA against the G query heads of the KV group (padded to
//     16 columns: every loaded byte serves all G heads);
//   - online softmax per head over the step's 32 keys;
//   - V rows go through a per-wave LDS tile and come back transposed
//     (ds_read_b64_tr_b16) as the B operand of O = P V on MFMA; the S^T
//     accumulator layout is already P's A-operand layout.
// Each chunk's partial softmax statistics (row max m, row sum l, unnormalised
// O) go to the workspace.
// Kernel 2 (combine): per (sequence, query head) the chunk partials are
// merged with log-sum-exp weights (Jet-Long Eq. (7)'s merge with only
// disjoint parts) into O and the LSE.
#include "internal.hpp"

namespace prope {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kDThreads = 256;  // 4 waves
constexpr int kStep = 32;       // keys per wave step (two 16-key MFMA blocks)

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// gfx950 ds_read_b64_tr_b16: within each 16-lane group, lane j names row j/4
// and columns 4*(j%4) .. +3 of a 4 x 16 block of 16-bit values; lane i
// receives column i of the block, rows 0..3 in order.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// max / sum across the 4 lanes that hold the same head (l, l^16, l^32, l^48)
__device__ __forceinline__ float xgroup_max(float x) {
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
}
__device__ __forceinline__ float xgroup_sum(float x) {
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
}

// EARLY: the first step's K/V loads go out before the query rotation (the
// 1-head layout; the 4-head layout keeps them after the phase tables, which
// measured faster there)
template <int D, int MODE, bool EARLY>
__global__ __launch_bounds__(kDThreads, 2) void decode_split_kernel(const DecodeArgs a) {
  constexpr int KSTEPS = D / 32;             // 16x16x32 k-steps over the head dimension
  constexpr int DBLK = D / 16;               // 16-dim blocks of O
  constexpr int VROW = D + 16;               // V tile row stride (elements): transposing reads hit distinct banks
  constexpr int VCHUNKS = kStep * D / 8;     // 16-byte chunks of one V tile
  constexpr int VPL = VCHUNKS / 64;          // per lane
  constexpr int WAVES = kDThreads / 64;
  __shared__ __attribute__((aligned(16))) uint16_t vtile[WAVES][kStep * VROW];
  __shared__ uint2 ftab[D / 2];
  __shared__ float red_m[WAVES][16], red_l[WAVES][16];
  __shared__ float red_o[WAVES][16][D + 4];

  // A workgroup takes one chunk of a.chunk keys for a.hpw KV heads: wave w
  // serves head slot w % hpw and the (w / hpw)-th of the kw = 4 / hpw equal
  // parts of the chunk. With hpw = 4 the waves read 4 heads' slices of the same
  // rows, 4 * d * 2 contiguous bytes per row, which spreads the reads over more
  // DRAM channels than one head's slice; each wave then owns its partial. With
  // kw > 1 the waves of one head merge their partials in LDS.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hpw = a.hpw, kw = WAVES / a.hpw;
  const int kvh = blockIdx.y * hpw + wave % hpw;
  const int chunk = blockIdx.x;
  const int b = blockIdx.z;
  const int kl = lane & 15, kg = lane >> 4;
  const int G = a.G;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);  // a length outside [0, Lmax] never reads past the cache
  if (MODE == kBifocal) {  // correction frequencies of the query and key phases (all waves, before any exit)
    if (tid < D / 2) {
      uint64_t c = (uint64_t(a.fr.hi[tid]) << 32) | a.fr.lo[tid];
      if (a.interp && a.w_pre > 0) {  // theta_i / s - theta_i with s = L / w_pre when L > w_pre, else 0
        const uint64_t F = (uint64_t(a.f.hi[tid]) << 32) | a.f.lo[tid];
        c = L > a.w_pre ? muldiv_u64(F, static_cast<uint32_t>(a.w_pre), static_cast<uint32_t>(L)) - F : 0;
      }
      ftab[tid] = make_uint2(static_cast<uint32_t>(c), static_cast<uint32_t>(c >> 32));
    }
    __syncthreads();
  }
  const int jbeg = chunk * a.chunk;
  const size_t head_stride = size_t(a.n_chunks) * (D + 2);
  float* wsb = a.ws + (size_t(b) * a.Hq + size_t(kvh) * G) * head_stride + size_t(chunk) * (D + 2);

  if (jbeg >= L) {  // chunk past this sequence's length: empty partials (whole workgroup)
    if (lane < G && wave < hpw) {
      wsb[lane * head_stride] = -INFINITY;
      wsb[lane * head_stride + 1] = 0.f;
    }
    return;
  }
  const int jend = min(L, jbeg + a.chunk);
  const int pq = L - 1;
  const float sl2 = a.scale_log2;
  const int w0 = a.window_left;
  // ALiBi slope of this lane's head kl, log2 units (0: no bias)
  const float slope2 =
      (MODE != kBifocal && a.alibi && kl < G) ? a.alibi[size_t(kvh) * G + kl] * 1.4426950408889634f : 0.f;

  // ---- query operand (B of S^T = K Q^T): lane l holds head kl, dims 8kg + 32ks .. +7
  // in the local view (as given) and the remote view RoPE(q, dq), both bf16.
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + (size_t(b) * a.Hq + size_t(kvh) * G) * D;
  u32x4_t qloc[KSTEPS], qrem[KSTEPS];
  // remote scale: fixed, or Jet-Long Eq. (2)'s group size for this sequence's length
  const FastDiv sdv = a.w_pre > 0 ? make_fastdiv(static_cast<uint32_t>(max(1, L / a.w_pre + (L % a.w_pre != 0))))
                                  : a.scale_div;
  // correction index of position x: floor(x/s) - x (alias) or x itself (interpolation,
  // whose correction frequencies theta_i / s - theta_i are in fr)
  auto corr = [&](int x) __attribute__((always_inline)) {
    return a.interp ? x : static_cast<int>(fastdiv(static_cast<uint32_t>(x), sdv)) - x;
  };
  const int dq = MODE == kBifocal ? corr(pq) : 0;
  // this wave's keys
  const int per_wave = a.chunk / kw;
  const int wbeg = jbeg + (wave / hpw) * per_wave;
  const int wend = min(jend, wbeg + per_wave);
  const uint32_t rowk_b = uint32_t(a.Hkv) * D * 2;
  const size_t bofs = size_t(b) * a.Lmax * a.Hkv * D + size_t(kvh) * D;
  const uint32_t span = uint32_t(jend) * rowk_b;  // loads at or past jend read 0
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(static_cast<const uint16_t*>(a.k) + bofs, span);
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(static_cast<const uint16_t*>(a.v) + bofs, span);

  u32x4_t kraw[2][KSTEPS], vraw[VPL];
  auto load_v = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int c = lane + 64 * u;  // chunk c: key c / (D/8), 16-byte column c % (D/8)
      vraw[u] = bload16(vres, uint32_t(j0 + c / (D / 8)) * rowk_b + (c % (D / 8)) * 16);
    }
  };
  auto load_k = [&](int j0, int blk) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      kraw[blk][ks] = bload16(kres, uint32_t(j0 + 16 * blk + kl) * rowk_b + (8 * kg + 32 * ks) * 2);
  };

#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4_t w = {0, 0, 0, 0};
    if (kl < G) w = *reinterpret_cast<const u32x4_t*>(qg + size_t(kl) * D + 8 * kg + 32 * ks);
    qloc[ks] = w;
  }
  // EARLY: the first step's K/V loads between the query's loads and its
  // rotation, whose VALU work (and the phase tables') then overlaps their
  // latency. They are unconditional: a wave with no keys has wbeg >= jend, so
  // they fall past the resources' span and read 0, and with no branch around
  // them the wait before the rotation counts exactly the loads issued after
  // the query's (behind a branch it waits for all of them).
  if constexpr (EARLY) {
    load_v(wbeg);
    load_k(wbeg, 0);
    load_k(wbeg, 1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const u32x4_t w = qloc[ks];
    if (MODE == kBifocal) {
      u32x4_t y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pi = 4 * kg + 16 * ks + e;
        float sn, cs, y0, y1;
        const uint2 fq = ftab[pi];
        rope_sincos(dq, fq.x, fq.y, sn, cs);
        rot_pair(bf16_lo(w[e]), bf16_hi(w[e]), cs, sn, y0, y1);
        y[e] = pack_bf16(y0, y1);
      }
      qrem[ks] = y;
    }
  }
  // ---- remote-key rotation phases ------------------------------------------
  // Lane l rotates key j (block 0) and key j + 16 (block 1) of each step, for
  // its pairs 4kg + 16ks + e. When s divides 16, dk_j = floor(j/s) - j moves
  // by d16 = 16/s - 16 between those keys and by 2*d16 from step to step, so
  // each pair's phase (2^-32 turn units) advances by a fixed increment; the
  // carries dropped from the low 32 bits cost at most 2^-32 turn per step.
  // Otherwise every phase is formed exactly from the frequency table in LDS.
  const int sdiv = static_cast<int>(sdv.div);
  const bool affine = a.interp || (16 % sdiv) == 0;
  uint32_t ph[KSTEPS][4], inc[KSTEPS][4];
  if (MODE == kBifocal) {
    const int dk0 = corr(wbeg + kl);
    const int d16 = a.interp ? 16 : affine ? 16 / sdiv - 16 : 0;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 fk = ftab[4 * kg + 16 * ks + e];
        ph[ks][e] = phase_top(dk0, fk.x, fk.y);
        inc[ks][e] = phase_top(d16, fk.x, fk.y);
      }
  }

  float m_run = -INFINITY, l_run = 0.f;  // per head kl (replicated over the 4 lane groups)
  f32x4_t oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* vt = vtile[wave];
  const int trow = 4 * kg + (kl >> 2);  // transposing-read row of this lane (block 0)
  const int tcol = 4 * (kl & 3);        // and column offset within a 16-dim block

  // Loads of the next step go out as soon as the registers they fill are free:
  // V right after this step's V is in LDS, each K block right after its scores,
  // so their latency overlaps this step's rotation and MFMA work.
  if (!EARLY && wbeg < wend) {
    load_v(wbeg);
    load_k(wbeg, 0);
    load_k(wbeg, 1);
  }
  for (int j0 = wbeg; j0 < wend; j0 += kStep) {
    const bool more = j0 + kStep < wend;
    // -- V of this step to LDS (row-major); read back transposed after the scores
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int c = lane + 64 * u;
      *reinterpret_cast<u32x4_t*>(&vt[(c / (D / 8)) * VROW + (c % (D / 8)) * 8]) = vraw[u];
    }
    if (more) load_v(j0 + kStep);
    // -- scores S^T (keys x heads) for the two 16-key blocks
    f32x4_t sc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int jb = j0 + 16 * blk;  // first key of the block
      // bifocal: does the block hold remote keys (pq - j > w0), local ones, or both?
      const bool any_remote = MODE == kBifocal && (pq - jb > w0);
      const bool any_local = MODE != kBifocal || (pq - (jb + 15) <= w0);
      f32x4_t srem = {0.f, 0.f, 0.f, 0.f}, sloc = {0.f, 0.f, 0.f, 0.f};
      if (any_local) {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) sloc = mfma16x16x32(kraw[blk][ks], qloc[ks], sloc);
      }
      if (any_remote) {
        const int j = jb + kl;  // this lane's key
        const int dk = affine ? 0 : corr(j);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          u32x4_t y;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t phk;
            if (affine) {
              phk = blk ? ph[ks][e] + inc[ks][e] : ph[ks][e];
            } else {
              const uint2 f = ftab[4 * kg + 16 * ks + e];
              phk = phase_top(dk, f.x, f.y);
            }
            float sn, cs, y0, y1;
            phase_sincos(phk, sn, cs);
            rot_pair(bf16_lo(kraw[blk][ks][e]), bf16_hi(kraw[blk][ks][e]), cs, sn, y0, y1);
            y[e] = pack_bf16(y0, y1);
          }
          srem = mfma16x16x32(y, qrem[ks], srem);
        }
      }
      // lane l holds S^T[key jb + 4kg + i][head kl]; route, mask and scale
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jb + 4 * kg + i;
        const int dist = pq - j;
        float v;
        if (MODE == kBifocal)
          v = dist > w0 ? srem[i] : sloc[i];
        else
          v = sloc[i];
        const bool keep = j < wend && (MODE == kBifocal || w0 < 0 || dist <= w0);
        const float bias = MODE == kBifocal ? 0.f : -slope2 * static_cast<float>(dist);
        sc[blk][i] = keep ? fmaf(v, sl2, bias) : -INFINITY;
      }
      if (more) load_k(j0 + kStep, blk);
    }
    if (MODE == kBifocal && affine) {  // the lane's block-0 key moves by 32
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) ph[ks][e] += 2 * inc[ks][e];
    }

    // -- online softmax per head over the 32 keys
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = xgroup_max(mx);
    const float mnew = fmaxf(m_run, mx);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mref);
    m_run = mnew;
    float pv[8], rs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(sc[0][i] - mref);
      pv[4 + i] = __builtin_amdgcn_exp2f(sc[1][i] - mref);
      rs += pv[i] + pv[4 + i];
    }
    l_run = l_run * alpha + rs;
    // P^T as the B operand: lane (head kl, group kg) k-slots 8kg + e are keys
    // 4kg + e (block 0) and 16 + 4kg + e - 4 (block 1): exactly its registers
    const u32x4_t pop = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                         pack_bf16(pv[6], pv[7])};
    // O^T is accumulated, so a lane's O values belong to its own head kl and
    // take its own alpha
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha;
    // -- O^T += V^T P^T: V^T operand rows = dims kl of each 16-dim block, k-slots = the keys above
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const u32x2_t va = lds_read_tr16(&vt[trow * VROW + 16 * db + tcol]);
      const u32x2_t vb = lds_read_tr16(&vt[(trow + 16) * VROW + 16 * db + tcol]);
      oacc[db] = mfma16x16x32(u32x4_t{va[0], va[1], vb[0], vb[1]}, pop, oacc[db]);
    }
  }

  // ---- partials: lane (kl, kg=0) holds head kl's m and l; lane (kl, kg) holds
  // O[head kl][dims 16db + 4kg + i]
  const float l_all = xgroup_sum(l_run);  // all lanes active for the cross-lane exchange
  if (kw == 1) {  // the wave's partial is the chunk's
    if (kg == 0 && kl < G) {
      wsb[kl * head_stride] = m_run;
      wsb[kl * head_stride + 1] = l_all;
    }
    if (kl < G) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) wsb[kl * head_stride + 2 + 16 * db + 4 * kg + i] = oacc[db][i];
    }
    return;
  }
  // merge the kw partials of each head slot in LDS
  if (kg == 0) {
    red_m[wave][kl] = m_run;
    red_l[wave][kl] = l_all;
  }
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[wave][kl][16 * db + 4 * kg + i] = oacc[db][i];
  __syncthreads();
  for (int idx = tid; idx < hpw * G * D; idx += kDThreads) {
    const int hs = idx / (G * D), g = (idx / D) % G, dd = idx % D;
    float M = -INFINITY;
    for (int q = 0; q < kw; ++q) M = fmaxf(M, red_m[hs + q * hpw][g]);
    const float Mref = M == -INFINITY ? 0.f : M;
    float acc = 0.f, lsum = 0.f;
    for (int q = 0; q < kw; ++q) {
      const int w = hs + q * hpw;
      const float wt = __builtin_amdgcn_exp2f(red_m[w][g] - Mref);
      acc = fmaf(wt, red_o[w][g][dd], acc);
      lsum = fmaf(wt, red_l[w][g], lsum);
    }
    float* dst = a.ws + (size_t(b) * a.Hq + size_t(blockIdx.y * hpw + hs) * G + g) * head_stride +
                 size_t(chunk) * (D + 2);
    dst[2 + dd] = acc;
    if (dd == 0) {
      dst[0] = M;
      dst[1] = lsum;
    }
  }
}

// One workgroup per (query head, sequence): thread (cg, dv) takes chunks cg,
// cg + CG, ... (one round of loads for up to 4 * CG chunks, as at 128K; short
// caches split into more chunks take a few rounds) and 4 dims of O, merges
// them against its own running max as it goes (the same log-sum-exp algebra as
// the split kernel), and the CG partial merges are combined once in LDS.
template <int D>
__global__ __launch_bounds__(1024) void decode_combine_kernel(const DecodeArgs a) {
  constexpr int NT = 1024;
  constexpr int DV = D / 4;       // float4 columns per partial
  constexpr int CG = NT / DV;     // chunk groups
  __shared__ float sm[CG], sl[CG];
  __shared__ float4 so[CG][DV];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);
  const int nc = (L + a.chunk - 1) / a.chunk;
  const size_t stride = D + 2;
  const float* wsb = a.ws + (size_t(b) * a.Hq + h) * size_t(a.n_chunks) * stride;
  const int dv = tid % DV, cg = tid / DV;

  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // Up to kBatch of this thread's chunks per round: all their loads go out
  // before the first use, so a round costs one memory latency (the partials
  // were just written by other compute units and come from memory), and the
  // merge is branch-free (a chunk past the end, or with no kept key, has
  // weight 0).
  constexpr int kBatch = 4;
  for (int c0 = cg; c0 < nc; c0 += kBatch * CG) {
    float mc[kBatch], lc[kBatch];
    float2 x0[kBatch], x1[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = min(c0 + u * CG, nc - 1);  // (nc >= 1 inside the loop)
      const float* part = wsb + size_t(c) * stride;
      const float2 ml = *reinterpret_cast<const float2*>(part);  // (m, l); partials are 8-byte aligned
      mc[u] = c0 + u * CG < nc ? ml.x : -INFINITY;
      lc[u] = ml.y;
      // partial O starts at float offset 2: read as two float2 to stay 8-byte aligned
      x0[u] = *reinterpret_cast<const float2*>(part + 2 + 4 * dv);
      x1[u] = *reinterpret_cast<const float2*>(part + 4 + 4 * dv);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float mn = fmaxf(m, mc[u]);
      const float mr = mn == -INFINITY ? 0.f : mn;  // nothing kept so far: both weights 0
      const float wo = __builtin_amdgcn_exp2f(m - mr), wc = __builtin_amdgcn_exp2f(mc[u] - mr);
      l = l * wo + lc[u] * wc;
      acc.x = acc.x * wo + x0[u].x * wc;
      acc.y = acc.y * wo + x0[u].y * wc;
      acc.z = acc.z * wo + x1[u].x * wc;
      acc.w = acc.w * wo + x1[u].y * wc;
      m = mn;
    }
  }
  so[cg][dv] = acc;
  if (dv == 0) {
    sm[cg] = m;
    sl[cg] = l;
  }
  __syncthreads();
  if (tid < DV) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < CG; ++g) M = fmaxf(M, sm[g]);
    const float Mref = M == -INFINITY ? 0.f : M;
    float lsum = 0.f;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      const float w = __builtin_amdgcn_exp2f(sm[g] - Mref);
      lsum = fmaf(w, sl[g], lsum);
      const float4 o = so[g][tid];
      t.x = fmaf(w, o.x, t.x);
      t.y = fmaf(w, o.y, t.y);
      t.z = fmaf(w, o.z, t.z);
      t.w = fmaf(w, o.w, t.w);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint2 packed;
    packed.x = pack_bf16(t.x * inv, t.y * inv);
    packed.y = pack_bf16(t.z * inv, t.w * inv);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + (size_t(b) * a.Hq + h) * D + 4 * tid) = packed;
    if (a.lse && tid == 0)
      a.lse[size_t(b) * a.Hq + h] = lsum > 0.f ? (M + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
  }
}

template <int D, int MODE>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  if (a.hpw == 1)
    hipLaunchKernelGGL((decode_split_kernel<D, MODE, true>), dim3(a.n_chunks, a.Hkv / a.hpw, a.B), dim3(kDThreads),
                       0, stream, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, MODE, false>), dim3(a.n_chunks, a.Hkv / a.hpw, a.B), dim3(kDThreads),
                       0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.Hq, a.B), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.D == 128) {
    switch (a.mode) {
      case kNope: return launch_d<128, kNope>(a, stream);
      case kRope: return launch_d<128, kRope>(a, stream);
      default: return launch_d<128, kBifocal>(a, stream);
    }
  }
  switch (a.mode) {
    case kNope: return launch_d<64, kNope>(a, stream);
    case kRope: return launch_d<64, kRope>(a, stream);
    default: return launch_d<64, kBifocal>(a, stream);
  }
}

}  // namespace prope
