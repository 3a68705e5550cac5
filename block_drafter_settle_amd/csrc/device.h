// Device helpers shared by the gfx950 kernel sources (types, the MFMA,
// operand layouts of internal.h, reductions, int4 unpacking).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace dfl {

typedef _Float16 f16;
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

static constexpr int kThreads = 256;

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// A-layout half index of (m, k) inside one 16-row block.
__device__ __forceinline__ size_t a_idx(int m, int k) {
  return ((size_t)(k >> 5) * 64 + ((k >> 3) & 3) * 16 + (m & 15)) * 8 + (k & 7);
}

// v as two f16 halves, hi = f16(v) and lo = f16(v − hi). The empty asm
// pins v as one rounded f32 first: left free, the compiler may contract the
// product that makes v into each half differently (an f16-result fma for
// one, the rounded f32 for the other), and then hi + lo misses v by an
// ulp of hi.
__device__ __forceinline__ void split_f16(float v, f16& hi, f16& lo) {
  asm volatile("" : "+v"(v));
  hi = (f16)v;
  lo = (f16)(v - (float)hi);
}

// Stores v's f16 pair in a key/value row: hi at row[i], lo at row[kd + i].
__device__ __forceinline__ void put_pair(f16* row, int kd, int i, float v) {
  f16 hi, lo;
  split_f16(v, hi, lo);
  row[i] = hi;
  row[kd + i] = lo;
}

// Stores v at A-layout index idx: plane 0 its f16 rounding and, when ps (the
// plane stride in halves) is nonzero, plane 1 the f16 rounding of what is left.
__device__ __forceinline__ void put_a(f16* xa, long ps, size_t idx, float v) {
  f16 hi, lo;
  split_f16(v, hi, lo);
  xa[idx] = hi;
  if (ps) xa[ps + idx] = lo;
}

// A load that marks its lines non-temporal: weights are read once per pass,
// and streaming them with this hint keeps them from displacing what is
// reused (activations, partial sums). Measured here it also raises the
// sustained read rate of a whole-chip stream. T must be a scalar or an
// ext_vector_type.
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ long map_tile(const TileMap& mp, int t) {
  return (long)(t / mp.seg) * mp.seg_stride + mp.seg_off + t % mp.seg;
}

__device__ __forceinline__ float half_bits(uint32_t b) {
  return (float)__builtin_bit_cast(f16, (uint16_t)(b & 0xffffu));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over a 256-thread block; every thread gets the total (fixed order).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Σ_s p[s·ss] over the K splits of a GEMM, in four chains (split s into
// chain s % 4 for every whole group of four, the rest into chain 0), in a
// fixed order: the same splits give the same sum. Up to 16 loads are issued
// before any add, so a sum over ≤ 16 splits costs one memory round trip
// (a chain of dependent adds would hold each load until the previous one).
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int splits, long ss) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int s = 0;
  for (; s + 16 <= splits; s += 16) {
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = p[(size_t)(s + e) * ss];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      a0 += v[e];
      a1 += v[e + 1];
      a2 += v[e + 2];
      a3 += v[e + 3];
    }
  }
  const int rem = splits - s, full = rem & ~3;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = e < rem ? p[(size_t)(s + e) * ss] : 0.f;
#pragma unroll
  for (int e = 0; e < 16; e += 4)
    if (e < full) {
      a0 += v[e];
      a1 += v[e + 1];
      a2 += v[e + 2];
      a3 += v[e + 3];
    }
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (e >= full && e < rem) a0 += v[e];
  return (a0 + a1) + (a2 + a3);
}

// (w & mask) | m in one v_and_or_b32: gfx9's three-operand encoding takes no
// literal, so the mask rides in an SGPR and m in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t m) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(m));
  return r;
}

// Eight int4 codes of one I4T word → eight f16 integers in column order.
// A nibble u' at bits 0–3 of a half over the exponent pattern of 1024 reads
// 1024 + u'; at bits 4–7 it reads 1024 + 16·u'. Both map exactly to
// q = u' − 8.
__device__ __forceinline__ h8 unpack_i4(uint32_t w) {
  const uint32_t M = 0x64006400u;
  const uint32_t w2 = w >> 8;
  const h2 q0 = __builtin_bit_cast(h2, and_or(w, 0x000F000Fu, M)) - (h2){1032, 1032};
  const h2 q1 = __builtin_bit_cast(h2, and_or(w, 0x00F000F0u, M)) * (h2){0.0625, 0.0625} -
                (h2){72, 72};
  const h2 q2 = __builtin_bit_cast(h2, and_or(w2, 0x000F000Fu, M)) - (h2){1032, 1032};
  const h2 q3 = __builtin_bit_cast(h2, and_or(w2, 0x00F000F0u, M)) * (h2){0.0625, 0.0625} -
                (h2){72, 72};
  return (h8){q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
}

// One 128-column span of R int4 tiles against four A-layout steps of PL
// planes (a, a2): per step and tile t = a·q (+ a2·q) on MFMA with the codes q
// as exact f16 integers, then acc += s·t with the group's scale s. Every
// product of the span is formed first and the scalings applied after, in the
// same order: the MFMAs run back to back instead of each waiting on the FMAs
// that free a temporary. Costs 16·R more VGPRs than i4_span_step.
template <int R, int PL>
__device__ __forceinline__ void i4_span_deferred(const uint4* c, const uint2* sc, const h8* a,
                                                 const h8* a2, f4* acc) {
  f4 t[4][R];
  float s[4][R];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t word = u == 0 ? c[r].x : u == 1 ? c[r].y : u == 2 ? c[r].z : c[r].w;
      const uint32_t sb = u < 2 ? sc[r].x : sc[r].y;
      s[u][r] = half_bits((u & 1) ? (sb >> 16) : sb);
      const h8 q = unpack_i4(word);
      t[u][r] = mfma16(a[u], q, (f4){0.f, 0.f, 0.f, 0.f});
      if (PL == 2) t[u][r] = mfma16(a2[u], q, t[u][r]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] += s[u][r] * t[u][r];
}

// As i4_span_deferred, each step's R products formed before their scalings
// (R temporaries).
template <int R, int PL>
__device__ __forceinline__ void i4_span_step(const uint4* c, const uint2* sc, const h8* a,
                                             const h8* a2, f4* acc) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f4 t[R];
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t word = u == 0 ? c[r].x : u == 1 ? c[r].y : u == 2 ? c[r].z : c[r].w;
      const uint32_t sb = u < 2 ? sc[r].x : sc[r].y;
      s[r] = half_bits((u & 1) ? (sb >> 16) : sb);
      const h8 q = unpack_i4(word);
      t[r] = mfma16(a[u], q, (f4){0.f, 0.f, 0.f, 0.f});
      if (PL == 2) t[r] = mfma16(a2[u], q, t[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] += s[r] * t[r];
  }
}

// The A fragments of span p: four steps of each plane.
template <int PL>
__device__ __forceinline__ void load_span(const h8* xp, const h8* xq, int p, h8* a, h8* a2) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    a[u] = xp[(size_t)(4 * p + u) * 64];
    if (PL == 2) a2[u] = xq[(size_t)(4 * p + u) * 64];
  }
}

// Workgroup barrier for LDS publication only: waits for this wave's LDS
// traffic (lgkmcnt 0), then meets. __syncthreads would also wait for every
// global load in flight (vmcnt 0), draining prefetched weights or K/V.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

template <int N_OUT>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N_OUT) with expcnt/lgkmcnt left at their maxima (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt((N_OUT & 15) | (7 << 4) | (15 << 8) | ((N_OUT >> 4) << 14));
}

}  // namespace dfl
