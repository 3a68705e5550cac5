// gfx950 kernels of the DFlash 2 drafter's settle and block passes.
//
// What each kernel computes is defined on the docs.rs page
// "cortiq_engine/dflash.rs" (cortiq-engine 0.8.78): `rms`, `rotate`, `conv`,
// `mlp`, `Drafter::block` (the attention), `settle_rows`, `select_with`,
// `top_k`. Operand layouts (A-layout, F16T, I4T, tile maps) are described
// in internal.h.
//
// Every matrix product runs on v_mfma_f32_16x16x32_f16: activations are
// rounded to f16, int4 codes enter the MFMA as exact small integers and
// each 32-column group's partial is scaled by its f16 scale in f32, so the
// dequantised weight q·s is used exactly. Accumulation is f32 throughout.
#include "internal.h"

#include <climits>
#include <math.h>

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
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Eight int4 codes of one I4T word → eight f16 integers in column order.
// A nibble u' at bits 0–3 of a half over the exponent pattern of 1024 reads
// 1024 + u'; at bits 4–7 it reads 1024 + 16·u'. Both map exactly to
// q = u' − 8.
__device__ __forceinline__ h8 unpack_i4(uint32_t w) {
  const uint32_t M = 0x64006400u;
  const uint32_t w2 = w >> 8;
  const h2 q0 = __builtin_bit_cast(h2, (w & 0x000F000Fu) | M) - (h2){1032, 1032};
  const h2 q1 = __builtin_bit_cast(h2, (w & 0x00F000F0u) | M) * (h2){0.0625, 0.0625} - (h2){72, 72};
  const h2 q2 = __builtin_bit_cast(h2, (w2 & 0x000F000Fu) | M) - (h2){1032, 1032};
  const h2 q3 = __builtin_bit_cast(h2, (w2 & 0x00F000F0u) | M) * (h2){0.0625, 0.0625} - (h2){72, 72};
  return (h8){q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
}

// ------------------------------------------------------------------ GEMMs

// Skinny GEMM, f16 weights: each wave owns R row tiles over its K split.
template <int R>
__global__ __launch_bounds__(kThreads) void k_gemm_f16(const f16* __restrict__ xa, int K,
                                                       const f16* __restrict__ w, TileMap mp,
                                                       int N, int sps, float* __restrict__ out,
                                                       long split_stride) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KS = K >> 5;
  const int sp = blockIdx.y, mb = blockIdx.z;
  const int s0 = sp * sps, s1 = min(KS, s0 + sps);
  const int t0 = (blockIdx.x * 4 + wave) * R;
  if (t0 >= mp.ntiles) return;
  const h8* xp = reinterpret_cast<const h8*>(xa + (size_t)mb * 16 * K) + lane;
  const h8* wp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = min(t0 + r, mp.ntiles - 1);
    wp[r] = reinterpret_cast<const h8*>(w) + (size_t)map_tile(mp, t) * KS * 64 + lane;
  }
  f4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = (f4){0.f, 0.f, 0.f, 0.f};
  int s = s0;
  for (; s + 4 <= s1; s += 4) {
    h8 a[4], b[4][R];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = xp[(size_t)(s + u) * 64];
#pragma unroll
      for (int r = 0; r < R; ++r) b[u][r] = wp[r][(size_t)(s + u) * 64];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mfma16(a[u], b[u][r], acc[r]);
  }
  for (; s < s1; ++s) {
    const h8 a = xp[(size_t)s * 64];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = mfma16(a, wp[r][(size_t)s * 64], acc[r]);
  }
  float* o = out + (size_t)sp * split_stride + (size_t)mb * 16 * N;
  const int j = lane >> 4, n = lane & 15;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r, col = t * 16 + n;
    if (t < mp.ntiles && col < N)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[(size_t)(4 * j + v) * N + col] = acc[r][v];
  }
}

// One 128-column span of R int4 tiles against four A-layout steps.
template <int R>
__device__ __forceinline__ void i4_span(const uint4* c, const uint2* sc, const h8* a, f4* acc) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t word = u == 0 ? c[r].x : u == 1 ? c[r].y : u == 2 ? c[r].z : c[r].w;
      const uint32_t sb = u < 2 ? sc[r].x : sc[r].y;
      const float s = half_bits((u & 1) ? (sb >> 16) : sb);
      const f4 t = mfma16(a[u], unpack_i4(word), (f4){0.f, 0.f, 0.f, 0.f});
      acc[r] += s * t;
    }
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void k_gemm_i4(const f16* __restrict__ xa, int K,
                                                      const uint4* __restrict__ codes,
                                                      const uint2* __restrict__ scales,
                                                      TileMap mp, int N, int pps,
                                                      float* __restrict__ out, long split_stride) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KT = K >> 7;
  const int sp = blockIdx.y, mb = blockIdx.z;
  const int p0 = sp * pps, p1 = min(KT, p0 + pps);
  const int t0 = (blockIdx.x * 4 + wave) * R;
  if (t0 >= mp.ntiles) return;
  const h8* xp = reinterpret_cast<const h8*>(xa + (size_t)mb * 16 * K) + lane;
  const uint4* cp[R];
  const uint2* scp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const long st = map_tile(mp, min(t0 + r, mp.ntiles - 1));
    cp[r] = codes + (size_t)st * KT * 64 + lane;
    scp[r] = scales + (size_t)st * KT * 16 + (lane & 15);
  }
  f4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = (f4){0.f, 0.f, 0.f, 0.f};
  int p = p0;
  for (; p + 2 <= p1; p += 2) {
    uint4 c0[R], c1[R];
    uint2 s0[R], s1[R];
    h8 a0[4], a1[4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      c0[r] = cp[r][(size_t)p * 64];
      c1[r] = cp[r][(size_t)(p + 1) * 64];
      s0[r] = scp[r][(size_t)p * 16];
      s1[r] = scp[r][(size_t)(p + 1) * 16];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a0[u] = xp[(size_t)(4 * p + u) * 64];
      a1[u] = xp[(size_t)(4 * p + 4 + u) * 64];
    }
    i4_span<R>(c0, s0, a0, acc);
    i4_span<R>(c1, s1, a1, acc);
  }
  if (p < p1) {
    uint4 c0[R];
    uint2 s0[R];
    h8 a0[4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      c0[r] = cp[r][(size_t)p * 64];
      s0[r] = scp[r][(size_t)p * 16];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) a0[u] = xp[(size_t)(4 * p + u) * 64];
    i4_span<R>(c0, s0, a0, acc);
  }
  float* o = out + (size_t)sp * split_stride + (size_t)mb * 16 * N;
  const int j = lane >> 4, n = lane & 15;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r, col = t * 16 + n;
    if (t < mp.ntiles && col < N)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[(size_t)(4 * j + v) * N + col] = acc[r][v];
  }
}

// gate/up over the full K, SwiGLU in the epilogue (`mlp`: silu(g)·u with
// silu(a) = a/(1+e^−a)). Block b: waves 0, 1 take gate tiles 2b, 2b+1;
// waves 2, 3 the up tiles of the same rows.
__global__ __launch_bounds__(kThreads) void k_gemm_glu(const f16* __restrict__ xa, int K,
                                                       const uint4* __restrict__ codes,
                                                       const uint2* __restrict__ scales,
                                                       int ftiles, f16* __restrict__ ma) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KT = K >> 7;
  const int ft = 2 * blockIdx.x + (wave & 1);
  const long st = wave < 2 ? ft : ftiles + ft;
  const h8* xp = reinterpret_cast<const h8*>(xa) + lane;
  const uint4* cp = codes + (size_t)st * KT * 64 + lane;
  const uint2* scp = scales + (size_t)st * KT * 16 + (lane & 15);
  f4 acc[1] = {(f4){0.f, 0.f, 0.f, 0.f}};
  int p = 0;
  for (; p + 2 <= KT; p += 2) {
    uint4 c0[1] = {cp[(size_t)p * 64]}, c1[1] = {cp[(size_t)(p + 1) * 64]};
    uint2 s0[1] = {scp[(size_t)p * 16]}, s1[1] = {scp[(size_t)(p + 1) * 16]};
    h8 a0[4], a1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a0[u] = xp[(size_t)(4 * p + u) * 64];
      a1[u] = xp[(size_t)(4 * p + 4 + u) * 64];
    }
    i4_span<1>(c0, s0, a0, acc);
    i4_span<1>(c1, s1, a1, acc);
  }
  if (p < KT) {
    uint4 c0[1] = {cp[(size_t)p * 64]};
    uint2 s0[1] = {scp[(size_t)p * 16]};
    h8 a0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a0[u] = xp[(size_t)(4 * p + u) * 64];
    i4_span<1>(c0, s0, a0, acc);
  }
  __shared__ float up[2][16][17];
  const int j = lane >> 4, n = lane & 15;
  if (wave >= 2)
#pragma unroll
    for (int v = 0; v < 4; ++v) up[wave - 2][4 * j + v][n] = acc[0][v];
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * j + v;
      const float g = acc[0][v];
      const float val = g / (1.f + expf(-g)) * up[wave][m][n];
      ma[a_idx(m, ft * 16 + n)] = (f16)val;
    }
  }
}

// The head over rows 1..k (logits [k][width]) and, in blocks past
// head_groups, the selector projection of all 16 rows (hp [16][rank]).
__global__ __launch_bounds__(kThreads) void k_head(const f16* __restrict__ xa, int K,
                                                   const f16* __restrict__ head, int wtiles,
                                                   int width, int k, float* __restrict__ logits,
                                                   const f16* __restrict__ sel, int stiles,
                                                   int rank, float* __restrict__ hp,
                                                   int head_groups) {
  constexpr int R = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool is_sel = (int)blockIdx.x >= head_groups;
  const f16* w = is_sel ? sel : head;
  const int ntiles = is_sel ? stiles : wtiles;
  const int grp = is_sel ? blockIdx.x - head_groups : blockIdx.x;
  const int KS = K >> 5;
  const int t0 = (grp * 4 + wave) * R;
  if (t0 >= ntiles) return;
  const h8* xp = reinterpret_cast<const h8*>(xa) + lane;
  const h8* wp[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wp[r] = reinterpret_cast<const h8*>(w) + (size_t)min(t0 + r, ntiles - 1) * KS * 64 + lane;
  f4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = (f4){0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= KS; s += 4) {
    h8 a[4], b[4][R];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = xp[(size_t)(s + u) * 64];
#pragma unroll
      for (int r = 0; r < R; ++r) b[u][r] = wp[r][(size_t)(s + u) * 64];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mfma16(a[u], b[u][r], acc[r]);
  }
  for (; s < KS; ++s) {
    const h8 a = xp[(size_t)s * 64];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = mfma16(a, wp[r][(size_t)s * 64], acc[r]);
  }
  const int j = lane >> 4, n = lane & 15;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r, col = t * 16 + n;
    if (t >= ntiles) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * j + v;
      if (is_sel) {
        if (col < rank) hp[(size_t)m * rank + col] = acc[r][v];
      } else if (m >= 1 && m <= k && col < width) {
        logits[(size_t)(m - 1) * width + col] = acc[r][v];
      }
    }
  }
}

// ----------------------------------------------------------- row kernels

// f32 rows → A-layout f16; one thread per 8 columns of one row.
__global__ __launch_bounds__(kThreads) void k_to_a(const float* __restrict__ x, long ld, int m,
                                                   int K, f16* __restrict__ xa) {
  const int mb = blockIdx.y;
  const long t = (long)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (long)(K >> 3) * 16) return;
  const int i = t & 15, j = (t >> 4) & 3;
  const long s = t >> 6;
  const int row = mb * 16 + i;
  h8 v = (h8){0, 0, 0, 0, 0, 0, 0, 0};
  if (row < m) {
    const float4* p = reinterpret_cast<const float4*>(x + (size_t)row * ld + s * 32 + j * 8);
    const float4 lo = p[0], hi = p[1];
    v = (h8){(f16)lo.x, (f16)lo.y, (f16)lo.z, (f16)lo.w, (f16)hi.x, (f16)hi.y, (f16)hi.z, (f16)hi.w};
  }
  reinterpret_cast<h8*>(xa + (size_t)mb * 16 * K)[t] = v;
}

// `rms` of the split-summed rows → A-layout f16 (the settle's hidden norm).
__global__ __launch_bounds__(kThreads) void k_sum_norm(const float* __restrict__ part, int splits,
                                                       long ss, int N, const float* __restrict__ w,
                                                       float eps, f16* __restrict__ xa) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const float* pr = part + (size_t)row * N;
  float sq = 0.f;
  for (int i = threadIdx.x; i < N; i += kThreads) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += pr[(size_t)s * ss + i];
    sq += v * v;
  }
  sq = block_sum(sq, red);
  const float scale = 1.f / sqrtf(sq / N + eps);
  f16* out = xa + (size_t)(row >> 4) * 16 * N;
  for (int i = threadIdx.x; i < N; i += kThreads) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += pr[(size_t)s * ss + i];
    out[a_idx(row & 15, i)] = (f16)(v * scale * w[i]);
  }
}

// Rows [E[anchor], E[mask]…] and their `rms` by the first layer's gain.
__global__ __launch_bounds__(kThreads) void k_embed_norm(const f16* __restrict__ embed, int anchor,
                                                         int mask, int hs,
                                                         const float* __restrict__ w, float eps,
                                                         float* __restrict__ h,
                                                         float* __restrict__ x,
                                                         f16* __restrict__ xa) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const f16* e = embed + (size_t)(r == 0 ? anchor : mask) * hs;
  float sq = 0.f;
  for (int i = threadIdx.x; i < hs; i += kThreads) {
    const float v = (float)e[i];
    h[(size_t)r * hs + i] = v;
    sq += v * v;
  }
  sq = block_sum(sq, red);
  const float scale = 1.f / sqrtf(sq / hs + eps);
  for (int i = threadIdx.x; i < hs; i += kThreads) {
    const float y = (float)e[i] * scale * w[i];
    x[(size_t)r * hs + i] = y;
    xa[a_idx(r, i)] = (f16)y;
  }
}

// Conv stage 0 of row r (`conv`): xc[r][i] = Σ_{o ≤ min(kn−1, r)}
// (base[0][o][i] + d[r][0][o][i/gs])·x[r−o][i]. Also keeps row r's summed
// kernel projection (both stages) for stage 1.
__global__ __launch_bounds__(kThreads) void k_conv0(const float* __restrict__ x,
                                                    const float* __restrict__ dpart, int splits,
                                                    long ss, const float* __restrict__ base,
                                                    int hs, int gs, int kn, f16* __restrict__ xca,
                                                    float* __restrict__ dsum) {
  extern __shared__ float dl[];
  const int r = blockIdx.x;
  const int G = hs / gs, P = 2 * kn * G;
  for (int i = threadIdx.x; i < P; i += kThreads) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += dpart[(size_t)s * ss + (size_t)r * P + i];
    dl[i] = v;
    dsum[(size_t)r * P + i] = v;
  }
  __syncthreads();
  const int taps = min(kn, r + 1);
  for (int i = threadIdx.x; i < hs; i += kThreads) {
    const int g = i / gs;
    float acc = 0.f;
    for (int o = 0; o < taps; ++o)
      acc += (base[(size_t)o * hs + i] + dl[o * G + g]) * x[(size_t)(r - o) * hs + i];
    xca[a_idx(r, i)] = (f16)acc;
  }
}

// Conv stage 1 of the sub-layer's output into the residual, then the next
// `rms`: h[r] += Σ_o (base[1][o] + d[r][1][o][g])·out[r−o]; x = rms(h[r], w).
__global__ __launch_bounds__(kThreads) void k_conv1_norm(float* __restrict__ h,
                                                         const float* __restrict__ opart,
                                                         int splits, long ss,
                                                         const float* __restrict__ dsum,
                                                         const float* __restrict__ base, int hs,
                                                         int gs, int kn,
                                                         const float* __restrict__ w, float eps,
                                                         float* __restrict__ x,
                                                         f16* __restrict__ xa) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int G = hs / gs, P = 2 * kn * G;
  const int taps = min(kn, r + 1);
  const float* b1 = base + (size_t)kn * hs;
  const float* d1 = dsum + (size_t)r * P + (size_t)kn * G;
  float sq = 0.f;
  for (int i = threadIdx.x; i < hs; i += kThreads) {
    const int g = i / gs;
    float acc = 0.f;
    for (int o = 0; o < taps; ++o) {
      float ov = 0.f;
      for (int s = 0; s < splits; ++s) ov += opart[(size_t)s * ss + (size_t)(r - o) * hs + i];
      acc += (b1[(size_t)o * hs + i] + d1[o * G + g]) * ov;
    }
    const float hn = h[(size_t)r * hs + i] + acc;
    h[(size_t)r * hs + i] = hn;
    sq += hn * hn;
  }
  sq = block_sum(sq, red);
  const float scale = 1.f / sqrtf(sq / hs + eps);
  for (int i = threadIdx.x; i < hs; i += kThreads) {
    const float y = h[(size_t)r * hs + i] * scale * w[i];
    x[(size_t)r * hs + i] = y;
    xa[a_idx(r, i)] = (f16)y;
  }
}

// One head of one row: split-summed values at columns col0 + i and
// col0 + i + hd/2 for the lane's pairs i = lane, lane + 64.
struct Pairs {
  float lo[2], hi[2];
};

__device__ __forceinline__ Pairs load_pairs(const float* part, int splits, long ss, long base,
                                            int half) {
  Pairs p;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + 64 * c;
    p.lo[c] = p.hi[c] = 0.f;
    if (i < half)
      for (int s = 0; s < splits; ++s) {
        p.lo[c] += part[(size_t)s * ss + base + i];
        p.hi[c] += part[(size_t)s * ss + base + i + half];
      }
  }
  return p;
}

// `rms` per head by `gain`, then `rotate` to `pos` (half-split pairs) if rot.
__device__ __forceinline__ void norm_rope(Pairs& p, int hd, const float* gain, float eps,
                                          const float* inv, long pos, int rot) {
  const int half = hd >> 1;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c)
    if (threadIdx.x + 64 * c < half) sq += p.lo[c] * p.lo[c] + p.hi[c] * p.hi[c];
  sq = wave_sum(sq);
  const float scale = 1.f / sqrtf(sq / hd + eps);
  const float fpos = (float)pos;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + 64 * c;
    if (i >= half) continue;
    const float a = p.lo[c] * scale * gain[i];
    const float b = p.hi[c] * scale * gain[i + half];
    if (rot) {
      const float ang = fpos * inv[i];
      float sn, cs;
      sincosf(ang, &sn, &cs);
      p.lo[c] = a * cs - b * sn;
      p.hi[c] = b * cs + a * sn;
    } else {
      p.lo[c] = a;
      p.hi[c] = b;
    }
  }
}

// Block q/k/v: split-summed, q and k normed per head and rotated to a+r;
// q in A-layout per head for the attention, k and v f32 [16][kd].
__global__ __launch_bounds__(64) void k_qkv_post(const float* __restrict__ part, int splits,
                                                 long ss, int nh, int kv, int hd,
                                                 const float* __restrict__ qn,
                                                 const float* __restrict__ kn,
                                                 const float* __restrict__ inv, long pos0,
                                                 int rot, float eps, f16* __restrict__ qa,
                                                 float* __restrict__ kb, float* __restrict__ vb) {
  const int r = blockIdx.x, hh = blockIdx.y;
  const int qd = nh * hd, kd = kv * hd, N = qd + 2 * kd, half = hd >> 1;
  const int col0 = hh < nh ? hh * hd : (hh < nh + kv ? qd + (hh - nh) * hd : qd + kd + (hh - nh - kv) * hd);
  Pairs p = load_pairs(part, splits, ss, (long)r * N + col0, half);
  if (hh < nh + kv) norm_rope(p, hd, hh < nh ? qn : kn, eps, inv, pos0 + r, rot);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + 64 * c;
    if (i >= half) continue;
    if (hh < nh) {
      f16* q = qa + (size_t)hh * 16 * hd;
      q[a_idx(r, i)] = (f16)p.lo[c];
      q[a_idx(r, i + half)] = (f16)p.hi[c];
    } else {
      float* dst = hh < nh + kv ? kb + (size_t)r * kd + (hh - nh) * hd
                                : vb + (size_t)r * kd + (hh - nh - kv) * hd;
      dst[i] = p.lo[c];
      dst[i + half] = p.hi[c];
    }
  }
}

// Settle's keys and values of every layer into the store (`settle_rows`).
__global__ __launch_bounds__(64) void k_settle_kv(const float* __restrict__ part, int splits,
                                                  long ss, int L, int kv, int hd,
                                                  const float* __restrict__ knorm,
                                                  const float* __restrict__ inv,
                                                  const int* __restrict__ rot, long pos0,
                                                  float eps, float* __restrict__ sk,
                                                  float* __restrict__ sv, long cap, long row0) {
  const int r = blockIdx.x, l = blockIdx.y, hh = blockIdx.z;
  const int kd = kv * hd, N = L * 2 * kd, half = hd >> 1;
  const bool isk = hh < kv;
  const int g = isk ? hh : hh - kv;
  Pairs p = load_pairs(part, splits, ss, (long)r * N + (long)l * 2 * kd + (isk ? 0 : kd) + g * hd,
                       half);
  if (isk) norm_rope(p, hd, knorm + (size_t)l * hd, eps, inv, pos0 + r, rot[l]);
  float* dst = (isk ? sk : sv) + ((size_t)l * cap + row0 + r) * kd + (size_t)g * hd;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + 64 * c;
    if (i >= half) continue;
    dst[i] = p.lo[c];
    dst[i + half] = p.hi[c];
  }
}

// -------------------------------------------------------------- attention

// Split-context attention (`Drafter::block`'s inner loop). Block (c, g, z):
// kv head g, its q heads 4z..4z+3, and key chunk c — context keys
// [c·chunk, min(n, (c+1)·chunk)) of the layer's range, or for c == nchunks
// the block's own B keys. Each wave keeps one q head's 16 query rows and an
// online softmax over 32-key steps: S^T = K·Q^T and O^T += V^T·P^T on MFMA,
// K and V converted to f16 in LDS. Writes the chunk's (max, sum, O) for the
// merge.
template <int HD>
__global__ __launch_bounds__(kThreads) void k_attn(const f16* __restrict__ qa,
                                                   const float* __restrict__ sk,
                                                   const float* __restrict__ sv,
                                                   const float* __restrict__ kb,
                                                   const float* __restrict__ vb, int B, int nh,
                                                   int kv, int n, long lo_pos, long a, int window,
                                                   int chunk, int nchunks, float scale,
                                                   float* __restrict__ pacc,
                                                   float2* __restrict__ pml) {
  constexpr int KST = HD + 8;   // LDS row stride of K (halfs)
  constexpr int VST = 32 + 8;   // LDS row stride of V^T (halfs)
  constexpr int EPT = HD / 8;   // staged elements per thread per 32 keys
  __shared__ f16 Ks[32 * KST];
  __shared__ f16 Vt[HD * VST];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x, g = blockIdx.y;
  const int rep = nh / kv;
  const int qi = blockIdx.z * 4 + wave;
  const bool active = qi < rep;
  const int hq = g * rep + min(qi, rep - 1);
  const int kd = kv * HD;
  const bool blk = c == nchunks;
  const int k_first = blk ? 0 : c * chunk;
  const int count = blk ? B : min(chunk, n - k_first);
  const float* kbase = blk ? kb + (size_t)g * HD : sk + (size_t)k_first * kd + (size_t)g * HD;
  const float* vbase = blk ? vb + (size_t)g * HD : sv + (size_t)k_first * kd + (size_t)g * HD;
  const long pos_base = lo_pos + k_first;

  h8 qf[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s)
    qf[s] = *reinterpret_cast<const h8*>(qa + (size_t)hq * 16 * HD + ((size_t)s * 64 + lane) * 8);

  const int r = lane & 15, j = lane >> 4;
  const long lim = window > 0 ? a + r + 1 - window : LONG_MIN;
  float m_run = -INFINITY, l_run = 0.f;
  f4 acc[HD / 16];
#pragma unroll
  for (int d = 0; d < HD / 16; ++d) acc[d] = (f4){0.f, 0.f, 0.f, 0.f};

  // staging: thread t copies key t%32, dims (t/32)·EPT .. +EPT
  const int skey = threadIdx.x & 31, sd0 = (threadIdx.x >> 5) * EPT;
  float4 kreg[EPT / 4], vreg[EPT / 4];
  auto fetch = [&](int k0) {
    const bool ok = k0 + skey < count;
    const float4* kp = reinterpret_cast<const float4*>(kbase + (size_t)(k0 + skey) * kd + sd0);
    const float4* vp = reinterpret_cast<const float4*>(vbase + (size_t)(k0 + skey) * kd + sd0);
#pragma unroll
    for (int e = 0; e < EPT / 4; ++e) {
      kreg[e] = ok ? kp[e] : make_float4(0.f, 0.f, 0.f, 0.f);
      vreg[e] = ok ? vp[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (count > 0) fetch(0);
  for (int k0 = 0; k0 < count; k0 += 32) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT / 4; ++e) {
      const float4 kk = kreg[e], vv = vreg[e];
      *reinterpret_cast<h4*>(&Ks[skey * KST + sd0 + 4 * e]) =
          (h4){(f16)kk.x, (f16)kk.y, (f16)kk.z, (f16)kk.w};
      Vt[(sd0 + 4 * e + 0) * VST + skey] = (f16)vv.x;
      Vt[(sd0 + 4 * e + 1) * VST + skey] = (f16)vv.y;
      Vt[(sd0 + 4 * e + 2) * VST + skey] = (f16)vv.z;
      Vt[(sd0 + 4 * e + 3) * VST + skey] = (f16)vv.w;
    }
    __syncthreads();
    if (k0 + 32 < count) fetch(k0 + 32);

    // scores: st[h][v] = S^T[key 16h + 4j + v][query r]
    f4 st[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      st[hb] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        const h8 ka = *reinterpret_cast<const h8*>(&Ks[(16 * hb + (lane & 15)) * KST + 32 * s + 8 * j]);
        st[hb] = mfma16(ka, qf[s], st[hb]);
      }
    }
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 16 * (e >> 2) + 4 * j + (e & 3);
      const int idx = k0 + key;
      const bool ok = idx < count && (blk || window == 0 || pos_base + idx >= lim);
      p[e] = ok ? st[e >> 2][e & 3] * scale : -INFINITY;
      mx = fmaxf(mx, p[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float corr = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = p[e] == -INFINITY ? 0.f : expf(p[e] - m_new);
      ps += p[e];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * corr + ps;
    m_run = m_new;
    const h8 pb = (h8){(f16)p[0], (f16)p[1], (f16)p[2], (f16)p[3],
                       (f16)p[4], (f16)p[5], (f16)p[6], (f16)p[7]};
#pragma unroll
    for (int d = 0; d < HD / 16; ++d) {
      const f16* vrow = &Vt[(16 * d + (lane & 15)) * VST];
      const h4 v0 = *reinterpret_cast<const h4*>(vrow + 4 * j);
      const h4 v1 = *reinterpret_cast<const h4*>(vrow + 16 + 4 * j);
      const h8 va = (h8){v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      acc[d] = mfma16(va, pb, acc[d] * corr);
    }
  }
  if (!active) return;
  const size_t slot = ((size_t)g * (nchunks + 1) + c) * rep + qi;
  float* po = pacc + (slot * 16 + r) * HD;
#pragma unroll
  for (int d = 0; d < HD / 16; ++d)
#pragma unroll
    for (int v = 0; v < 4; ++v) po[16 * d + 4 * j + v] = acc[d][v];
  if (j == 0) pml[slot * 16 + r] = make_float2(m_run, l_run);
}

// Softmax-merge of the chunks of one (q head, row) → y in A-layout f16.
__global__ void k_attn_merge(const float* __restrict__ pacc, const float2* __restrict__ pml,
                             int nh, int kv, int hd, int nchunks, f16* __restrict__ ya) {
  const int hq = blockIdx.x, r = blockIdx.y, d = threadIdx.x;
  const int rep = nh / kv, g = hq / rep, qi = hq % rep;
  float M = -INFINITY;
  for (int c = 0; c <= nchunks; ++c)
    M = fmaxf(M, pml[(((size_t)g * (nchunks + 1) + c) * rep + qi) * 16 + r].x);
  float L = 0.f, y = 0.f;
  for (int c = 0; c <= nchunks; ++c) {
    const size_t slot = ((size_t)g * (nchunks + 1) + c) * rep + qi;
    const float2 ml = pml[slot * 16 + r];
    if (ml.x == -INFINITY) continue;
    const float f = expf(ml.x - M);
    L += ml.y * f;
    y += pacc[(slot * 16 + r) * hd + d] * f;
  }
  ya[a_idx(r, hq * hd + d)] = (f16)(y / L);
}

// ------------------------------------------------------- top-k, selector

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Exact top-`top` (value desc, index asc) of cnt pairs in LDS; the taken
// entry is retired each round. 256 threads. Writes out_v/out_i[0..top).
__device__ void block_topk(float* sv, int* si, int cnt, int top, float* out_v, int* out_i) {
  __shared__ float rv[4];
  __shared__ int ri[4], ro[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float bv = -INFINITY;
  int bi = INT_MAX, bslot = -1;
  auto rescan = [&]() {
    bv = -INFINITY;
    bi = INT_MAX;
    bslot = -1;
    for (int e = tid; e < cnt; e += kThreads)
      if (better(sv[e], si[e], bv, bi)) {
        bv = sv[e];
        bi = si[e];
        bslot = e;
      }
  };
  rescan();
  for (int it = 0; it < top; ++it) {
    float v = bv;
    int i = bi, ow = tid;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(v, o, 64);
      const int i2 = __shfl_xor(i, o, 64), ow2 = __shfl_xor(ow, o, 64);
      if (better(v2, i2, v, i)) {
        v = v2;
        i = i2;
        ow = ow2;
      }
    }
    if (lane == 0) {
      rv[wave] = v;
      ri[wave] = i;
      ro[wave] = ow;
    }
    __syncthreads();
    float V = rv[0];
    int I = ri[0], OW = ro[0];
    for (int w = 1; w < 4; ++w)
      if (better(rv[w], ri[w], V, I)) {
        V = rv[w];
        I = ri[w];
        OW = ro[w];
      }
    if (tid == 0) {
      out_v[it] = V;
      out_i[it] = I;
    }
    if (tid == OW && bslot >= 0) {
      sv[bslot] = -INFINITY;
      si[bslot] = INT_MAX;
      rescan();
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void k_topk_slice(const float* __restrict__ logits,
                                                         int width, int top, int slice,
                                                         int nslices, float* __restrict__ cv,
                                                         int* __restrict__ ci) {
  extern __shared__ float lds[];
  float* sv = lds;
  int* si = reinterpret_cast<int*>(lds + slice);
  const int j = blockIdx.y, sl = blockIdx.x;
  const int b0 = sl * slice, cnt = max(0, min(slice, width - b0));
  const float* row = logits + (size_t)j * width + b0;
  for (int e = threadIdx.x; e < cnt; e += kThreads) {
    sv[e] = row[e];
    si[e] = b0 + e;
  }
  __syncthreads();
  const size_t o = ((size_t)j * nslices + sl) * top;
  block_topk(sv, si, cnt, top, cv + o, ci + o);
}

__global__ __launch_bounds__(kThreads) void k_topk_merge(const float* __restrict__ cv,
                                                         const int* __restrict__ ci, int cnt,
                                                         int top, int* __restrict__ cand,
                                                         float* __restrict__ unary) {
  extern __shared__ float lds[];
  float* sv = lds;
  int* si = reinterpret_cast<int*>(lds + cnt);
  const int j = blockIdx.x;
  for (int e = threadIdx.x; e < cnt; e += kThreads) {
    sv[e] = cv[(size_t)j * cnt + e];
    si[e] = ci[(size_t)j * cnt + e];
  }
  __syncthreads();
  block_topk(sv, si, cnt, top, unary + (size_t)j * top, cand + (size_t)j * top);
}

// `select_with`'s chain. Every (row j, predecessor candidate tp, candidate t)
// score unary + Σ_r (P[prev]·hp[j])[r]·C[tok][r] is formed in parallel (the
// predecessor of row j ≥ 1 is one of row j−1's candidates), then one thread
// walks the rows keeping the first strict maximum.
__global__ __launch_bounds__(kThreads) void k_select(const int* __restrict__ cand,
                                                     const float* __restrict__ unary,
                                                     const float* __restrict__ hp, int k, int top,
                                                     int rank, const f16* __restrict__ pbook,
                                                     const f16* __restrict__ cbook, int vocab,
                                                     int anchor, const int* __restrict__ forced,
                                                     float* __restrict__ score,
                                                     int* __restrict__ chosen) {
  extern __shared__ float tab[];
  const int tpn = forced ? 1 : top;
  const int total = top + (k - 1) * tpn * top;
  for (int e = threadIdx.x; e < total; e += kThreads) {
    int j, tp, t;
    if (e < top) {
      j = 0;
      tp = 0;
      t = e;
    } else {
      const int f = e - top;
      j = 1 + f / (tpn * top);
      tp = (f / top) % tpn;
      t = f % top;
    }
    const int prev = j == 0 ? anchor : (forced ? forced[j] : cand[(size_t)(j - 1) * top + tp]);
    const int tok = cand[(size_t)j * top + t];
    if (prev < 0 || prev >= vocab || tok < 0 || tok >= vocab) {  // no such token: never chosen
      tab[e] = -INFINITY;
      continue;
    }
    const f16* P = pbook + (size_t)prev * rank;
    const f16* C = cbook + (size_t)tok * rank;
    const float* H = hp + (size_t)j * rank;
    float dot = 0.f;
    for (int q = 0; q < rank; ++q) dot += ((float)P[q] * H[q]) * (float)C[q];
    tab[e] = unary[(size_t)j * top + t] + dot;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int tp = 0;
  for (int j = 0; j < k; ++j) {
    const float* row = tab + (j == 0 ? 0 : top + (size_t)(j - 1) * tpn * top + (size_t)tp * top);
    float best = -INFINITY;
    int bt = 0;
    for (int t = 0; t < top; ++t) {
      score[(size_t)j * top + t] = row[t];
      if (row[t] > best) {
        best = row[t];
        bt = t;
      }
    }
    chosen[j] = cand[(size_t)j * top + bt];
    tp = forced ? 0 : bt;
  }
}

// --------------------------------------------------------------- debug

__global__ void k_dequant_i4(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                             TileMap mp, int rows, int K, float* __restrict__ out) {
  const long idx = (long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long)rows * K) return;
  const int row = idx / K, k = idx % K;
  const int t = row >> 4, n = row & 15, KT = K >> 7;
  const long st = map_tile(mp, t);
  const int p = k >> 7, u = (k >> 5) & 3, j = (k >> 3) & 3, e = k & 7;
  const uint32_t word = codes[(((size_t)st * KT + p) * 64 + j * 16 + n) * 4 + u];
  const int pos = (e & 1) ? 16 + 2 * (e - 1) : 2 * e;
  const int q = (int)((word >> pos) & 15u) - 8;
  const uint16_t sb = scales[(((size_t)st * KT + p) * 16 + n) * 4 + u];
  out[idx] = (float)q * half_bits(sb);
}

__global__ void k_sum_rows(const float* __restrict__ part, int splits, long ss, int rows, int N,
                           float* __restrict__ out) {
  const long idx = (long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long)rows * N) return;
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += part[(size_t)s * ss + idx];
  out[idx] = v;
}

// ------------------------------------------------------------- launchers

static inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }

template <int R>
static void launch_f16(hipStream_t st, const uint16_t* xa, int K, int mblocks, const uint16_t* w,
                       TileMap map, int N, int splits, int sps, float* out, long ss) {
  dim3 grid(cdiv(map.ntiles, 4 * R), splits, mblocks);
  k_gemm_f16<R><<<grid, kThreads, 0, st>>>(reinterpret_cast<const f16*>(xa), K,
                                           reinterpret_cast<const f16*>(w), map, N, sps, out, ss);
}

void gemm_f16(hipStream_t st, const uint16_t* xa, int K, int mblocks, const uint16_t* w,
              TileMap map, int N, int splits, int sps, float* out, long ss) {
  launch_f16<2>(st, xa, K, mblocks, w, map, N, splits, sps, out, ss);
}

void gemm_i4(hipStream_t st, const uint16_t* xa, int K, int mblocks, const uint8_t* codes,
             const uint16_t* scales, TileMap map, int N, int splits, int pps, float* out,
             long ss) {
  dim3 grid(cdiv(map.ntiles, 4), splits, mblocks);
  k_gemm_i4<1><<<grid, kThreads, 0, st>>>(reinterpret_cast<const f16*>(xa), K,
                                          reinterpret_cast<const uint4*>(codes),
                                          reinterpret_cast<const uint2*>(scales), map, N, pps, out,
                                          ss);
}

void gemm_glu(hipStream_t st, const uint16_t* xa, int K, const uint8_t* codes,
              const uint16_t* scales, int ftiles, uint16_t* ma) {
  k_gemm_glu<<<ftiles / 2, kThreads, 0, st>>>(reinterpret_cast<const f16*>(xa), K,
                                              reinterpret_cast<const uint4*>(codes),
                                              reinterpret_cast<const uint2*>(scales), ftiles,
                                              reinterpret_cast<f16*>(ma));
}

void head_sel(hipStream_t st, const uint16_t* xa, int K, const uint16_t* head, int width, int k,
              float* logits, const uint16_t* sel, int rank, float* hp) {
  const int wtiles = cdiv(width, 16), stiles = cdiv(rank, 16);
  const int hg = cdiv(wtiles, 16), sg = cdiv(stiles, 16);
  k_head<<<hg + sg, kThreads, 0, st>>>(reinterpret_cast<const f16*>(xa), K,
                                       reinterpret_cast<const f16*>(head), wtiles, width, k, logits,
                                       reinterpret_cast<const f16*>(sel), stiles, rank, hp, hg);
}

void to_a(hipStream_t st, const float* x, long ld, int m, int K, uint16_t* xa) {
  dim3 grid(cdiv((long)(K / 8) * 16, kThreads), cdiv(m, 16));
  k_to_a<<<grid, kThreads, 0, st>>>(x, ld, m, K, reinterpret_cast<f16*>(xa));
}

void sum_norm(hipStream_t st, const float* part, int splits, long ss, int rows, int N,
              const float* w, float eps, uint16_t* xa) {
  k_sum_norm<<<rows, kThreads, 0, st>>>(part, splits, ss, N, w, eps, reinterpret_cast<f16*>(xa));
}

void embed_norm(hipStream_t st, const uint16_t* embed, int anchor, int mask, int rows, int hs,
                const float* w, float eps, float* h, float* x, uint16_t* xa) {
  k_embed_norm<<<rows, kThreads, 0, st>>>(reinterpret_cast<const f16*>(embed), anchor, mask, hs, w,
                                          eps, h, x, reinterpret_cast<f16*>(xa));
}

void conv0(hipStream_t st, const float* x, const float* dpart, int splits, long ss,
           const float* base, int rows, int hs, int gs, int kn, uint16_t* xca, float* dsum) {
  const size_t lds = sizeof(float) * 2 * kn * (hs / gs);
  k_conv0<<<rows, kThreads, lds, st>>>(x, dpart, splits, ss, base, hs, gs, kn,
                                       reinterpret_cast<f16*>(xca), dsum);
}

void conv1_norm(hipStream_t st, float* h, const float* opart, int splits, long ss,
                const float* dsum, const float* base, int rows, int hs, int gs, int kn,
                const float* w, float eps, float* x, uint16_t* xa) {
  k_conv1_norm<<<rows, kThreads, 0, st>>>(h, opart, splits, ss, dsum, base, hs, gs, kn, w, eps, x,
                                          reinterpret_cast<f16*>(xa));
}

void qkv_post(hipStream_t st, const float* part, int splits, long ss, int rows, int nh, int kv,
              int hd, const float* q_norm, const float* k_norm, const float* inv, long pos0,
              int rot, float eps, uint16_t* qa, float* kb, float* vb) {
  dim3 grid(rows, nh + 2 * kv);
  k_qkv_post<<<grid, 64, 0, st>>>(part, splits, ss, nh, kv, hd, q_norm, k_norm, inv, pos0, rot, eps,
                                  reinterpret_cast<f16*>(qa), kb, vb);
}

void settle_kv(hipStream_t st, const float* part, int splits, long ss, int rows, int layers,
               int kv, int hd, const float* k_norm, const float* inv, const int* rot, long pos0,
               float eps, float* sk, float* sv, long cap, long row0) {
  dim3 grid(rows, layers, 2 * kv);
  k_settle_kv<<<grid, 64, 0, st>>>(part, splits, ss, layers, kv, hd, k_norm, inv, rot, pos0, eps,
                                   sk, sv, cap, row0);
}

void attention(hipStream_t st, const uint16_t* qa, const float* sk, const float* sv,
               const float* kb, const float* vb, int B, int nh, int kv, int hd, int n,
               long lo_pos, long a, int window, int chunk, int nchunks, float scale, float* pacc,
               float* pml) {
  const int rep = nh / kv;
  dim3 grid(nchunks + 1, kv, cdiv(rep, 4));
  const f16* q = reinterpret_cast<const f16*>(qa);
  float2* ml = reinterpret_cast<float2*>(pml);
  if (hd == 64)
    k_attn<64><<<grid, kThreads, 0, st>>>(q, sk, sv, kb, vb, B, nh, kv, n, lo_pos, a, window,
                                          chunk, nchunks, scale, pacc, ml);
  else if (hd == 128)
    k_attn<128><<<grid, kThreads, 0, st>>>(q, sk, sv, kb, vb, B, nh, kv, n, lo_pos, a, window,
                                           chunk, nchunks, scale, pacc, ml);
  else
    k_attn<256><<<grid, kThreads, 0, st>>>(q, sk, sv, kb, vb, B, nh, kv, n, lo_pos, a, window,
                                           chunk, nchunks, scale, pacc, ml);
}

void attn_merge(hipStream_t st, const float* pacc, const float* pml, int nh, int kv, int hd,
                int nchunks, int B, uint16_t* ya) {
  dim3 grid(nh, B);
  k_attn_merge<<<grid, hd, 0, st>>>(pacc, reinterpret_cast<const float2*>(pml), nh, kv, hd, nchunks,
                                    reinterpret_cast<f16*>(ya));
}

void topk_slice(hipStream_t st, const float* logits, int k, int width, int top, int slice,
                int nslices, float* cv, int* ci) {
  dim3 grid(nslices, k);
  k_topk_slice<<<grid, kThreads, (size_t)slice * 8, st>>>(logits, width, top, slice, nslices, cv, ci);
}

void topk_merge(hipStream_t st, const float* cv, const int* ci, int k, int cnt, int top, int* cand,
                float* unary) {
  k_topk_merge<<<k, kThreads, (size_t)cnt * 8, st>>>(cv, ci, cnt, top, cand, unary);
}

void select_chain(hipStream_t st, const int* cand, const float* unary, const float* hp, int k,
                  int top, int rank, const uint16_t* pbook, const uint16_t* cbook, int vocab,
                  int anchor, const int* forced, float* score, int* chosen) {
  const int tpn = forced ? 1 : top;
  const size_t lds = sizeof(float) * (size_t)(top + (k - 1) * tpn * top);
  k_select<<<1, kThreads, lds, st>>>(cand, unary, hp, k, top, rank,
                                     reinterpret_cast<const f16*>(pbook),
                                     reinterpret_cast<const f16*>(cbook), vocab, anchor, forced,
                                     score, chosen);
}

void dequant_i4(hipStream_t st, const uint8_t* codes, const uint16_t* scales, TileMap map,
                int rows, int K, float* out) {
  k_dequant_i4<<<cdiv((long)rows * K, kThreads), kThreads, 0, st>>>(
      reinterpret_cast<const uint32_t*>(codes), scales, map, rows, K, out);
}

void sum_rows(hipStream_t st, const float* part, int splits, long ss, int rows, int N,
              float* out) {
  k_sum_rows<<<cdiv((long)rows * N, kThreads), kThreads, 0, st>>>(part, splits, ss, rows, N, out);
}

}  // namespace dfl
