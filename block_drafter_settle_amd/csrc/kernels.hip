// gfx950 kernels of the DFlash 2 drafter's settle and block passes.
//
// What each kernel computes is defined on the docs.rs page
// "cortiq_engine/dflash.rs" (cortiq-engine 0.8.78): `rms`, `rotate`, `conv`,
// `mlp`, `Drafter::block` (the attention), `settle_rows`, `select_with`,
// `top_k`. Operand layouts (A-layout, F16T, I4T, tile maps) are described
// in internal.h.
//
// Every matrix product runs on v_mfma_f32_16x16x32_f16. An activation
// operand is one or two f16 planes (internal.h): with two, the product is
// the sum of both planes' products, so the f32 activation enters with about
// 22 significant bits. int4 codes enter the MFMA as exact small integers
// and each 32-column group's partial is scaled by its f16 scale in f32, so
// the dequantised weight q·s is used exactly. Accumulation is f32
// throughout.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <climits>
#include <math.h>

namespace dfl {

// ------------------------------------------------------------------ GEMMs

// Many-row GEMM, f16 weights, two activation planes (the settle's fc at up
// to 256 rows, and the f16 matrices of the debug product above 16 rows). A
// block holds all 16 row blocks (256 rows; rows past the input are never
// written out) of both planes against kBigNT weight tiles over its K split;
// both planes' products go into one accumulator.
//  - Eight waves, two on each SIMD, each with a 4 × 8-tile accumulator:
//    wave w multiplies row blocks 4(w%4)..+3 of both planes by weight tiles
//    8(w/4)..+7, 64 MFMAs a 32-column step.
//  - Every step's 48 fragments (32 row, 16 weight; 1 KB each, in their
//    memory layout) are copied global → LDS by the waves' async loads
//    (global_load_lds_dwordx4: lane l's 16 bytes land at dst + 16·l), six a
//    wave, into a three-stage ring, two steps ahead; one barrier a step.
//  - A step reads its eight weight fragments, then runs eight groups of
//    eight MFMAs (one row fragment against the eight weight fragments), each
//    group's row fragment read one group ahead: only a couple of LDS reads
//    are in flight, so the MFMAs wait on none but the one they use (with a
//    whole step's reads in flight, the 4-bit LDS counter forces a wait for
//    all of them, and a single wave per SIMD with 256 accumulators leaves the
//    register allocator no room: both measured at half the MFMA rate).
// Blocks are numbered split-fastest.
static constexpr int kBigNT = 16, kBigStages = 3, kBigWaves = 8;
static constexpr int kBigFrags = 2 * 16 + kBigNT;            // fragments a step
static constexpr int kBigPerWave = kBigFrags / kBigWaves;    // async copies a wave issues a step
static constexpr size_t kBigLds = sizeof(h8) * kBigStages * kBigFrags * 64;  // 144 KB
static_assert(kBigFrags % kBigWaves == 0, "every wave copies as many fragments");

__global__ __launch_bounds__(64 * kBigWaves) void k_gemm_big_f16(const f16* __restrict__ xa, long ps, int K, int mblocks,
                    const f16* __restrict__ w, TileMap mp, int N, int splits, int sps,
                    float* __restrict__ out, long split_stride) {
  extern __shared__ h8 stage[];  // [kBigStages][kBigFrags][64]: row fragments (plane, block), then weight tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave & 3, cw = wave >> 2;
  const int KS = K >> 5;
  const int sp = blockIdx.x % splits;
  const int s0 = sp * sps, s1 = min(KS, s0 + sps);
  const int t0 = (blockIdx.x / splits) * kBigNT;
  const h8* xg = reinterpret_cast<const h8*>(xa);
  const h8* wg = reinterpret_cast<const h8*>(w);
  const h8* fsrc[kBigPerWave];  // this wave's fragments at step 0 (uniform)
#pragma unroll
  for (int i = 0; i < kBigPerWave; ++i) {
    const int f = wave * kBigPerWave + i;
    fsrc[i] = f < 32 ? xg + (size_t)(f / 16) * (ps / 8) + (size_t)(f % 16) * 2 * K
                     : wg + (size_t)map_tile(mp, min(t0 + f - 32, mp.ntiles - 1)) * KS * 64;
  }
  // async copies of step s into its stage; past the split's end the last
  // step is copied again, so that every step issues the same loads
  auto issue = [&](int s) {
    const int sc = min(s, s1 - 1);
    h8* dst = stage + (size_t)(s % kBigStages) * kBigFrags * 64 + (wave * kBigPerWave) * 64;
#pragma unroll
    for (int i = 0; i < kBigPerWave; ++i)
      __builtin_amdgcn_global_load_lds(fsrc[i] + (size_t)sc * 64 + lane, dst + i * 64, 16, 0, 0);
  };
  f4 acc[4][8];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[b][t] = (f4){0.f, 0.f, 0.f, 0.f};
  issue(s0);
  issue(s0 + 1);
  for (int s = s0; s < s1; ++s) {
    // the copies of steps up to s + 1 are issued: once this wave's of step
    // s are in (those of s + 1 may remain), the barrier makes the stage of
    // s complete and every wave's reads of step s − 1 done, so its stage
    // takes the copies two steps ahead
    wait_vm<kBigPerWave>();
    lds_barrier();
    issue(s + 2);
    const h8* st = stage + (size_t)(s % kBigStages) * kBigFrags * 64;
    h8 bf[8], af[2];
#pragma unroll
    for (int t = 0; t < 8; ++t) bf[t] = st[(32 + cw * 8 + t) * 64 + lane];
    af[0] = st[(rw * 4) * 64 + lane];
#pragma unroll
    for (int g = 0; g < 8; ++g) {  // group g: plane g / 4, row block 4·rw + g % 4
      if (g + 1 < 8) af[(g + 1) & 1] = st[(((g + 1) / 4) * 16 + rw * 4 + (g + 1) % 4) * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[g % 4][t] = mfma16(af[g & 1], bf[t], acc[g % 4][t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const int j = lane >> 4, n = lane & 15;
  float* o = out + (size_t)sp * split_stride;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int mb = rw * 4 + b;
    if (mb >= mblocks) continue;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tt = t0 + cw * 8 + t, col = tt * 16 + n;
      if (tt < mp.ntiles && col < N)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[(size_t)(mb * 16 + 4 * j + v) * N + col] = acc[b][t][v];
    }
  }
}

template <int R, int PL>
__global__ __launch_bounds__(kThreads) void k_gemm_i4(const f16* __restrict__ xa, long ps, int K,
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
  const h8* xq = reinterpret_cast<const h8*>(xa + ps * (PL - 1) + (size_t)mb * 16 * K) + lane;
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
    h8 a0[4], a1[4], b0[4], b1[4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      c0[r] = ld_stream(&cp[r][(size_t)p * 64]);
      c1[r] = ld_stream(&cp[r][(size_t)(p + 1) * 64]);
      s0[r] = ld_stream(&scp[r][(size_t)p * 16]);
      s1[r] = ld_stream(&scp[r][(size_t)(p + 1) * 16]);
    }
    load_span<PL>(xp, xq, p, a0, b0);
    load_span<PL>(xp, xq, p + 1, a1, b1);
    i4_span_step<R, PL>(c0, s0, a0, b0, acc);
    i4_span_step<R, PL>(c1, s1, a1, b1, acc);
  }
  if (p < p1) {
    uint4 c0[R];
    uint2 s0[R];
    h8 a0[4], b0[4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      c0[r] = ld_stream(&cp[r][(size_t)p * 64]);
      s0[r] = ld_stream(&scp[r][(size_t)p * 16]);
    }
    load_span<PL>(xp, xq, p, a0, b0);
    i4_span_step<R, PL>(c0, s0, a0, b0, acc);
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

// The head over rows 1..k (logits [k][width]) and, in blocks past
// head_groups, the selector projection of all 16 rows (hp [16][rank]).
// Head blocks also record, per draft row, the largest logit of each 256
// columns (gmax [k][ceil(width/256)]) for the selection's threshold, and
// block 0 clears the selection's candidate counters. Each wave covers R
// 16-column tiles, which share every A fragment it loads, and keeps 32 weight
// fragments in flight (32 / R steps of its R tiles); the weights are read
// with non-temporal loads.
template <int PL, int R>
__global__ __launch_bounds__(kThreads) void k_head(const f16* __restrict__ xa, long ps, int K,
                                                   const f16* __restrict__ head, int wtiles,
                                                   int width, int k, float* __restrict__ logits,
                                                   const f16* __restrict__ sel, int stiles,
                                                   int rank, float* __restrict__ hp,
                                                   int head_groups, int ngroups,
                                                   float* __restrict__ gmax,
                                                   int* __restrict__ counters) {
  static_assert(R == 4 || R == 8, "256-column groups are whole waves");
  constexpr int kWpg = 16 / R;  // waves per 256 columns
  constexpr int kGpb = 4 / kWpg;     // 256-column groups per block
  constexpr int U = 32 / R;     // steps a round
  __shared__ float wm[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool is_sel = (int)blockIdx.x >= head_groups;
  const f16* w = is_sel ? sel : head;
  const int ntiles = is_sel ? stiles : wtiles;
  const int grp = is_sel ? blockIdx.x - head_groups : blockIdx.x;
  const int KS = K >> 5;
  const int t0 = (grp * 4 + wave) * R;
  f4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = (f4){0.f, 0.f, 0.f, 0.f};
  if (t0 < ntiles) {
    const h8* xp = reinterpret_cast<const h8*>(xa) + lane;
    const h8* xq = reinterpret_cast<const h8*>(xa + ps * (PL - 1)) + lane;
    const h8* wp[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      wp[r] = reinterpret_cast<const h8*>(w) + (size_t)min(t0 + r, ntiles - 1) * KS * 64 + lane;
    int s = 0;
    for (; s + U <= KS; s += U) {
      h8 a[U], a2[U], b[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[u] = xp[(size_t)(s + u) * 64];
        if (PL == 2) a2[u] = xq[(size_t)(s + u) * 64];
#pragma unroll
        for (int r = 0; r < R; ++r) b[u][r] = ld_stream(&wp[r][(size_t)(s + u) * 64]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r] = mfma16(a[u], b[u][r], acc[r]);
          if (PL == 2) acc[r] = mfma16(a2[u], b[u][r], acc[r]);
        }
    }
    for (; s < KS; ++s) {
      const h8 a = xp[(size_t)s * 64];
      h8 a2;
      if (PL == 2) a2 = xq[(size_t)s * 64];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const h8 b = ld_stream(&wp[r][(size_t)s * 64]);
        acc[r] = mfma16(a, b, acc[r]);
        if (PL == 2) acc[r] = mfma16(a2, b, acc[r]);
      }
    }
  }
  const int j = lane >> 4, n = lane & 15;
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r, col = t * 16 + n;
    if (t >= ntiles) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * j + v;
      if (is_sel) {
        if (col < rank) hp[(size_t)m * rank + col] = acc[r][v];
      } else if (col < width) {
        if (m >= 1 && m <= k) logits[(size_t)(m - 1) * width + col] = acc[r][v];
        mx[v] = fmaxf(mx[v], acc[r][v]);
      }
    }
  }
  if (is_sel) return;  // uniform per block
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx[v] = fmaxf(mx[v], __shfl_xor(mx[v], o, 64));
  if (n == 0)
#pragma unroll
    for (int v = 0; v < 4; ++v) wm[wave][4 * j + v] = mx[v];
  __syncthreads();
  if (threadIdx.x < 16 * kGpb) {
    const int m = threadIdx.x & 15, gh = threadIdx.x >> 4;
    float g = wm[gh * kWpg][m];
#pragma unroll
    for (int w = 1; w < kWpg; ++w) g = fmaxf(g, wm[gh * kWpg + w][m]);
    const int gi = blockIdx.x * kGpb + gh;
    if (m >= 1 && m <= k && gi < ngroups) gmax[(size_t)(m - 1) * ngroups + gi] = g;
    if (blockIdx.x == 0 && gh == 0) counters[m] = 0;
  }
}

// ----------------------------------------------------------- row kernels

// f32 rows → A-layout f16 (plane 1 at xa + ps when ps is nonzero); one
// thread per 8 columns of one row.
__global__ __launch_bounds__(kThreads) void k_to_a(RowSrc x, int m, int K, f16* __restrict__ xa,
                                                   long ps) {
  const int mb = blockIdx.y;
  const long t = (long)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (long)(K >> 3) * 16) return;
  const int i = t & 15, j = (t >> 4) & 3;
  const long s = t >> 6;
  const int row = mb * 16 + i;
  float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (row < m) {
    const int r1 = row - x.n0, r2 = r1 - x.n1;
    const float* src = r1 < 0 ? x.p[0] + (size_t)row * x.ld
                       : r2 < 0 ? x.p[1] + (size_t)r1 * x.ld
                                : x.p[2] + (size_t)r2 * x.ld;
    const float4* p = reinterpret_cast<const float4*>(src + s * 32 + j * 8);
    const float4 lo = p[0], hi = p[1];
    f[0] = lo.x, f[1] = lo.y, f[2] = lo.z, f[3] = lo.w;
    f[4] = hi.x, f[5] = hi.y, f[6] = hi.z, f[7] = hi.w;
  }
  h8 v, r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f16 h, l;
    split_f16(f[e], h, l);
    v[e] = h;
    r[e] = l;
  }
  reinterpret_cast<h8*>(xa + (size_t)mb * 16 * K)[t] = v;
  if (ps) reinterpret_cast<h8*>(xa + ps + (size_t)mb * 16 * K)[t] = r;
}

// The row kernels below split each row into chunks of kChunk channels, one
// workgroup per (chunk, row). The producer of a row writes each chunk's sum
// of squares; `rms` is then finished by its consumer (k_conv0 and
// k_settle_kv scale the projection of h ⊙ gain) or, for the final norm
// before the head, by `k_norm_apply`.
static constexpr int kChunk = 256;

// Split-summed rows (the settle's t = fc·taps), each chunk's Σt², and
// u = t ⊙ w (w: hidden_norm's gain) as the two-plane A-layout operand of the
// settle's K/V projection (plane 1 at xa + ps); rms's per-row scale is applied to that
// projection's output (k_settle_kv), so no separate norm pass runs.
__global__ __launch_bounds__(kThreads) void k_rowsum_sq(const float* __restrict__ part, int splits,
                                                        long ss, int N, const float* __restrict__ w,
                                                        f16* __restrict__ xa, long ps,
                                                        float* __restrict__ sqp, int nchunk) {
  __shared__ float red[4];
  const int r = blockIdx.y, c = blockIdx.x, i = c * kChunk + threadIdx.x;
  float v = 0.f;
  if (i < N) {
    v = sum_splits(part + (size_t)r * N + i, splits, ss);
    put_a(xa, ps, (size_t)(r >> 4) * 16 * N + a_idx(r & 15, i), v * w[i]);
  }
  const float sq = block_sum(v * v, red);
  if (threadIdx.x == 0) sqp[(size_t)r * nchunk + c] = sq;
}

// `rms`: y = h·(1/sqrt(Σh²/N + eps))·w for one 256-channel chunk of row r,
// the row's Σh² gathered from the producer's `nchunk` partial sums (in a
// fixed order, so every chunk of a row gets the same scale); y to f32 (if
// x) and to A-layout f16 planes.
__global__ __launch_bounds__(kThreads) void k_norm_apply(const float* __restrict__ h,
                                                         const float* __restrict__ sqp,
                                                         int nchunk, int N,
                                                         const float* __restrict__ w, float eps,
                                                         float* __restrict__ x,
                                                         f16* __restrict__ xa, long ps) {
  __shared__ float red[4];
  const int r = 16 * blockIdx.z + blockIdx.y, c = blockIdx.x, i = c * kChunk + threadIdx.x;
  float part = 0.f;
  for (int q = threadIdx.x; q < nchunk; q += kThreads) part += sqp[(size_t)r * nchunk + q];
  const float ss = block_sum(part, red);
  const float scale = 1.f / sqrtf(ss / N + eps);
  if (i >= N) return;
  const float y = h[(size_t)r * N + i] * scale * w[i];
  if (x) x[(size_t)r * N + i] = y;
  put_a(xa, ps, (size_t)(r >> 4) * 16 * N + a_idx(r & 15, i), y);
}

// The block's rows [E[anchor], E[mask]…] (f16 → f32), each chunk's Σh²,
// and u = h ⊙ w (w: the first norm's gain) as A-layout f16 planes: the
// kernel projection takes u, and rms's per-row scale is applied to its
// product afterwards (k_conv0), so no separate norm pass runs.
__global__ __launch_bounds__(kThreads) void k_embed(const f16* __restrict__ embed, SeqTok tok,
                                                    int mask, int hs, float* __restrict__ h,
                                                    float* __restrict__ sqp, int nchunk,
                                                    const float* __restrict__ w,
                                                    f16* __restrict__ xa, long ps) {
  __shared__ float red[4];
  // block row m of sequence s (its rows are 16s..16s+15, its A-layout block s)
  const int m = blockIdx.y, sq = blockIdx.z, r = 16 * sq + m;
  const int c = blockIdx.x, i = c * kChunk + threadIdx.x;
  float v = 0.f;
  if (i < hs) {
    v = (float)embed[(size_t)(m == 0 ? tok.t[sq] : mask) * hs + i];
    h[(size_t)r * hs + i] = v;
    put_a(xa, ps, (size_t)sq * 16 * hs + a_idx(m, i), v * w[i]);
  }
  const float ssq = block_sum(v * v, red);
  if (threadIdx.x == 0) sqp[(size_t)r * nchunk + c] = ssq;
}

// Conv stage 0 (`conv`) of row r over a run of whole channel groups, with
// the sub-layer's `rms` folded in. The producer of h left each row's
// partial sums of squares (nchunk of them) and u = h ⊙ w as the kernel
// projection's input, so with s_q = 1/sqrt(Σh_q²/hs + eps):
//   x[q][i] = h[q][i]·s_q·w[i]            (the normed rows)
//   d[r]    = s_r · (Kp·u_r)             (= Kp·x_r)
//   xc[r][i] = Σ_{o ≤ min(kn−1, r)} (base[0][o][i] + d[r][0][o][i/gs])·x[r−o][i].
// The split-summed, scaled kernel projection of these groups, both stages,
// is kept for stage 1.
__global__ __launch_bounds__(kThreads) void k_conv0(const float* __restrict__ h,
                                                    const float* __restrict__ sqp, int nchunk,
                                                    const float* __restrict__ w, float eps,
                                                    const float* __restrict__ dpart, int splits,
                                                    long ss, const float* __restrict__ base,
                                                    int hs, int gs, int kn, int gpw,
                                                    f16* __restrict__ xca, long ps,
                                                    float* __restrict__ dsum) {
  extern __shared__ float dl[];  // [2·kn][ng]
  __shared__ float sc[16];       // s of rows r − o, o < taps (kn ≤ 16)
  // block row m of sequence sq: row r of every row-major buffer
  const int m = blockIdx.y, sq = blockIdx.z, r = 16 * sq + m;
  const int G = hs / gs, P = 2 * kn * G;
  const int g0 = blockIdx.x * gpw, ng = min(G, g0 + gpw) - g0;
  const int taps = min(kn, m + 1);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wave o sums row r − o's partial sums of squares; every workgroup of a
  // row sums them in the same order, so all of them get the same scale. The
  // loads are issued ahead of the projection's split sums below (neither
  // waits for the other).
  float q = 0.f;
  if (wave < taps) {
    // four loads in flight a round (hs/32 ≤ 256 partials take one round)
    const float* sqr = sqp + (size_t)(r - wave) * nchunk;
    for (int c = lane; c < nchunk; c += 256) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = c + 64 * e < nchunk ? sqr[c + 64 * e] : 0.f;
      q += ((v[0] + v[1]) + v[2]) + v[3];
    }
  }
  // the first channel of this thread: its rows, base taps and gain, loaded
  // ahead of the barriers
  constexpr int kPre = 4;
  const int i0 = g0 * gs + threadIdx.x, iend = (g0 + ng) * gs;
  const bool pre = i0 < iend;
  float hx[kPre], bs[kPre], wi = 0.f;
#pragma unroll
  for (int o = 0; o < kPre; ++o) {
    hx[o] = pre && o < taps ? h[(size_t)(r - o) * hs + i0] : 0.f;
    bs[o] = pre && o < taps ? base[(size_t)o * hs + i0] : 0.f;
  }
  if (pre) wi = w[i0];
  for (int e = threadIdx.x; e < 2 * kn * ng; e += kThreads) {
    const int idx = (e / ng) * G + g0 + e % ng;
    dl[e] = sum_splits(dpart + (size_t)r * P + idx, splits, ss);
  }
  q = wave_sum(q);
  if (lane == 0 && wave < taps) sc[wave] = 1.f / sqrtf(q / hs + eps);
  for (int o = wave + kThreads / 64; o < taps; o += kThreads / 64) {  // kn > 4
    float q2 = 0.f;
    for (int c = lane; c < nchunk; c += 64) q2 += sqp[(size_t)(r - o) * nchunk + c];
    q2 = wave_sum(q2);
    if (lane == 0) sc[o] = 1.f / sqrtf(q2 / hs + eps);
  }
  __syncthreads();
  const float sr = sc[0];
  for (int e = threadIdx.x; e < 2 * kn * ng; e += kThreads) {
    const int idx = (e / ng) * G + g0 + e % ng;
    const float v = sr * dl[e];
    dl[e] = v;
    dsum[(size_t)r * P + idx] = v;
  }
  __syncthreads();
  if (pre) {
    const int g = i0 / gs - g0;
    float acc = 0.f;
#pragma unroll
    for (int o = 0; o < kPre; ++o)
      if (o < taps) acc += (bs[o] + dl[o * ng + g]) * (hx[o] * sc[o] * wi);
    for (int o = kPre; o < taps; ++o)
      acc += (base[(size_t)o * hs + i0] + dl[o * ng + g]) * (h[(size_t)(r - o) * hs + i0] * sc[o] * wi);
    put_a(xca, ps, (size_t)sq * 16 * hs + a_idx(m, i0), acc);
  }
  for (int i = i0 + kThreads; i < iend; i += kThreads) {  // conv groups wider than a block
    const int g = i / gs - g0;
    float acc = 0.f;
    for (int o = 0; o < taps; ++o)
      acc += (base[(size_t)o * hs + i] + dl[o * ng + g]) * (h[(size_t)(r - o) * hs + i] * sc[o] * w[i]);
    put_a(xca, ps, (size_t)sq * 16 * hs + a_idx(m, i), acc);
  }
}

// Conv stage 1 of the sub-layer's output into the residual:
// h[r][i] += Σ_o (base[1][o][i] + d[r][1][o][i/gs])·out[r−o][i], out being
// the split-summed GEMM output. One workgroup per kC1 channels and all
// rows: thread (c, r) split-sums out[r] at its channel once, and the taps
// read those sums from LDS. Also each (row, kC1 channels)'s Σh² of the new
// rows, sqp[r][blockIdx.x], and, when w (the next norm's gain) is given,
// u = h ⊙ w as A-layout f16 planes for the next kernel projection (k_conv0
// applies that norm's per-row scale).
static constexpr int kC1 = 32;
__global__ __launch_bounds__(kC1 * 16) void k_conv1(float* __restrict__ h,
                                                    const float* __restrict__ opart, int splits,
                                                    long ss, const float* __restrict__ dsum,
                                                    const float* __restrict__ base, int rows,
                                                    int hs, int gs, int kn,
                                                    float* __restrict__ sqp, int nchunk,
                                                    const float* __restrict__ w,
                                                    f16* __restrict__ xa, long ps) {
  constexpr int kPre = 4;  // taps whose coefficients are loaded ahead of the barrier
  __shared__ float v[16][kC1];
  // block row m of sequence sq (blockIdx.y): row r of every row-major buffer
  const int c = threadIdx.x % kC1, m = threadIdx.x / kC1, sq = blockIdx.y, r = 16 * sq + m;
  const int i = blockIdx.x * kC1 + c;
  const bool live = m < rows && i < hs;
  const int G = hs / gs, P = 2 * kn * G, taps = min(kn, m + 1), g = i / gs;
  const float* b1 = base + (size_t)kn * hs;
  const float* d1 = dsum + (size_t)r * P + (size_t)kn * G;
  // this thread's tap coefficients, old h and gain, loaded together with the
  // split sums (none of them waits for the barrier)
  float coef[kPre], hold = 0.f, wi = 0.f;
#pragma unroll
  for (int o = 0; o < kPre; ++o)
    coef[o] = live && o < taps ? b1[(size_t)o * hs + i] + d1[o * G + g] : 0.f;
  if (live) {
    hold = h[(size_t)r * hs + i];
    if (w) wi = w[i];
  }
  v[m][c] = live ? sum_splits(opart + (size_t)r * hs + i, splits, ss) : 0.f;
  __syncthreads();
  float hn = 0.f;
  if (live) {
    float acc = 0.f;
#pragma unroll
    for (int o = 0; o < kPre; ++o)
      if (o < taps) acc += coef[o] * v[m - o][c];
    for (int o = kPre; o < taps; ++o) acc += (b1[(size_t)o * hs + i] + d1[o * G + g]) * v[m - o][c];
    hn = hold + acc;
    h[(size_t)r * hs + i] = hn;
    if (w) put_a(xa, ps, (size_t)sq * 16 * hs + a_idx(m, i), hn * wi);
  }
  // Σh² over the kC1 channels of row r: the kC1 lanes that hold them
  float q2 = hn * hn;
#pragma unroll
  for (int o = kC1 / 2; o > 0; o >>= 1) q2 += __shfl_xor(q2, o, 64);
  if (c == 0 && m < rows) sqp[(size_t)r * nchunk + blockIdx.x] = q2;
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
    if (i < half) {
      p.lo[c] = sum_splits(part + base + i, splits, ss);
      p.hi[c] = sum_splits(part + base + i + half, splits, ss);
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
// q in A-layout per head for the attention, k and v as f16 pairs in the
// store's form, [kv][16][hi hd | lo hd] a sequence.
__global__ __launch_bounds__(64) void k_qkv_post(const float* __restrict__ part, int splits,
                                                 long ss, int nh, int kv, int hd,
                                                 const float* __restrict__ qn,
                                                 const float* __restrict__ kn,
                                                 const float* __restrict__ inv, SeqPos pos,
                                                 int rot, float eps, f16* __restrict__ qa,
                                                 long qps, f16* __restrict__ kb,
                                                 f16* __restrict__ vb) {
  // block row m of sequence sq (rows 16sq.. of part, kb, vb; its q heads at
  // qa + sq·nh·16·hd), at position a_sq + m
  const int m = blockIdx.x, hh = blockIdx.y, sq = blockIdx.z, r = 16 * sq + m;
  const int qd = nh * hd, kd = kv * hd, N = qd + 2 * kd, half = hd >> 1;
  const int col0 = hh < nh ? hh * hd : (hh < nh + kv ? qd + (hh - nh) * hd : qd + kd + (hh - nh - kv) * hd);
  Pairs p = load_pairs(part, splits, ss, (long)r * N + col0, half);
  if (hh < nh + kv) norm_rope(p, hd, hh < nh ? qn : kn, eps, inv, pos.a[sq] + m, rot);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + 64 * c;
    if (i >= half) continue;
    if (hh < nh) {
      f16* q = qa + ((size_t)sq * nh + hh) * 16 * hd;
      put_a(q, qps, a_idx(m, i), p.lo[c]);
      put_a(q, qps, a_idx(m, i + half), p.hi[c]);
    } else {
      const int g = hh < nh + kv ? hh - nh : hh - nh - kv;
      f16* dst = (hh < nh + kv ? kb : vb) + (size_t)sq * 16 * 2 * kd +
                 ((size_t)g * 16 + m) * 2 * hd;
      put_pair(dst, hd, i, p.lo[c]);
      put_pair(dst, hd, i + half, p.hi[c]);
    }
  }
}

// Settle's keys and values of every layer into the store (`settle_rows`).
__global__ __launch_bounds__(64) void k_settle_kv(const float* __restrict__ part, int splits,
                                                  long ss, int L, int kv, int hd,
                                                  const float* __restrict__ knorm,
                                                  const float* __restrict__ inv,
                                                  const int* __restrict__ rot, long pos0,
                                                  float eps, const float* __restrict__ sqp,
                                                  int nchunk, int hs,
                                                  const StoreSlot* __restrict__ tab, long row0,
                                                  long row_end) {
  const int r = blockIdx.x, l = blockIdx.y, hh = blockIdx.z;
  const StoreSlot so = tab[l];
  // a row that a later row of the same settle call takes the ring place of
  // (cap rows on) is not written: it would race with that row in this launch,
  // and the layer does not keep it
  if (row0 + r < row_end - so.cap) return;
  const int kd = kv * hd, N = L * 2 * kd, half = hd >> 1;
  const bool isk = hh < kv;
  const int g = isk ? hh : hh - kv;
  Pairs p = load_pairs(part, splits, ss, (long)r * N + (long)l * 2 * kd + (isk ? 0 : kd) + g * hd,
                       half);
  // the hidden norm's scale of row r (the projection took t ⊙ w), summed in
  // the same order by every workgroup of the row
  float q = 0.f;
  for (int c = threadIdx.x; c < nchunk; c += 64) q += sqp[(size_t)r * nchunk + c];
  const float sr = 1.f / sqrtf(wave_sum(q) / hs + eps);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    p.lo[c] *= sr;
    p.hi[c] *= sr;
  }
  if (isk) norm_rope(p, hd, knorm + (size_t)l * hd, eps, inv, pos0 + r, rot[l]);
  f16* dst = reinterpret_cast<f16*>(isk ? so.k : so.v) +
             ((size_t)g * so.cap + (row0 + r) % so.cap) * 2 * hd;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + 64 * c;
    if (i >= half) continue;
    put_pair(dst, hd, i, p.lo[c]);
    put_pair(dst, hd, i + half, p.hi[c]);
  }
}

// Rows r0 .. r0+n−1 of a ring of f16-pair rows against f32 rows: one thread
// per value; out: x = hi + lo into lin, else the pair of lin's x.
__global__ __launch_bounds__(kThreads) void k_store_rows(f16* __restrict__ ring, long cap, long r0,
                                                         float* __restrict__ lin, long n, int kv,
                                                         int hd, int out) {
  const long kd = (long)kv * hd, e = (long)blockIdx.x * kThreads + threadIdx.x;
  if (e >= n * kd) return;
  const long i = e / kd;
  const int c = (int)(e - i * kd), g = c / hd, x = c - g * hd;
  f16* row = ring + ((size_t)g * cap + (r0 + i) % cap) * 2 * hd;
  if (out)
    lin[e] = (float)row[x] + (float)row[hd + x];
  else
    put_pair(row, hd, x, lin[e]);
}

// ------------------------------------------------------- top-k, selector

// Orders this wave's LDS accesses (lane 0's writes before every lane's reads).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// `top_k`'s order: the larger value first, the smaller index among equals.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Exact first `want` entries in `top_k` order of up to 64·VPL (value, index)
// pairs held VPL per lane (entry u of lane l is pair l + 64u), by `want`
// rounds of a wave-wide arg-best in which the winning lane retires its entry.
// Lane 0 writes the results to out_v/out_i.
template <int VPL>
__device__ void wave_select(float (&v)[VPL], int (&ix)[VPL], int want, float* out_v,
                            int* out_i) {
  const int lane = threadIdx.x & 63;
  uint64_t taken = 0;
  float bv;
  int bi, bs;
  auto rescan = [&]() {
    bv = -INFINITY;
    bi = INT_MAX;
    bs = -1;
#pragma unroll
    for (int u = 0; u < VPL; ++u)
      if (!((taken >> u) & 1) && better(v[u], ix[u], bv, bi)) {
        bv = v[u];
        bi = ix[u];
        bs = u;
      }
  };
  rescan();
  for (int it = 0; it < want; ++it) {
    float wv = bv;
    int wi = bi, wl = lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(wv, o, 64);
      const int i2 = __shfl_xor(wi, o, 64), l2 = __shfl_xor(wl, o, 64);
      if (better(v2, i2, wv, wi) || (v2 == wv && i2 == wi && l2 < wl)) {
        wv = v2;
        wi = i2;
        wl = l2;
      }
    }
    if (lane == 0) {
      out_v[it] = wv;
      out_i[it] = wi;
    }
    if (lane == wl && bs >= 0) {
      taken |= 1ull << bs;
      rescan();
    }
  }
}

// Selection of the top `top` logits of a row, exactly, in two launches:
//   k_collect  T = the top-th largest of the row's 256-column maxima (at
//              least `top` logits are ≥ T, and only the < top column groups
//              whose maximum exceeds T can hold logits > T), found by every
//              workgroup of the row alike; then every logit > T, and of the
//              logits equal to T the first `top` by index in each
//              2048-column slice, into the row's list;
//   k_pairs    the exact top `top` of that list (it holds the row's top
//              `top` by construction), then the selector's scores.
static constexpr int kSliceVPL = 32;  // a collect wave covers 64·32 = 2048 columns

// The row maxima of 256-column groups (for the selector entry point, whose
// logits do not come from the head kernel); block (0, 0) clears the counters.
__global__ __launch_bounds__(kThreads) void k_rowmax(const float* __restrict__ logits, int width,
                                                     int ngroups, float* __restrict__ gmax,
                                                     int* __restrict__ counters, long lseq) {
  __shared__ float red[4];
  const int g = blockIdx.x, j = blockIdx.y, c = g * 256 + threadIdx.x;
  // sequence blockIdx.z of a batched selection: its logits and its scratch
  logits += blockIdx.z * lseq;
  gmax += (size_t)blockIdx.z * 16 * ngroups;
  counters += blockIdx.z * 16;
  float v = c < width ? logits[(size_t)j * width + c] : -INFINITY;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0)
    gmax[(size_t)j * ngroups + g] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (g == 0 && j == 0 && threadIdx.x < 16) counters[threadIdx.x] = 0;
}

// An unsigned key whose order is the order of the floats (−0 below +0; NaN
// is not produced by the head).
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// T of a row: the top-th largest of its ngroups column-group maxima, by a
// radix select over the maxima's order keys, eight bits a pass from the top:
// each pass counts the candidates still matching the chosen prefix per next
// byte, and a suffix scan over the 256 counts picks the byte holding the
// top-th largest. All kThreads threads of the block call it; every thread
// gets T.
static constexpr int kThreshPer = 8;  // maxima per thread: ngroups ≤ 2048
__device__ float row_threshold(const float* __restrict__ gm, int ngroups, int top) {
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ uint32_t sel[2];  // chosen byte, rank still wanted inside it
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (ngroups < top) return -INFINITY;  // fewer groups than candidates: every logit is one
  uint32_t key[kThreshPer];
#pragma unroll
  for (int u = 0; u < kThreshPer; ++u) {
    const int e = t + kThreads * u;
    key[u] = e < ngroups ? order_key(gm[e]) : 0u;
  }
  uint32_t prefix = 0, mask = 0;
  int want = top;  // rank (1-based) of the wanted key among those matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kThreshPer; ++u)
      if (t + kThreads * u < ngroups && (key[u] & mask) == prefix)
        atomicAdd(&hist[(key[u] >> shift) & 255], 1);
    __syncthreads();
    // suffix sums over bytes: thread t holds byte 255 − t, so an inclusive
    // prefix scan over t is the count of keys with byte ≥ 255 − t
    const int c = hist[255 - t];
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    for (int w = 0; w < wave; ++w) inc += wsum[w];
    const int above = inc - c;  // keys with a larger byte
    if (above < want && inc >= want) {
      sel[0] = 255 - t;
      sel[1] = want - above;
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    mask |= 255u << shift;
    want = (int)sel[1];
    __syncthreads();
  }
  return key_float(prefix);
}

// Append (value, index) for the lanes with `take`, in lane order, to row j's list.
__device__ __forceinline__ void append(bool take, float v, int idx, int* counter, float* lv,
                                       int* li, int cap) {
  const uint64_t mask = __ballot(take);
  if (!mask) return;
  const int lane = threadIdx.x & 63;
  int base = 0;
  if (lane == 0) base = atomicAdd(counter, __popcll(mask));
  base = __shfl(base, 0, 64);
  const int pos = base + __popcll(mask & ((1ull << lane) - 1));
  if (take && pos < cap) {
    lv[pos] = v;
    li[pos] = idx;
  }
}

__global__ __launch_bounds__(kThreads) void k_collect(const float* __restrict__ logits, int width,
                                                      int top, int nslices,
                                                      const float* __restrict__ gmax, int ngroups,
                                                      int* __restrict__ counters,
                                                      float* __restrict__ lv, int* __restrict__ li,
                                                      int cap, long lseq) {
  const int lane = threadIdx.x & 63, j = blockIdx.y;
  logits += blockIdx.z * lseq;
  gmax += (size_t)blockIdx.z * 16 * ngroups;
  counters += blockIdx.z * 16;
  lv += (size_t)blockIdx.z * 16 * cap;
  li += (size_t)blockIdx.z * 16 * cap;
  const int sl = blockIdx.x * 4 + (threadIdx.x >> 6);
  // every workgroup of row j finds the same T (the whole block, before any
  // wave leaves)
  const float T = row_threshold(gmax + (size_t)j * ngroups, ngroups, top);
  if (sl >= nslices) return;
  // a slice whose 256-column groups all peak below T holds no logit ≥ T:
  // skip it without reading its logits
  constexpr int kGroups = 64 * kSliceVPL / 256;
  const int g = sl * kGroups + lane;
  const bool hot = lane < kGroups && g < ngroups && gmax[(size_t)j * ngroups + g] >= T;
  if (!__ballot(hot)) return;
  const int b0 = sl * 64 * kSliceVPL;
  const float* row = logits + (size_t)j * width;
  float v[kSliceVPL];
#pragma unroll
  for (int u = 0; u < kSliceVPL; ++u) {
    const int e = b0 + lane + 64 * u;
    v[u] = e < width ? row[e] : -INFINITY;
  }
  float* rv = lv + (size_t)j * cap;
  int* ri = li + (size_t)j * cap;
#pragma unroll
  for (int u = 0; u < kSliceVPL; ++u) append(v[u] > T, v[u], b0 + lane + 64 * u, counters + j, rv, ri, cap);
  // ties at T: the first `top` of this slice in index order (u major, lane minor)
  int taken = 0;
  for (int u = 0; u < kSliceVPL && taken < top; ++u) {
    const int e = b0 + lane + 64 * u;
    const bool eq = e < width && v[u] == T;
    const uint64_t mask = __ballot(eq);
    const int rank_in = __popcll(mask & ((1ull << lane) - 1));
    const bool take = eq && rank_in < top - taken;
    append(take, v[u], e, counters + j, rv, ri, cap);
    taken += min(__popcll(mask), top - taken);
  }
}

// The exact top `want` of row's list (count entries), in `top_k` order, into
// out_v/out_i (LDS, ≥ 32 + 64 entries): passes of up to 64·VPL entries,
// each pass re-selecting from the best so far plus new entries.
template <int VPL>
__device__ void list_pass(const float* rv, const int* ri, int e0, int n_new, float* best_v,
                          int* best_i, int nbest, int want) {
  const int lane = threadIdx.x & 63;
  float v[VPL];
  int ix[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const int e = lane + 64 * u;  // entries [0, nbest) are the best so far
    if (e < nbest) {
      v[u] = best_v[e];
      ix[u] = best_i[e];
    } else if (e < nbest + n_new) {
      v[u] = rv[e0 + e - nbest];
      ix[u] = ri[e0 + e - nbest];
    } else {
      v[u] = -INFINITY;
      ix[u] = INT_MAX;
    }
  }
  wave_lds_sync();
  wave_select<VPL>(v, ix, want, best_v, best_i);
  wave_lds_sync();
}

__device__ void select_list(const float* rv, const int* ri, int count, int want, float* best_v,
                            int* best_i) {
  int nbest = 0, e0 = 0;
  do {
    const int room = 64 * 64 - nbest;
    const int n_new = min(count - e0, room);
    const int tot = nbest + n_new;
    if (tot <= 64)
      list_pass<1>(rv, ri, e0, n_new, best_v, best_i, nbest, want);
    else if (tot <= 256)
      list_pass<4>(rv, ri, e0, n_new, best_v, best_i, nbest, want);
    else if (tot <= 1024)
      list_pass<16>(rv, ri, e0, n_new, best_v, best_i, nbest, want);
    else
      list_pass<64>(rv, ri, e0, n_new, best_v, best_i, nbest, want);
    nbest = want;
    e0 += n_new;
  } while (e0 < count);
}

// The first `want` entries in `top_k` order of a row's list of n ≤ kRankMax
// entries, by rank, within one wave: an entry's rank is the number of
// entries better than it (a strict order, indices being distinct), so the
// entry of rank q < want lands at out[q]. The list is staged in the wave's
// LDS (sv, si).
static constexpr int kRankMax = 512;
__device__ void rank_select(const float* rv, const int* ri, int n, int want, float* sv, int* si,
                            float* out_v, int* out_i) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < n; e += 64) {
    sv[e] = rv[e];
    si[e] = ri[e];
  }
  wave_lds_sync();
  for (int e = lane; e < n; e += 64) {
    const float v = sv[e];
    const int i = si[e];
    int rank = 0;
    for (int f = 0; f < n; ++f) rank += better(sv[f], si[f], v, i);
    if (rank < want) {
      out_v[rank] = v;
      out_i[rank] = i;
    }
  }
  wave_lds_sync();
}

// Row j's top candidates and row j−1's (j ≥ 1: its candidates are row j's
// predecessors), then the scores of row j's candidates under every
// predecessor (or the anchor for j = 0, or forced[j]), `select_with`:
// unary + Σ_q (P[prev][q]·hp[j][q])·C[tok][q]. One block per row: wave 0
// selects row j and wave 1 row j−1 at the same time (lists longer than
// kRankMax take wave_select passes instead); the predecessors' P rows times
// hp[j], and the candidates' C rows, are staged in LDS once; each thread
// then forms whole dot products, and each table row's first largest score
// (the chain's choice for that predecessor) is found in the block.
static constexpr int kSelTop = 32, kSelRank = 256;
__global__ __launch_bounds__(256) void k_pairs(const float* __restrict__ lv,
                                               const int* __restrict__ li,
                                               const int* __restrict__ counters, int cap, int top,
                                               int tpn, const float* __restrict__ hp, int rank,
                                               const f16* __restrict__ pbook,
                                               const f16* __restrict__ cbook, int vocab,
                                               SeqTok anchors, long hseq,
                                               const int* __restrict__ forced,
                                               int* __restrict__ cand, float* __restrict__ unary,
                                               float* __restrict__ tab, int* __restrict__ best) {
  __shared__ float uv[2][32 + 64];
  __shared__ int uc[2][32 + 64];
  __shared__ float sv[2][kRankMax];
  __shared__ int si[2][kRankMax];
  __shared__ float ph[kSelTop][kSelRank];       // P[prev_p]·hp[j]
  __shared__ uint32_t cw[kSelTop][kSelRank / 2 + 1];  // C[tok_u] as f16 pairs (odd row stride)
  __shared__ float sc[kSelTop][kSelTop + 1];
  const int j = blockIdx.x, k = gridDim.x;
  // sequence sq of a batched selection: its lists, projections, table and
  // outputs
  const int sq = blockIdx.z, anchor = anchors.t[sq];
  lv += (size_t)sq * 16 * cap;
  li += (size_t)sq * 16 * cap;
  counters += sq * 16;
  hp += sq * hseq;
  cand += (size_t)sq * k * top;
  unary += (size_t)sq * k * top;
  tab += (size_t)sq * top * (1 + 15 * top);
  best += (size_t)sq * (1 + 15 * top);
  const int t = threadIdx.x, wave = t >> 6;
  const bool prev_row = j > 0 && !forced;
  const int np = j == 0 ? 1 : tpn;  // predecessors: this row's table rows
  if (wave == 0 || (wave == 1 && prev_row)) {
    const int row = j - wave;
    const int n = min(counters[row], cap);
    if (n <= kRankMax)
      rank_select(lv + (size_t)row * cap, li + (size_t)row * cap, n, top, sv[wave], si[wave],
                  uv[wave], uc[wave]);
    else
      select_list(lv + (size_t)row * cap, li + (size_t)row * cap, n, top, uv[wave], uc[wave]);
  }
  __syncthreads();
  if (t < top) {
    cand[(size_t)j * top + t] = uc[0][t];
    unary[(size_t)j * top + t] = uv[0][t];
  }
  const int rh = (rank + 1) >> 1;
  if ((rank & 7) == 0) {
    // 16-byte pieces of the rows (8 values), every thread's loads issued
    // before any is used: one round trip for the codebook gathers
    constexpr int kMaxPer = kSelTop * kSelRank / 8 / 256;  // pieces a thread, at most
    const int r8 = rank >> 3;
    uint4 pv[kMaxPer], cv[kMaxPer];
    float4 h0[kMaxPer], h1[kMaxPer];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int e = t + 256 * i;
      if (e < np * r8) {
        const int pi = e / r8, q0 = 8 * (e - pi * r8);
        const int prev = j == 0 ? anchor : (forced ? forced[j] : uc[1][pi]);
        const bool ok = prev >= 0 && prev < vocab;
        pv[i] = ok ? *reinterpret_cast<const uint4*>(pbook + (size_t)prev * rank + q0)
                   : make_uint4(0, 0, 0, 0);
        h0[i] = *reinterpret_cast<const float4*>(hp + (size_t)j * rank + q0);
        h1[i] = *reinterpret_cast<const float4*>(hp + (size_t)j * rank + q0 + 4);
      }
      if (e < top * r8) {
        const int u = e / r8, q0 = 8 * (e - u * r8);
        const int tok = uc[0][u];
        cv[i] = tok >= 0 && tok < vocab
                    ? *reinterpret_cast<const uint4*>(cbook + (size_t)tok * rank + q0)
                    : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int e = t + 256 * i;
      if (e < np * r8) {
        const int pi = e / r8, q0 = 8 * (e - pi * r8);
        const uint32_t w[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
        const float hv[8] = {h0[i].x, h0[i].y, h0[i].z, h0[i].w, h1[i].x, h1[i].y, h1[i].z, h1[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ph[pi][q0 + 2 * k] = half_bits(w[k]) * hv[2 * k];
          ph[pi][q0 + 2 * k + 1] = half_bits(w[k] >> 16) * hv[2 * k + 1];
        }
      }
      if (e < top * r8) {
        const int u = e / r8, q2 = 4 * (e - u * r8);
        cw[u][q2] = cv[i].x;
        cw[u][q2 + 1] = cv[i].y;
        cw[u][q2 + 2] = cv[i].z;
        cw[u][q2 + 3] = cv[i].w;
      }
    }
  } else {
    for (int e = t; e < np * 2 * rh; e += 256) {  // an odd rank's last pair padded with 0
      const int pi = e / (2 * rh), q = e - pi * 2 * rh;
      const int prev = j == 0 ? anchor : (forced ? forced[j] : uc[1][pi]);
      const bool ok = q < rank && prev >= 0 && prev < vocab;
      ph[pi][q] = ok ? (float)pbook[(size_t)prev * rank + q] * hp[(size_t)j * rank + q] : 0.f;
    }
    for (int e = t; e < top * rh; e += 256) {
      const int u = e / rh, q = 2 * (e - u * rh);
      const int tok = uc[0][u];
      const bool ok = tok >= 0 && tok < vocab;
      const f16* cr = cbook + (size_t)(ok ? tok : 0) * rank;
      const f16 c0 = ok ? cr[q] : (f16)0.f, c1 = ok && q + 1 < rank ? cr[q + 1] : (f16)0.f;
      cw[u][q >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, c0) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, c1) << 16);
    }
  }
  __syncthreads();
  // entry (p, u): threads of a wave share p and take consecutive u
  for (int e = t; e < np * top; e += 256) {
    const int pi = e / top, u = e - pi * top;
    const int prev = j == 0 ? anchor : (forced ? forced[j] : uc[1][pi]);
    const int tok = uc[0][u];
    // eight partial sums, so that the LDS reads of four pairs are in flight
    float dp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int q2 = 0;
    for (; q2 + 4 <= rh; q2 += 4)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = cw[u][q2 + k];
        dp[2 * k] += ph[pi][2 * (q2 + k)] * half_bits(w);
        dp[2 * k + 1] += ph[pi][2 * (q2 + k) + 1] * half_bits(w >> 16);
      }
    for (int k = 0; q2 < rh; ++q2, ++k) {
      const uint32_t w = cw[u][q2];
      dp[2 * k] += ph[pi][2 * q2] * half_bits(w);
      dp[2 * k + 1] += ph[pi][2 * q2 + 1] * half_bits(w >> 16);
    }
    const float dot = ((dp[0] + dp[1]) + (dp[2] + dp[3])) + ((dp[4] + dp[5]) + (dp[6] + dp[7]));
    const bool ok = prev >= 0 && prev < vocab && tok >= 0 && tok < vocab;
    const float score = ok ? uv[0][u] + dot : -INFINITY;
    sc[pi][u] = score;
    const size_t trow = j == 0 ? 0 : 1 + (size_t)(j - 1) * tpn + pi;
    tab[trow * top + u] = score;
  }
  __syncthreads();
  // each table row's first strictly largest score (candidate 0 when every
  // score is −∞)
  for (int pi = t; pi < np; pi += 256) {
    float bv = -INFINITY;
    int bt = 0;
    for (int u = 0; u < top; ++u)
      if (sc[pi][u] > bv) {
        bv = sc[pi][u];
        bt = u;
      }
    best[j == 0 ? 0 : 1 + (size_t)(j - 1) * tpn + pi] = bt;
  }
}

// The chain: row by row, the candidate chosen under the predecessor chosen
// before it. k_pairs already found each (row, predecessor) table row's
// first largest score, so the walk is a chase through that small index
// table in LDS (one thread); then the block copies each row's scores under
// its predecessor and writes the chosen tokens.
__global__ __launch_bounds__(kThreads) void k_chain(const float* __restrict__ tab,
                                                    const int* __restrict__ best,
                                                    const int* __restrict__ cand, int k, int top,
                                                    int tpn, float* __restrict__ score,
                                                    int* __restrict__ chosen) {
  extern __shared__ int lb[];  // best [1 + (k−1)·tpn], then the walk: table row, choice per row
  // sequence blockIdx.z of a batched selection
  tab += (size_t)blockIdx.z * top * (1 + 15 * top);
  best += (size_t)blockIdx.z * (1 + 15 * top);
  cand += (size_t)blockIdx.z * k * top;
  score += (size_t)blockIdx.z * k * top;
  chosen += (size_t)blockIdx.z * k;
  const int nb = 1 + (k - 1) * tpn;
  int* lrow = lb + nb;
  int* lch = lrow + k;
  for (int e = threadIdx.x; e < nb; e += kThreads) lb[e] = best[e];
  __syncthreads();
  if (threadIdx.x == 0) {
    int tp = 0;
    for (int j = 0; j < k; ++j) {
      const int row = j == 0 ? 0 : 1 + (j - 1) * tpn + tp;
      const int t = lb[row];
      lrow[j] = row;
      lch[j] = t;
      tp = tpn == 1 ? 0 : t;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < k * top; e += kThreads) {
    const int j = e / top, t = e - j * top;
    score[e] = tab[(size_t)lrow[j] * top + t];
  }
  if (threadIdx.x < k) chosen[threadIdx.x] = cand[(size_t)threadIdx.x * top + lch[threadIdx.x]];
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
  out[idx] = sum_splits(part + idx, splits, ss);
}

// ------------------------------------------------------------- launchers

// ---------------------------------------------------------------- probes

// Streaming read: every 16-byte element once, each wave over its own
// contiguous chunk, eight 1 KB blocks (64 lanes × 16 B) in flight,
// non-temporal. The xor keeps the loads; sink is written only on an
// impossible value.
__global__ __launch_bounds__(kThreads) void k_probe_read(const u32x4* __restrict__ p, long n,
                                                         uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63;
  const long waves = (long)gridDim.x * (kThreads / 64);
  const long w = (long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const long per = ((n + waves - 1) / waves + 64 * U - 1) / (64 * U) * (64 * U);
  const long b0 = w * per, b1 = min(n, b0 + per);
  uint32_t x = 0;
  long i = b0 + lane;
  for (; i + 64 * (U - 1) < b1; i += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_stream(p + i + 64 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += 64) {
    const u32x4 v = ld_stream(p + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9e3779b9u) sink[0] = x;
}

// Back-to-back MFMAs: 32 independent accumulators a wave, operands in
// registers. sink is written only on an impossible value.
__global__ __launch_bounds__(kThreads) void k_probe_mfma(int steps, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  h8 a[4], b[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = (h8){(f16)(1e-3f * (lane + r))};
#pragma unroll
  for (int t = 0; t < 8; ++t) b[t] = (h8){(f16)(1e-3f * (lane - t))};
  f4 acc[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[r][t] = (f4){0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < steps; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[r][t] = mfma16(a[r], b[t], acc[r][t]);
  float x = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < 8; ++t) x += acc[r][t][0] + acc[r][t][3];
  if (x == 1234.5f) sink[0] = x;
}

static inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }

void gemm_big_f16(hipStream_t st, const uint16_t* xa, long ps, int K, int mblocks,
                  const uint16_t* w, TileMap map, int N, int splits, int sps, float* out,
                  long ss) {
  const unsigned blocks = cdiv(map.ntiles, kBigNT) * splits;
  // the ring takes 144 KB of the compute unit's 160 KB LDS
  static const hipError_t lds_ok = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm_big_f16), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kBigLds);
  (void)lds_ok;  // a refusal surfaces as the launch's error
  k_gemm_big_f16<<<blocks, 64 * kBigWaves, kBigLds, st>>>(
      reinterpret_cast<const f16*>(xa), ps, K, mblocks, reinterpret_cast<const f16*>(w), map, N,
      splits, sps, out, ss);
}

template <int R, int PL>
static void launch_i4(hipStream_t st, const uint16_t* xa, long ps, int K, int mblocks,
                      const uint8_t* codes, const uint16_t* scales, TileMap map, int N, int splits,
                      int pps, float* out, long ss) {
  dim3 grid(cdiv(map.ntiles, 4 * R), splits, mblocks);
  k_gemm_i4<R, PL><<<grid, kThreads, 0, st>>>(reinterpret_cast<const f16*>(xa), ps, K,
                                              reinterpret_cast<const uint4*>(codes),
                                              reinterpret_cast<const uint2*>(scales), map, N, pps,
                                              out, ss);
}

// every caller passes two planes (ps ≠ 0)
void gemm_i4(hipStream_t st, const uint16_t* xa, long ps, int K, int mblocks, const uint8_t* codes,
             const uint16_t* scales, TileMap map, int N, int splits, int pps, float* out, long ss) {
  launch_i4<2, 2>(st, xa, ps, K, mblocks, codes, scales, map, N, splits, pps, out, ss);
}

// Eight tiles a wave need at least this many workgroups (one a compute
// unit); a narrower head (a shortlisted width: 65536 columns give 128) takes
// four tiles a wave and twice the workgroups, which measured 912 -> 842 us a
// 27B block at width 65536.
static constexpr int kHeadMinGroups = 256;

void head_sel(hipStream_t st, const uint16_t* xa, long ps, int K, const uint16_t* head, int width,
              int k, float* logits, const uint16_t* sel, int rank, float* hp, SelectScratch sc) {
  const int wtiles = cdiv(width, 16), stiles = cdiv(rank, 16);
  const f16* x = reinterpret_cast<const f16*>(xa);
  const f16* hw = reinterpret_cast<const f16*>(head);
  const f16* sw = reinterpret_cast<const f16*>(sel);
  // eight tiles a wave while that still gives every compute unit a
  // workgroup, else four (a shortlisted width)
  const bool r8 = cdiv(wtiles, 4 * 8) >= kHeadMinGroups;
  const int R = r8 ? 8 : 4;
  const int hg = cdiv(wtiles, 4 * R), sg = cdiv(stiles, 4 * R);
  const unsigned g = hg + sg;
  const int ng = cdiv(width, 256);
  // two planes (ps ≠ 0), as every caller passes
  if (r8)
    k_head<2, 8><<<g, kThreads, 0, st>>>(x, ps, K, hw, wtiles, width, k, logits, sw, stiles, rank,
                                         hp, hg, ng, sc.gmax, sc.counters);
  else
    k_head<2, 4><<<g, kThreads, 0, st>>>(x, ps, K, hw, wtiles, width, k, logits, sw, stiles, rank,
                                         hp, hg, ng, sc.gmax, sc.counters);
}

void to_a(hipStream_t st, const RowSrc& x, int m, int K, uint16_t* xa, long ps) {
  dim3 grid(cdiv((long)(K / 8) * 16, kThreads), cdiv(m, 16));
  k_to_a<<<grid, kThreads, 0, st>>>(x, m, K, reinterpret_cast<f16*>(xa), ps);
}

void to_a(hipStream_t st, const float* x, long ld, int m, int K, uint16_t* xa, long ps) {
  to_a(st, RowSrc{{x, x, x}, m, 0, ld}, m, K, xa, ps);
}

void rowsum_sq(hipStream_t st, const float* part, int splits, long ss, int rows, int N,
               const float* w, uint16_t* xa, long ps, float* sqp) {
  const int nch = cdiv(N, kChunk);
  k_rowsum_sq<<<dim3(nch, rows), kThreads, 0, st>>>(part, splits, ss, N, w,
                                                    reinterpret_cast<f16*>(xa), ps, sqp, nch);
}

// Probe launches; the caller times them (one workgroup of 256 threads is
// four waves; 512 workgroups place two waves on every SIMD of 256 units).
void probe_read(hipStream_t st, const void* p, long bytes, uint32_t* sink) {
  k_probe_read<<<4096, kThreads, 0, st>>>(reinterpret_cast<const u32x4*>(p), bytes / 16, sink);
}
void probe_mfma(hipStream_t st, int workgroups, int steps, float* sink) {
  k_probe_mfma<<<workgroups, kThreads, 0, st>>>(steps, sink);
}

int row_chunks(int N) { return cdiv(N, kChunk); }
int conv1_chunks(int hs) { return cdiv(hs, kC1); }

void norm_apply(hipStream_t st, const float* h, const float* sqp, int nchunk, int rows, int N,
                const float* w, float eps, float* x, uint16_t* xa, long ps, int nseq) {
  k_norm_apply<<<dim3(cdiv(N, kChunk), rows, nseq), kThreads, 0, st>>>(
      h, sqp, nchunk, N, w, eps, x, reinterpret_cast<f16*>(xa), ps);
}

void embed(hipStream_t st, const uint16_t* emb, const int* anchors, int nseq, int mask, int rows,
           int hs, float* h, float* sqp, const float* w, uint16_t* xa, long ps) {
  const int nch = cdiv(hs, kChunk);
  SeqTok tok{};
  for (int i = 0; i < nseq; ++i) tok.t[i] = anchors[i];
  k_embed<<<dim3(nch, rows, nseq), kThreads, 0, st>>>(reinterpret_cast<const f16*>(emb), tok,
                                                      mask, hs, h, sqp, nch, w,
                                                      reinterpret_cast<f16*>(xa), ps);
}

void conv0(hipStream_t st, const float* h, const float* sqp, int nchunk, const float* w, float eps,
           const float* dpart, int splits, long ss, const float* base, int rows, int hs, int gs,
           int kn, uint16_t* xca, long ps, float* dsum, int nseq) {
  const int G = hs / gs, gpw = std::max(1, kChunk / gs);
  const size_t lds = sizeof(float) * 2 * kn * gpw;
  k_conv0<<<dim3(cdiv(G, gpw), rows, nseq), kThreads, lds, st>>>(
      h, sqp, nchunk, w, eps, dpart, splits, ss, base, hs, gs, kn, gpw,
      reinterpret_cast<f16*>(xca), ps, dsum);
}

void conv1(hipStream_t st, float* h, const float* opart, int splits, long ss, const float* dsum,
           const float* base, int rows, int hs, int gs, int kn, float* sqp, const float* w,
           uint16_t* xa, long ps, int nseq) {
  const int nch = conv1_chunks(hs);
  k_conv1<<<dim3(nch, nseq), kC1 * 16, 0, st>>>(h, opart, splits, ss, dsum, base, rows, hs, gs, kn,
                                                sqp, nch, w, reinterpret_cast<f16*>(xa), ps);
}

void qkv_post(hipStream_t st, const float* part, int splits, long ss, int rows, int nh, int kv,
              int hd, const float* q_norm, const float* k_norm, const float* inv, const long* pos,
              int nseq, int rot, float eps, uint16_t* qa, long qps, uint16_t* kb, uint16_t* vb) {
  dim3 grid(rows, nh + 2 * kv, nseq);
  SeqPos sp{};
  for (int i = 0; i < nseq; ++i) sp.a[i] = pos[i];
  k_qkv_post<<<grid, 64, 0, st>>>(part, splits, ss, nh, kv, hd, q_norm, k_norm, inv, sp, rot, eps,
                                  reinterpret_cast<f16*>(qa), qps, reinterpret_cast<f16*>(kb),
                                  reinterpret_cast<f16*>(vb));
}

void settle_kv(hipStream_t st, const float* part, int splits, long ss, int rows, int layers,
               int kv, int hd, const float* k_norm, const float* inv, const int* rot, long pos0,
               float eps, const float* sqp, int hs, const StoreSlot* tab, long row0,
               long row_end) {
  dim3 grid(rows, layers, 2 * kv);
  k_settle_kv<<<grid, 64, 0, st>>>(part, splits, ss, layers, kv, hd, k_norm, inv, rot, pos0, eps,
                                   sqp, cdiv(hs, kChunk), hs, tab, row0, row_end);
}

void store_rows(hipStream_t st, uint16_t* ring, long cap, long r0, float* lin, long n, int kv,
                int hd, bool out) {
  if (n <= 0) return;
  k_store_rows<<<cdiv(n * kv * hd, kThreads), kThreads, 0, st>>>(
      reinterpret_cast<f16*>(ring), cap, r0, lin, n, kv, hd, out ? 1 : 0);
}

int topk_slices(int width) { return cdiv(width, 64 * kSliceVPL); }

int topk_cap(int width, int top) {
  // logits > T lie in < top column groups of 256; ties add ≤ top a slice
  return ((top - 1) * 256 + top * topk_slices(width) + 63) / 64 * 64;
}

void select_all(hipStream_t st, const float* logits, bool have_gmax, int k, int width, int top,
                const float* hp, int rank, const uint16_t* pbook, const uint16_t* cbook,
                int vocab, int anchor, const int* forced, SelectScratch sc, int* cand,
                float* unary, float* score, int* chosen) {
  select_batch(st, 1, logits, 0, have_gmax, k, width, top, hp, 0, rank, pbook, cbook, vocab,
               &anchor, forced, sc, cand, unary, score, chosen);
}

void select_batch(hipStream_t st, int nseq, const float* logits, long lseq, bool have_gmax, int k,
                  int width, int top, const float* hp, long hseq, int rank,
                  const uint16_t* pbook, const uint16_t* cbook, int vocab, const int* anchors,
                  const int* forced, SelectScratch sc, int* cand, float* unary, float* score,
                  int* chosen) {
  const int ngroups = cdiv(width, 256), ns = topk_slices(width), cap = topk_cap(width, top);
  SeqTok an{};
  for (int i = 0; i < nseq; ++i) an.t[i] = anchors[i];
  if (!have_gmax)
    k_rowmax<<<dim3(ngroups, k, nseq), kThreads, 0, st>>>(logits, width, ngroups, sc.gmax,
                                                          sc.counters, lseq);
  k_collect<<<dim3(cdiv(ns, 4), k, nseq), kThreads, 0, st>>>(logits, width, top, ns, sc.gmax,
                                                             ngroups, sc.counters, sc.lv, sc.li,
                                                             cap, lseq);
  const int tpn = forced ? 1 : top;
  k_pairs<<<dim3(k, 1, nseq), 256, 0, st>>>(sc.lv, sc.li, sc.counters, cap, top, tpn, hp, rank,
                                            reinterpret_cast<const f16*>(pbook),
                                            reinterpret_cast<const f16*>(cbook), vocab, an, hseq,
                                            forced, cand, unary, sc.tab, sc.best);
  const size_t lds = sizeof(int) * ((size_t)(1 + (k - 1) * tpn) + 2 * k);
  k_chain<<<dim3(1, 1, nseq), kThreads, lds, st>>>(sc.tab, sc.best, cand, k, top, tpn, score,
                                                   chosen);
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
