// The block pass's 16-row projections with two activation planes: the int4
// q/k/v, o and down, and the f16 kernel projections.
//
// These kernels are compiled on their own with MFMA results in VGPRs
// (-mllvm -amdgpu-mfma-vgpr-form): every MFMA result is scaled by its
// group's f16 scale in VALU right away, which in the accumulator-register
// form costs a v_accvgpr_read per element.
//
// The projections are those of `Drafter::block` on the docs.rs page
// "cortiq_engine/dflash.rs" (cortiq-engine 0.8.78).
#include "device.h"
#include "internal.h"

#include <algorithm>

namespace dfl {

// A 16-row int4 GEMM against two activation planes. Workgroup (g, sp): NW
// waves × R row tiles (tile group g) over spans [sp·KS, sp·KS + KS) of K.
// The workgroup copies the two planes' A fragments of its spans into LDS
// once; every wave issues all of its weight loads before the copy's wait,
// so a wave's whole share is in flight at once. Writes partial sums
// out[sp][m][col].
template <int R, int NW, int KS>
__global__ __launch_bounds__(64 * NW) void k_i4_block(const f16* __restrict__ xa, long ps, int K,
                                                      const uint4* __restrict__ codes,
                                                      const uint2* __restrict__ scales,
                                                      TileMap mp, int N, float* __restrict__ out,
                                                      long split_stride) {
  constexpr int kSteps = KS * 4;                 // 32-column steps a workgroup covers
  constexpr int kFrags = 2 * kSteps * 64;        // h8 fragments of both planes
  constexpr int kPer = (kFrags + 64 * NW - 1) / (64 * NW);
  __shared__ h8 al[2][kSteps][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KT = K >> 7;
  const int sp = blockIdx.y;
  const int p0 = sp * KS, np = min(KS, KT - p0);
  const int t0 = (blockIdx.x * NW + wave) * R;
  // the A copy: fragment e = (plane, step, lane)
  const h8* x0 = reinterpret_cast<const h8*>(xa);
  const h8* x1 = reinterpret_cast<const h8*>(xa + ps);
  h8 areg[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    const int pl = e / (kSteps * 64), st = (e / 64) % kSteps;
    if (e < kFrags && st < np * 4) areg[i] = (pl ? x1 : x0)[(size_t)(p0 * 4 + st) * 64 + (e & 63)];
  }
  uint4 c[KS][R];
  uint2 s[KS][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const long st = map_tile(mp, min(t0 + r, mp.ntiles - 1));
    const uint4* cp = codes + (size_t)st * KT * 64 + lane;
    const uint2* scp = scales + (size_t)st * KT * 16 + (lane & 15);
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int p = p0 + min(u, np - 1);
      c[u][r] = ld_stream(&cp[(size_t)p * 64]);
      s[u][r] = ld_stream(&scp[(size_t)p * 16]);
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    const int pl = e / (kSteps * 64), st = (e / 64) % kSteps;
    if (e < kFrags && st < np * 4) al[pl][st][e & 63] = areg[i];
  }
  // LDS writes done, then a bare s_barrier: a __syncthreads here would also
  // wait for the weight loads still in flight
  lds_barrier();
  f4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    if (u < np) {
      h8 a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = al[0][u * 4 + q][lane];
        b[q] = al[1][u * 4 + q][lane];
      }
      i4_span_deferred<R, 2>(c[u], s[u], a, b, acc);
    }
  }
  if (t0 >= mp.ntiles) return;
  float* o = out + (size_t)sp * split_stride;
  const int j = lane >> 4, n = lane & 15;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r, col = t * 16 + n;
    if (t < mp.ntiles && col < N)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[(size_t)(4 * j + v) * N + col] = acc[r][v];
  }
}

// The 16-row f16 GEMM of the kernel projections, two activation planes:
// as k_i4_block with f16 weight tiles, KS 32-column steps a split. Each
// wave holds all KS·R weight fragments of its share in registers.
template <int R, int NW, int KS>
__global__ __launch_bounds__(64 * NW) void k_f16_block(const f16* __restrict__ xa, long ps, int K,
                                                       const f16* __restrict__ w, TileMap mp,
                                                       int N, float* __restrict__ out,
                                                       long split_stride) {
  constexpr int kFrags = 2 * KS * 64;
  constexpr int kPer = (kFrags + 64 * NW - 1) / (64 * NW);
  __shared__ h8 al[2][KS][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KST = K >> 5;
  const int sp = blockIdx.y;
  const int s0 = sp * KS, ns = min(KS, KST - s0);
  const int t0 = (blockIdx.x * NW + wave) * R;
  const h8* x0 = reinterpret_cast<const h8*>(xa);
  const h8* x1 = reinterpret_cast<const h8*>(xa + ps);
  h8 areg[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    const int pl = e / (KS * 64), st = (e / 64) % KS;
    if (e < kFrags && st < ns) areg[i] = (pl ? x1 : x0)[(size_t)(s0 + st) * 64 + (e & 63)];
  }
  h8 b[KS][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const long st = map_tile(mp, min(t0 + r, mp.ntiles - 1));
    const h8* wp = reinterpret_cast<const h8*>(w) + (size_t)st * KST * 64 + lane;
#pragma unroll
    for (int u = 0; u < KS; ++u) b[u][r] = ld_stream(&wp[(size_t)(s0 + min(u, ns - 1)) * 64]);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    const int pl = e / (KS * 64), st = (e / 64) % KS;
    if (e < kFrags && st < ns) al[pl][st][e & 63] = areg[i];
  }
  lds_barrier();
  f4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    if (u < ns) {
      const h8 a = al[0][u][lane], a2 = al[1][u][lane];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[r] = mfma16(a, b[u][r], acc[r]);
        acc[r] = mfma16(a2, b[u][r], acc[r]);
      }
    }
  }
  if (t0 >= mp.ntiles) return;
  float* o = out + (size_t)sp * split_stride;
  const int j = lane >> 4, n = lane & 15;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r, col = t * 16 + n;
    if (t < mp.ntiles && col < N)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[(size_t)(4 * j + v) * N + col] = acc[r][v];
  }
}

static inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }

// waves per workgroup of k_i4_block; tiles a wave (R) and spans a split
// (ks) are the caller's
static constexpr int kBlkNW = 4;

int i4_block_splits(int K, int ks) { return (int)cdiv(K / 128, ks); }

template <int R, int KS>
static void launch_i4_block(hipStream_t st, const f16* x, long ps, int K, const uint4* c,
                            const uint2* s, TileMap map, int N, float* out, long ss) {
  const dim3 grid(cdiv(map.ntiles, R * kBlkNW), i4_block_splits(K, KS));
  k_i4_block<R, kBlkNW, KS><<<grid, 64 * kBlkNW, 0, st>>>(x, ps, K, c, s, map, N, out, ss);
}

void gemm_i4_block(hipStream_t st, const uint16_t* xa, long ps, int K, const uint8_t* codes,
                   const uint16_t* scales, TileMap map, int N, int R, int ks, float* out,
                   long ss) {
  const f16* x = reinterpret_cast<const f16*>(xa);
  const uint4* c = reinterpret_cast<const uint4*>(codes);
  const uint2* s = reinterpret_cast<const uint2*>(scales);
  // the shapes the callers use: (2, 2) for o and the debug matvec, (2, 8)
  // for q/k/v and down
  (void)R;
  if (ks == 2)
    launch_i4_block<2, 2>(st, x, ps, K, c, s, map, N, out, ss);
  else
    launch_i4_block<2, 8>(st, x, ps, K, c, s, map, N, out, ss);
}


// k_f16_block: two tiles a wave (16 a workgroup), 16 steps (512 columns) a
// split; measured faster on the kernel projections than one tile a wave
static constexpr int kF16R = 2, kF16NW = 8, kF16KS = 16;

int f16_block_splits(int K) { return (int)cdiv(K / 32, kF16KS); }

void gemm_f16_block(hipStream_t st, const uint16_t* xa, long ps, int K, const uint16_t* w,
                    TileMap map, int N, float* out, long ss) {
  const dim3 grid(cdiv(map.ntiles, kF16R * kF16NW), f16_block_splits(K));
  k_f16_block<kF16R, kF16NW, kF16KS><<<grid, 64 * kF16NW, 0, st>>>(
      reinterpret_cast<const f16*>(xa), ps, K, reinterpret_cast<const f16*>(w), map, N, out, ss);
}

}  // namespace dfl
