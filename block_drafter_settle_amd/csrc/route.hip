// The router margin (`Route::margin` on the docs.rs page
// "cortiq_engine/dflash.rs", cortiq-engine 0.8.78): for a target row x at
// the tip, u = x / max(‖x‖, 1e-12), and for each of the two subspaces
// (mean μ, basis rows b_r, r < rank; f16 as the sidecar keeps them)
//   err = ‖ d − Σ_r c_r b_r ‖₂,   d = u − μ,   c_r = ⟨d, b_r⟩
// (the page names the reconstruction error without printing it; this is
// the residual's norm after removing the components along the basis rows);
// margin = err(chain) − err(block).
//
// Grids put the row last (blockIdx.y) and the (subspace, basis part) first,
// padded to a multiple of 8: consecutive workgroups go to the 8 XCDs in
// turn, so every row's workgroup for one part of a basis lands on the same
// XCD and the basis is fetched into its L2 once, not once per row.
//
// Three launches, all sums in a fixed order:
//   k_route_coef   block (row, subspace, 16 basis rows): ‖x‖, d in LDS, and
//                  each wave's four c_r (a lane takes 8 channels a step, in
//                  16-byte loads of the basis row);
//   k_route_resid  block (row, subspace, 2048 channels), 8 channels a
//                  thread: e = d − Σ_r c_r b_r and the chunk's Σ e²;
//   k_route_final  per row: the two errors and their difference.
#include "device.h"
#include "internal.h"

#include <algorithm>

namespace dfl {

static constexpr int kRouteRowsPerBlock = 16;  // basis rows a k_route_coef block forms

struct RouteSub {
  const f16* mean;
  const f16* basis;
  int rank;
};

__device__ __forceinline__ const RouteSub& route_sub(const RouteSub& b, const RouteSub& c, int s) {
  return s == 0 ? b : c;
}

// ‖row‖ (floored at 1e-12), every thread of the block gets it
__device__ float route_norm(const float* __restrict__ row, int hidden, float* red) {
  float q = 0.f;
  for (int i = threadIdx.x; i < hidden; i += kThreads) q += row[i] * row[i];
  return fmaxf(sqrtf(block_sum(q, red)), 1e-12f);
}

__global__ __launch_bounds__(kThreads) void k_route_coef(const float* __restrict__ rows,
                                                         int hidden, RouteSub blk, RouteSub chn,
                                                         float* __restrict__ coef,
                                                         float* __restrict__ nrm) {
  __shared__ float d[kRouteMaxHidden];
  __shared__ float red[4];
  const int m = blockIdx.y, s = blockIdx.x & 1, z = blockIdx.x >> 1;
  const RouteSub& sub = route_sub(blk, chn, s);
  const float* row = rows + (size_t)m * hidden;
  const float n = route_norm(row, hidden, red);
  if (z == 0 && threadIdx.x == 0) nrm[m * 2 + s] = n;
  const int r0 = z * kRouteRowsPerBlock;
  if (r0 >= sub.rank) return;  // whole block
  for (int i = threadIdx.x; i < hidden; i += kThreads)
    d[i] = row[i] / n - (float)sub.mean[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kRouteRowsPerBlock / 4; ++j) {
    const int r = r0 + 4 * wave + j;
    if (r >= sub.rank) break;  // uniform in the wave
    const f16* b = sub.basis + (size_t)r * hidden;
    float acc = 0.f;
#pragma unroll 4
    for (int i = 8 * lane; i < hidden; i += 512) {
      const h8 w = *reinterpret_cast<const h8*>(b + i);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)w[e] * d[i + e];
    }
    acc = wave_sum(acc);
    if (lane == 0) coef[(size_t)(m * 2 + s) * kRouteMaxRank + r] = acc;
  }
}

static constexpr int kRouteResidChans = 8 * kThreads;  // channels a k_route_resid block takes

__global__ __launch_bounds__(kThreads) void k_route_resid(const float* __restrict__ rows,
                                                          int hidden, RouteSub blk, RouteSub chn,
                                                          const float* __restrict__ coef,
                                                          const float* __restrict__ nrm,
                                                          float* __restrict__ part, int nchunk) {
  __shared__ float c[kRouteMaxRank];
  __shared__ float red[4];
  const int m = blockIdx.y, s = blockIdx.x & 1, ch = blockIdx.x >> 1;
  if (ch >= nchunk) return;  // padding of the grid (whole workgroup)
  const RouteSub& sub = route_sub(blk, chn, s);
  for (int r = threadIdx.x; r < sub.rank; r += kThreads)
    c[r] = coef[(size_t)(m * 2 + s) * kRouteMaxRank + r];
  __syncthreads();
  const int i0 = ch * kRouteResidChans + 8 * threadIdx.x;
  float q = 0.f;
  if (i0 < hidden) {  // hidden is a multiple of 128: all 8 channels or none
    const float n = nrm[m * 2 + s];
    const float* x = rows + (size_t)m * hidden + i0;
    float e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = x[k] / n - (float)sub.mean[i0 + k];
#pragma unroll 4
    for (int r = 0; r < sub.rank; ++r) {
      const h8 w = *reinterpret_cast<const h8*>(sub.basis + (size_t)r * hidden + i0);
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] -= c[r] * (float)w[k];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) q += e[k] * e[k];
  }
  q = block_sum(q, red);
  if (threadIdx.x == 0) part[(size_t)(m * 2 + s) * nchunk + ch] = q;
}

__global__ __launch_bounds__(64) void k_route_final(const float* __restrict__ part, int nchunk,
                                                    float* __restrict__ margin) {
  const int m = blockIdx.x, lane = threadIdx.x;
  float q[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float a = 0.f;
    for (int k = lane; k < nchunk; k += 64) a += part[(size_t)(m * 2 + s) * nchunk + k];
    q[s] = wave_sum(a);
  }
  if (lane == 0) margin[m] = sqrtf(q[1]) - sqrtf(q[0]);
}

static inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }

int route_chunks(int hidden) { return (int)cdiv(hidden, kRouteResidChans); }

void route_margin(hipStream_t st, const float* rows, int m, int hidden, const uint16_t* bmean,
                  const uint16_t* bbasis, int brank, const uint16_t* cmean,
                  const uint16_t* cbasis, int crank, float* coef, float* nrm, float* part,
                  float* margin) {
  const RouteSub b{reinterpret_cast<const f16*>(bmean), reinterpret_cast<const f16*>(bbasis),
                   brank};
  const RouteSub c{reinterpret_cast<const f16*>(cmean), reinterpret_cast<const f16*>(cbasis),
                   crank};
  const int rz = std::max(1, (int)cdiv(std::max(brank, crank), kRouteRowsPerBlock));
  const int nchunk = route_chunks(hidden);
  const unsigned pad8 = 8;
  k_route_coef<<<dim3(cdiv(2 * rz, pad8) * pad8, m), kThreads, 0, st>>>(rows, hidden, b, c, coef,
                                                                       nrm);
  k_route_resid<<<dim3(cdiv(2 * nchunk, pad8) * pad8, m), kThreads, 0, st>>>(
      rows, hidden, b, c, coef, nrm, part, nchunk);
  k_route_final<<<m, 64, 0, st>>>(part, nchunk, margin);
}

}  // namespace dfl
