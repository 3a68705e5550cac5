// gate/up with SwiGLU at 16 rows, streamed: the whole K of a tile pair in
// one workgroup, the weights read once as a stream (the two f16 planes of the
// activation are tiny next to them).
//
// Layout of the work: a workgroup of eight waves owns a range of tile pairs
// (gate tile g and up tile ftiles + g of the stored matrix). Wave w holds the
// A fragments of its own KSW spans of K (128 columns each) in registers for
// the whole kernel and walks the workgroup's pairs in order. Its weight loads
// run through a register ring: as soon as one (pair, span) item has been
// multiplied, its registers are refilled with the same span of the next
// pair, so a wave always has loads in flight while it does arithmetic. Each
// wave leaves its partial gate and up tiles of every pair in LDS; after the
// loop the workgroup meets once, sums the eight waves' partials in wave
// order and writes silu(gate)·up into the A-layout planes of the down
// projection.
//
// No global store happens inside the loop: on this architecture stores and
// loads share one wait counter, and a store pending among the loads makes
// every later wait drain all loads in flight.
//
// Compiled with MFMA results in VGPRs (-mllvm -amdgpu-mfma-vgpr-form).
//
// `mlp` (silu(a) = a/(1+e^−a) times up) and the projections follow the
// docs.rs page "cortiq_engine/dflash.rs" (cortiq-engine 0.8.78),
// `Drafter::block`.
#include "device.h"
#include "internal.h"

#include <algorithm>

namespace dfl {

static constexpr int kSW = 8;     // waves per workgroup
static constexpr int kGmax = 8;   // tile pairs a workgroup holds in LDS
static constexpr int kWgs = 256;  // one eight-wave workgroup per compute unit

template <int KSW>
__global__ __launch_bounds__(64 * kSW) void k_glu_stream(const f16* __restrict__ xa, long ps,
                                                         int K, const uint4* __restrict__ codes,
                                                         const uint2* __restrict__ scales,
                                                         int ftiles, f16* __restrict__ ma,
                                                         long mps) {
  __shared__ f4 red[kGmax][2][kSW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KT = K >> 7;
  const int w0 = wave * KSW;
  const int nsp = max(0, min(KSW, KT - w0));         // this wave's spans
  const int nwv = min(kSW, (KT + KSW - 1) / KSW);    // waves with spans
  const int g0 = (int)((long)blockIdx.x * ftiles / gridDim.x);
  const int g1 = (int)((long)(blockIdx.x + 1) * ftiles / gridDim.x);
  if (g0 >= g1) return;  // whole workgroup: no barrier is reached
  const int plast = w0 + max(nsp, 1) - 1;  // clamp for the wave's spare slots

  if (wave < nwv) {
    const uint4* cp = codes + lane;
    const uint2* sp = scales + (lane & 15);
    uint4 c[KSW][2];
    uint2 s[KSW][2];
    // (pair g, span slot u): loads of the gate and the up tile. Past the last
    // pair every wave still issues the same loads, so that every wait in the
    // loop counts the same loads, but of one small block at the matrix's
    // start that all workgroups share (it stays in L2): re-reading the last
    // pair instead was measured as 23 % more HBM traffic.
    auto issue = [&](int g, int u) {
      const bool past = g >= g1;
      const long p = min(w0 + u, plast);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const long tp = past ? 0 : (r == 0 ? g : (long)ftiles + g) * KT + p;
        c[u][r] = ld_stream(&cp[tp * 64]);
        s[u][r] = ld_stream(&sp[tp * 16]);
      }
    };
    h8 a0[KSW][4], a1[KSW][4];
    const h8* x0 = reinterpret_cast<const h8*>(xa) + lane;
    const h8* x1 = reinterpret_cast<const h8*>(xa + ps) + lane;
#pragma unroll
    for (int u = 0; u < KSW; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t i = (size_t)(4 * min(w0 + u, plast) + q) * 64;
        a0[u][q] = x0[i];
        a1[u][q] = x1[i];
      }
#pragma unroll
    for (int u = 0; u < KSW; ++u) issue(g0, u);
#pragma unroll
    for (int u = 0; u < KSW; ++u)
      if (u >= nsp)  // a spare slot adds zero
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a0[u][q] = (h8){};
          a1[u][q] = (h8){};
        }
    for (int g = g0; g < g1; ++g) {
      f4 acc[2] = {(f4){0.f, 0.f, 0.f, 0.f}, (f4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int u = 0; u < KSW; ++u) {
        i4_span_step<2, 2>(c[u], s[u], a0[u], a1[u], acc);
        issue(g + 1, u);
      }
      red[g - g0][0][wave][lane] = acc[0];
      red[g - g0][1][wave][lane] = acc[1];
    }
  }
  lds_barrier();

  const int j = lane >> 4, n = lane & 15;
  for (int g = g0 + wave; g < g1; g += kSW) {
    f4 sg = red[g - g0][0][0][lane], su = red[g - g0][1][0][lane];
    for (int v = 1; v < nwv; ++v) {
      sg += red[g - g0][0][v][lane];
      su += red[g - g0][1][v][lane];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
      put_a(ma, mps, a_idx(4 * j + v, g * 16 + n), sg[v] / (1.f + expf(-sg[v])) * su[v]);
  }
}

bool glu_stream_fits(int K) { return K / 128 <= kSW * 5; }

void gemm_glu_stream(hipStream_t st, const uint16_t* xa, long ps, int K, const uint8_t* codes,
                     const uint16_t* scales, int ftiles, uint16_t* ma, long mps) {
  const int KT = K / 128;
  const int ksw = (KT + kSW - 1) / kSW;
  const int gx = std::max(std::min(ftiles, kWgs), (ftiles + kGmax - 1) / kGmax);
  const f16* x = reinterpret_cast<const f16*>(xa);
  const uint4* c = reinterpret_cast<const uint4*>(codes);
  const uint2* s = reinterpret_cast<const uint2*>(scales);
  f16* m = reinterpret_cast<f16*>(ma);
  // spans per wave: the smallest template constant that covers K
  switch (ksw) {
    case 1: k_glu_stream<1><<<gx, 64 * kSW, 0, st>>>(x, ps, K, c, s, ftiles, m, mps); break;
    case 2: k_glu_stream<2><<<gx, 64 * kSW, 0, st>>>(x, ps, K, c, s, ftiles, m, mps); break;
    case 3: k_glu_stream<3><<<gx, 64 * kSW, 0, st>>>(x, ps, K, c, s, ftiles, m, mps); break;
    case 4: k_glu_stream<4><<<gx, 64 * kSW, 0, st>>>(x, ps, K, c, s, ftiles, m, mps); break;
    default: k_glu_stream<5><<<gx, 64 * kSW, 0, st>>>(x, ps, K, c, s, ftiles, m, mps); break;
  }
}

}  // namespace dfl
