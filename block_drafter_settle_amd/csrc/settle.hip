// The settle's keys and values of every layer at many rows, straight from
// the int4 codes: K_l = Wk_l·t and V_l = Wv_l·t (`settle_rows` on the docs.rs
// page "cortiq_engine/dflash.rs", cortiq-engine 0.8.78), t the hidden-normed
// rows as two f16 planes (hi, lo).
//
// Compiled with MFMA results in VGPRs (-mllvm -amdgpu-mfma-vgpr-form): each
// 32-column step's products are scaled by the group's f16 scale in VALU at
// once.
#include "device.h"
#include "internal.h"

#include <algorithm>

namespace dfl {

// A block holds all 16 row blocks (256 rows) of both planes against kKvNT
// int4 weight tiles over its K split. Eight waves, two on each SIMD: wave w
// multiplies row blocks 8(w%2)..+7 by tiles 4(w/2)..+3, so each tile's codes
// are decoded by two waves. A 32-column step is exactly one scale group: per
// (row block, tile) it takes t = a_hi·q + a_lo·q on MFMA with the codes q as
// exact f16 integers, then acc += s·t in f32, so the dequantised weight q·s
// enters exactly.
//  - row fragments (both planes): every step through a kKvStages LDS ring,
//    kKvStages − 1 steps ahead; each wave copies four of the 32;
//  - codes and scales: every 128-column span into an LDS double buffer (each
//    wave copies two tiles' codes, non-temporal, and their scales), one span
//    ahead.
// Splits fall on span boundaries, so every step of a split is a real one.
static constexpr int kKvNT = 16, kKvStages = 3, kKvWaves = 8;
static constexpr int kKvA = 32 / kKvWaves;  // row fragments a wave copies a step
static constexpr int kKvC = 3;              // copies a wave issues a span for its codes and scales
static constexpr size_t kKvLds =
    16 * (kKvStages * 2 * 16 * 64 + 2 * kKvNT * 64) + 4 * 2 * kKvNT * 32;  // 132 KB

__global__ __launch_bounds__(64 * kKvWaves) void k_gemm_kv_i4(const f16* __restrict__ xa, long ps,
                                                             int K, int mblocks,
                                                             const uint4* __restrict__ codes,
                                                             const uint32_t* __restrict__ scales,
                                                             TileMap mp, int N, int splits, int sps,
                                                             float* __restrict__ out,
                                                             long split_stride) {
  constexpr int D = kKvStages - 1;
  static_assert(D == 2, "the waits below count two steps of row copies in flight");
  // one dynamic LDS block (kKvLds bytes): row-fragment ring ast[stage][plane]
  // [row block][lane], codes cst[buffer][tile][lane], scales sst[buffer]
  // [tile][(n, pair)]. The waits below order the async copies and the LDS
  // reads. (Into static __shared__ arrays the compiler also waited for every
  // copy in flight before each LDS read, draining the ring every step: the
  // K/V stage of a 256-row settle took 83 against 71 us.)
  extern __shared__ uint4 kv_lds[];
  auto ast = reinterpret_cast<h8(*)[2][16][64]>(kv_lds);
  auto cst = reinterpret_cast<uint4(*)[kKvNT][64]>(kv_lds + kKvStages * 2 * 16 * 64);
  auto sst = reinterpret_cast<uint32_t(*)[kKvNT][32]>(kv_lds + kKvStages * 2 * 16 * 64 +
                                                      2 * kKvNT * 64);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave & 1, cw = wave >> 1;
  const int KT = K >> 7;
  const int sp = blockIdx.x % splits;
  const int p0 = sp * sps, p1 = min(KT, p0 + sps);
  const int s1 = 4 * p1;
  const int t0 = (blockIdx.x / splits) * kKvNT;
  const h8* xg = reinterpret_cast<const h8*>(xa);
  const h8* asrc[kKvA];
#pragma unroll
  for (int i = 0; i < kKvA; ++i) {
    const int f = wave * kKvA + i;  // plane f / 16, row block f % 16
    asrc[i] = xg + (size_t)(f / 16) * (ps / 8) + (size_t)(f % 16) * 2 * K + lane;
  }
  const uint4* csrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    csrc[i] = codes + (size_t)map_tile(mp, min(t0 + 2 * wave + i, mp.ntiles - 1)) * KT * 64 + lane;
  // a dword copy moves 64 dwords: tiles 2w (lanes 0–31) and 2w + 1 (32–63)
  const uint32_t* ssrc =
      scales + (size_t)map_tile(mp, min(t0 + 2 * wave + (lane >> 5), mp.ntiles - 1)) * KT * 32 +
      (lane & 31);
  auto issue_a = [&](int s) {
    const int sc = min(s, s1 - 1);
#pragma unroll
    for (int i = 0; i < kKvA; ++i) {
      const int f = wave * kKvA + i;
      __builtin_amdgcn_global_load_lds(asrc[i] + (size_t)sc * 64, &ast[s % kKvStages][f / 16][f % 16][0],
                                       16, 0, 0);
    }
  };
  auto issue_c = [&](int p) {
    const int pc = min(p, p1 - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(csrc[i] + (size_t)pc * 64, &cst[p & 1][2 * wave + i][0], 16, 0, 2);
    __builtin_amdgcn_global_load_lds(ssrc + (size_t)pc * 32, &sst[p & 1][2 * wave][0], 4, 0, 0);
  };
  f4 acc[8][4];
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[b][t] = (f4){0.f, 0.f, 0.f, 0.f};
  issue_c(p0);
  issue_a(4 * p0);
  issue_a(4 * p0 + 1);
  const int n = lane & 15;
  const uint32_t* cw32 = reinterpret_cast<const uint32_t*>(&cst[0][0][0]);
  for (int p = p0; p < p1; ++p) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = 4 * p + u;
      // this wave's copies of step s (and, at u = 0, of span p) are in: the
      // copies issued after them may remain (those of step s + 1, and at
      // u = 1, 2 also the next span's codes and scales, issued at u = 0)
      if (u == 0 || u == 3)
        wait_vm<kKvA>();
      else
        wait_vm<kKvA + kKvC>();
      lds_barrier();
      issue_a(s + D);
      if (u == 0) issue_c(p + 1);
      // this step's code word and scale of each of the wave's tiles, from the
      // span's buffers (rewritten only after the span's last step)
      h8 q[4];
      float sc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tile = cw * 4 + t;
        q[t] = unpack_i4(cw32[(((size_t)(p & 1) * kKvNT + tile) * 64 + lane) * 4 + u]);
        const uint32_t sb = sst[p & 1][tile][2 * n + (u >> 1)];
        sc[t] = half_bits((u & 1) ? (sb >> 16) : sb);
      }
      const int st = s % kKvStages;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const h8 a0 = ast[st][0][rw * 8 + b][lane];
        const h8 a1 = ast[st][1][rw * 8 + b][lane];
        // a row block's four products first, then their scaling (same
        // operations and order): the MFMAs do not each wait on the FMAs
        // that free one temporary
        f4 v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          v[t] = mfma16(a1, q[t], mfma16(a0, q[t], (f4){0.f, 0.f, 0.f, 0.f}));
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[b][t] += sc[t] * v[t];
      }
    }
  }
  wait_vm<0>();  // the copies issued past the split's end land before the workgroup leaves
  const int j = lane >> 4;
  float* o = out + (size_t)sp * split_stride;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int mb = rw * 8 + b;
    if (mb >= mblocks) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tt = t0 + cw * 4 + t, col = tt * 16 + n;
      if (tt < mp.ntiles && col < N)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[(size_t)(mb * 16 + 4 * j + v) * N + col] = acc[b][t][v];
    }
  }
}

static inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }

int kv_i4_groups(int ntiles) { return (int)cdiv(ntiles, kKvNT); }

void gemm_kv_i4(hipStream_t st, const uint16_t* xa, long ps, int K, int mblocks,
                const uint8_t* codes, const uint16_t* scales, TileMap map, int N, int splits,
                int sps, float* out, long ss) {
  const unsigned blocks = cdiv(map.ntiles, kKvNT) * splits;
  static const hipError_t lds_ok = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm_kv_i4), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kKvLds);
  (void)lds_ok;
  k_gemm_kv_i4<<<blocks, 64 * kKvWaves, kKvLds, st>>>(
      reinterpret_cast<const f16*>(xa), ps, K, mblocks, reinterpret_cast<const uint4*>(codes),
      reinterpret_cast<const uint32_t*>(scales), map, N, splits, sps, out, ss);
}

}  // namespace dfl
