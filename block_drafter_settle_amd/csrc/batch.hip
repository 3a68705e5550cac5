// Batched blocks: the blocks of several sequences that share one drafter's
// weights go through each weight matrix together. Sequence s owns A-layout
// block s of every operand (16 rows; its block's rows first), so the
// products see MB·16 rows (MB = 4 or 8 row blocks, a batch padded to it with
// blocks that are never read back) and every weight tile is read once for
// all of them. The projections are those of `Drafter::block` on the docs.rs
// page "cortiq_engine/dflash.rs" (cortiq-engine 0.8.78), for each sequence.
//
// Compiled with MFMA results in VGPRs (-mllvm -amdgpu-mfma-vgpr-form): the
// int4 kernel scales each 32-column product by its group's scale in VALU.
#include "device.h"
#include "internal.h"

#include <algorithm>

namespace dfl {

// Workgroups of eight waves over 16 weight tiles; wave w multiplies row
// blocks (w % 2)·MB/2 .. +MB/2 of both activation planes by tiles
// 4(w / 2) .. +3 (MB/2 × 4 accumulators): each row fragment a step is read
// from LDS by four waves and each weight tile by two, which keeps the LDS
// reads of a step under its MFMA time. The row fragments of every 32-column step go global → LDS
// by async copies into a three-stage ring, two steps ahead, shared by the
// eight waves.
static constexpr int kMbWaves = 8, kMbNT = 16, kMbStages = 3, kMbAhead = kMbStages - 1;

// int4 weights (I4T tiles): the tiles' codes and scales of every 128-column
// span go to LDS too (a double buffer, one span ahead; wave w copies tiles
// 2w, 2w + 1), and each wave reads its four tiles' codes and scales of a
// span into registers once. Each step is one scale group: t = a_hi·q +
// a_lo·q on the exact integer codes, then acc += s·t in f32. A step holds
// few products, so the row fragments run four steps ahead in a five-stage
// ring (copies from L2 take longer than two steps). Copies past the
// split's end repeat its last step or span (same data into a slot no step
// still reads).
// (The bodies are device templates behind one plain kernel per MB: a
// kernel template whose body holds these copy builtins gets no host stub.)
static constexpr int kMbI4Stages = 5;  // row-fragment ring stages of mb_i4

// LDS of mb_i4<MB>: the ring's stages of both planes' MB row fragments, two
// spans of 16 tiles' codes and their scales
static constexpr size_t mb_i4_lds(int MB) {
  return sizeof(h8) * (kMbI4Stages * 2 * MB * 64 + 2 * kMbNT * 64) +
         sizeof(uint32_t) * 2 * kMbNT * 32;
}

template <int MB>
__device__ __forceinline__ void mb_i4(const f16* __restrict__ xa, long ps, int K,
                                      const uint4* __restrict__ codes,
                                      const uint32_t* __restrict__ scales, TileMap mp, int N,
                                      int mblocks, int splits, int sps, float* __restrict__ out,
                                      long split_stride) {
  constexpr int CA = 2 * MB / kMbWaves;  // row-fragment copies a wave a step
  constexpr int CC = 3;                  // code and scale copies a wave a span
  static_assert(CA >= 1 && 2 * MB % kMbWaves == 0, "every wave copies as many row fragments");
  constexpr int ST = kMbI4Stages, AH = ST - 1;  // row-fragment ring stages, steps ahead
  static_assert(AH == 4, "the waits below count four steps of row fragments in flight");
  // one dynamic LDS block (mb_i4_lds(MB) bytes): the row-fragment ring
  // ast[stage][plane][row block][lane], codes cst[buffer][tile][lane] and
  // scales sst[buffer][tile][(n, pair)]. The waits below order the async
  // copies and the LDS reads (into static __shared__ arrays the compiler also
  // waited for every copy in flight before each LDS read, draining the ring).
  extern __shared__ h8 stage[];
  auto ast = reinterpret_cast<h8(*)[2][MB][64]>(stage);
  auto cst = reinterpret_cast<uint4(*)[kMbNT][64]>(stage + ST * 2 * MB * 64);
  auto sst = reinterpret_cast<uint32_t(*)[kMbNT][32]>(stage + ST * 2 * MB * 64 + 2 * kMbNT * 64);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KT = K >> 7;
  const int sp = blockIdx.x % splits;
  const int p0 = sp * sps, p1 = min(KT, p0 + sps);
  const int s1 = 4 * p1;
  const int t0 = (blockIdx.x / splits) * kMbNT;
  const h8* xg = reinterpret_cast<const h8*>(xa);
  const h8* asrc[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int f = wave * CA + i;  // plane f / MB, row block f % MB
    asrc[i] = xg + (size_t)(f / MB) * (ps / 8) + (size_t)(f % MB) * 2 * K + lane;
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
    for (int i = 0; i < CA; ++i) {
      const int f = wave * CA + i;
      __builtin_amdgcn_global_load_lds(asrc[i] + (size_t)sc * 64,
                                       &ast[s % ST][f / MB][f % MB][0], 16, 0, 0);
    }
  };
  auto issue_c = [&](int p) {
    const int pc = min(p, p1 - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(csrc[i] + (size_t)pc * 64, &cst[p & 1][2 * wave + i][0], 16, 0, 2);
    __builtin_amdgcn_global_load_lds(ssrc + (size_t)pc * 32, &sst[p & 1][2 * wave][0], 4, 0, 0);
  };
  constexpr int RB = MB / 2;
  const int rg = wave & 1, tg = wave >> 1;
  f4 acc[RB][4];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[b][t] = (f4){0.f, 0.f, 0.f, 0.f};
  issue_c(p0);
#pragma unroll
  for (int i = 0; i < AH; ++i) issue_a(4 * p0 + i);
  const int n = lane & 15;
  uint4 cw[4];
  uint2 sw[4];
  for (int p = p0; p < p1; ++p) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = 4 * p + u;
      // Issue order: span p0's codes, the row fragments of steps 4p0 ..
      // 4p0 + 3, then for every step t those of t + 4 and, when t starts
      // span q, the codes of span q + 1. Once this wave's copies of step s
      // and of span p are in, what was issued after them may remain: three
      // steps of row fragments, plus (past a span's first step) the next
      // span's codes.
      if (u == 0)
        wait_vm<3 * CA>();
      else
        wait_vm<3 * CA + CC>();
      lds_barrier();
      issue_a(s + AH);
      if (u == 0) {
        issue_c(p + 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          cw[t] = cst[p & 1][4 * tg + t][lane];
          sw[t] = *reinterpret_cast<const uint2*>(&sst[p & 1][4 * tg + t][2 * n]);
        }
      }
      h8 q[4];
      float sc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        q[t] = unpack_i4(u == 0 ? cw[t].x : u == 1 ? cw[t].y : u == 2 ? cw[t].z : cw[t].w);
        const uint32_t sb = u < 2 ? sw[t].x : sw[t].y;
        sc[t] = half_bits((u & 1) ? (sb >> 16) : sb);
      }
      const int st = s % ST;
      if (MB == 8) {
        // every product of the step first, then their scaling: the MFMAs
        // run back to back instead of waiting on the FMAs that free one
        // temporary (same operations, same order: the same bits)
        f4 v[RB][4];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const h8 a0 = ast[st][0][rg * RB + b][lane];
          const h8 a1 = ast[st][1][rg * RB + b][lane];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v[b][t] = mfma16(a1, q[t], mfma16(a0, q[t], (f4){0.f, 0.f, 0.f, 0.f}));
        }
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[b][t] += sc[t] * v[b][t];
      } else {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const h8 a0 = ast[st][0][rg * RB + b][lane];
          const h8 a1 = ast[st][1][rg * RB + b][lane];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            f4 v = mfma16(a0, q[t], (f4){0.f, 0.f, 0.f, 0.f});
            v = mfma16(a1, q[t], v);
            acc[b][t] += sc[t] * v;
          }
        }
      }
    }
  }
  wait_vm<0>();  // the copies issued past the split's end land before the workgroup leaves
  const int j = lane >> 4;
  float* o = out + (size_t)sp * split_stride;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rb = rg * RB + b;
    if (rb >= mblocks) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tt = t0 + 4 * tg + t, col = tt * 16 + n;
      if (tt < mp.ntiles && col < N)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[(size_t)(rb * 16 + 4 * j + v) * N + col] = acc[b][t][v];
    }
  }
}

// f16 weights (F16T tiles): the 16 weight fragments of a step go through
// the same ring as the row fragments (each wave copies the same number).
template <int MB>
__device__ __forceinline__ void mb_f16(const f16* __restrict__ xa, long ps, int K,
                                       const f16* __restrict__ w, TileMap mp, int N, int mblocks,
                                       int splits, int sps, float* __restrict__ out,
                                       long split_stride) {
  constexpr int FR = 2 * MB + kMbNT;    // fragments a step: row blocks of both planes, tiles
  constexpr int FPW = FR / kMbWaves;    // async copies a wave a step
  static_assert(FR % kMbWaves == 0, "every wave copies as many fragments");
  extern __shared__ h8 stage[];  // [kMbStages][FR][64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KS = K >> 5;
  const int sp = blockIdx.x % splits;
  const int s0 = sp * sps, s1 = min(KS, s0 + sps);
  const int t0 = (blockIdx.x / splits) * kMbNT;
  const h8* xg = reinterpret_cast<const h8*>(xa);
  const h8* wg = reinterpret_cast<const h8*>(w);
  const h8* fsrc[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int f = wave * FPW + i;
    fsrc[i] = f < 2 * MB ? xg + (size_t)(f / MB) * (ps / 8) + (size_t)(f % MB) * 2 * K
                         : wg + (size_t)map_tile(mp, min(t0 + f - 2 * MB, mp.ntiles - 1)) * KS * 64;
  }
  auto issue = [&](int s) {
    const int sc = min(s, s1 - 1);
    h8* dst = stage + (size_t)(s % kMbStages) * FR * 64 + (wave * FPW) * 64;
#pragma unroll
    for (int i = 0; i < FPW; ++i)
      __builtin_amdgcn_global_load_lds(fsrc[i] + (size_t)sc * 64 + lane, dst + i * 64, 16, 0, 0);
  };
  constexpr int RB = MB / 2;
  const int rg = wave & 1, tg = wave >> 1;
  f4 acc[RB][4];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[b][t] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMbAhead; ++i) issue(s0 + i);
  for (int s = s0; s < s1; ++s) {
    // this wave's copies of step s are in (those of s + 1 may remain); the
    // barrier completes the stage and retires every wave's reads of s − 1,
    // whose stage then takes step s + 2
    wait_vm<(kMbAhead - 1) * FPW>();
    lds_barrier();
    issue(s + kMbAhead);
    const h8* st = stage + (size_t)(s % kMbStages) * FR * 64;
    h8 bw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bw[t] = st[(2 * MB + 4 * tg + t) * 64 + lane];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const h8 a0 = st[(rg * RB + b) * 64 + lane], a1 = st[(MB + rg * RB + b) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[b][t] = mfma16(a0, bw[t], acc[b][t]);
        acc[b][t] = mfma16(a1, bw[t], acc[b][t]);
      }
    }
  }
  wait_vm<0>();  // the copies issued past the split's end land before the workgroup leaves
  const int j = lane >> 4, n = lane & 15;
  float* o = out + (size_t)sp * split_stride;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rb = rg * RB + b;
    if (rb >= mblocks) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tt = t0 + 4 * tg + t, col = tt * 16 + n;
      if (tt < mp.ntiles && col < N)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[(size_t)(rb * 16 + 4 * j + v) * N + col] = acc[b][t][v];
    }
  }
}

#define DFL_MB_KERNELS(MB)                                                                      \
  __global__ __launch_bounds__(64 * kMbWaves) void k_mb_i4_##MB(                                \
      const f16* __restrict__ xa, long ps, int K, const uint4* __restrict__ codes,              \
      const uint32_t* __restrict__ scales, TileMap mp, int N, int mblocks, int splits, int sps, \
      float* __restrict__ out, long split_stride) {                                             \
    mb_i4<MB>(xa, ps, K, codes, scales, mp, N, mblocks, splits, sps, out, split_stride);        \
  }                                                                                             \
  __global__ __launch_bounds__(64 * kMbWaves) void k_mb_f16_##MB(                               \
      const f16* __restrict__ xa, long ps, int K, const f16* __restrict__ w, TileMap mp, int N, \
      int mblocks, int splits, int sps, float* __restrict__ out, long split_stride) {           \
    mb_f16<MB>(xa, ps, K, w, mp, N, mblocks, splits, sps, out, split_stride);                   \
  }
DFL_MB_KERNELS(4)
DFL_MB_KERNELS(8)
#undef DFL_MB_KERNELS

// `mlp`'s activation for the batched gate/up product: the split-summed gate
// (columns 0..ffn) and up (ffn..2·ffn) of block row m of sequence s, then
// silu(gate)·up as A-layout planes of the down projection (block s).
__global__ __launch_bounds__(256) void k_glu_act(const float* __restrict__ part, int splits,
                                                 long ss, int ffn, f16* __restrict__ ma,
                                                 long mps) {
  const int i = blockIdx.x * 256 + threadIdx.x, m = blockIdx.y, sq = blockIdx.z;
  if (i >= ffn) return;
  const int r = 16 * sq + m;
  const float g = sum_splits(part + (size_t)r * 2 * ffn + i, splits, ss);
  const float u = sum_splits(part + (size_t)r * 2 * ffn + ffn + i, splits, ss);
  put_a(ma, mps, (size_t)sq * 16 * ffn + a_idx(m, i), g / (1.f + expf(-g)) * u);
}

static inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }

int mb_groups(int ntiles) { return (int)cdiv(ntiles, kMbNT); }


void gemm_mb_i4(hipStream_t st, const uint16_t* xa, long ps, int K, int MB, int mblocks,
                const uint8_t* codes, const uint16_t* scales, TileMap map, int N, int splits,
                int sps, float* out, long ss) {
  static const bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mb_i4_8),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mb_i4_lds(8));
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mb_i4_4),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mb_i4_lds(4));
    return true;
  }();
  (void)attr;
  const unsigned blocks = cdiv(map.ntiles, kMbNT) * splits;
  const f16* x = reinterpret_cast<const f16*>(xa);
  const uint4* c = reinterpret_cast<const uint4*>(codes);
  const uint32_t* s = reinterpret_cast<const uint32_t*>(scales);
  if (MB == 8)
    k_mb_i4_8<<<blocks, 64 * kMbWaves, mb_i4_lds(8), st>>>(x, ps, K, c, s, map, N, mblocks, splits,
                                                          sps, out, ss);
  else
    k_mb_i4_4<<<blocks, 64 * kMbWaves, mb_i4_lds(4), st>>>(x, ps, K, c, s, map, N, mblocks, splits,
                                                          sps, out, ss);
}

static constexpr size_t mb_f16_lds(int MB) { return sizeof(h8) * kMbStages * (2 * MB + kMbNT) * 64; }

void gemm_mb_f16(hipStream_t st, const uint16_t* xa, long ps, int K, int MB, int mblocks,
                 const uint16_t* w, TileMap map, int N, int splits, int sps, float* out,
                 long ss) {
  static const bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mb_f16_8),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mb_f16_lds(8));
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mb_f16_4),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mb_f16_lds(4));
    return true;
  }();
  (void)attr;
  const f16* x = reinterpret_cast<const f16*>(xa);
  const f16* wp = reinterpret_cast<const f16*>(w);
  const unsigned blocks = cdiv(map.ntiles, kMbNT) * splits;
  if (MB == 8)
    k_mb_f16_8<<<blocks, 64 * kMbWaves, mb_f16_lds(8), st>>>(x, ps, K, wp, map, N, mblocks, splits,
                                                            sps, out, ss);
  else
    k_mb_f16_4<<<blocks, 64 * kMbWaves, mb_f16_lds(4), st>>>(x, ps, K, wp, map, N, mblocks, splits,
                                                            sps, out, ss);
}

void glu_act(hipStream_t st, const float* part, int splits, long ss, int rows, int nseq, int ffn,
             uint16_t* ma, long mps) {
  k_glu_act<<<dim3(cdiv(ffn, 256), rows, nseq), 256, 0, st>>>(part, splits, ss, ffn,
                                                              reinterpret_cast<f16*>(ma), mps);
}

}  // namespace dfl
