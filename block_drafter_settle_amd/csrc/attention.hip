// Attention of the block pass over the context store and the block's own
// rows (`Drafter::block` on the docs.rs page "cortiq_engine/dflash.rs",
// cortiq-engine 0.8.78): split-context partial softmax states and their
// merge. Compiled on its own with MFMA results in VGPRs: the running
// accumulators are rescaled in VALU every step.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <climits>

namespace dfl {

// Split-context attention (`Drafter::block`'s inner loop). Block (g, c, z)
// (kv heads fastest: the workgroups that run together read all kv heads of
// the same context rows, whole rows of the store):
// kv head g, its q heads 4z..4z+3, and key chunk c — context keys
// [c·chunk, min(n, (c+1)·chunk)) of the layer's range, or for c == nchunks
// the block's own B keys. The context keys sit in the layer's ring of cap
// rows from row s0 on, wrapping at most once. Each wave keeps one q head's 16 query rows and an
// online softmax over 32-key steps: S^T = K·Q^T and O^T += V^T·P^T on MFMA.
// Every operand is an f16 pair (hi, lo = f16 of the rest): q's two A-layout
// planes (plane 1 at qa + qps), K and V as the store keeps them (per kv
// head, rows of hi [hd] then lo [hd]) staged into two LDS planes each, P
// split in registers; each product takes hi·hi + hi·lo + lo·hi, the dropped lo·lo
// term lying below f32 rounding. The softmax runs in base 2 (scores times
// log2 e, exp2 as one v_exp_f32). Writes the chunk's (max, sum, O) for the
// merge, the max in base-2 units.
// Batched blocks: blockIdx.z = nzq·s + z for sequence s, whose call is
// seqs.s[s] (its own store, range and chunking); its queries at
// qa + s·nh·16·hd, its block rows' keys and values at kb, vb + s·16·2kd halves,
// its chunk states at pacc, pml + s·nh·(kAttnMaxChunks + 1)·16·(hd, 1).
// A chunk index past the sequence's own chunks leaves at once.
template <int HD>
__global__ __launch_bounds__(kThreads) void k_attn(const f16* __restrict__ qa, long qps,
                                                   AttnSeqs seqs, int nzq,
                                                   const f16* __restrict__ kb,
                                                   const f16* __restrict__ vb, int B, int nh,
                                                   int kv, int window, float scale,
                                                   float* __restrict__ pacc,
                                                   float2* __restrict__ pml) {
  constexpr int KST = HD + 8;   // LDS row stride of K (halfs)
  constexpr int VST = 32 + 4;   // LDS row stride of V^T (halfs): 18 dwords, so 16 rows' 64-bit
                                // reads fall on distinct banks
  __shared__ f16 Ks[2][2][32 * KST];  // [buffer][plane]
  __shared__ f16 Vt[2][2][HD * VST];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the block's own keys first (y = 0, a short workgroup that then does not
  // trail the context chunks), then context chunk y − 1
  const int g = blockIdx.x, c = blockIdx.y == 0 ? seqs.s[blockIdx.z / nzq].nchunks : blockIdx.y - 1;
  const int sq = blockIdx.z / nzq;
  const AttnSeq& cs = seqs.s[sq];
  const int n = cs.n, chunk = cs.chunk, nchunks = cs.nchunks;
  if (blockIdx.y > 0 && c >= nchunks) return;  // whole workgroup
  const f16* __restrict__ sk = reinterpret_cast<const f16*>(cs.sk);
  const f16* __restrict__ sv = reinterpret_cast<const f16*>(cs.sv);
  const long cap = cs.cap, s0 = cs.s0, lo_pos = cs.lo, a = cs.a;
  const int rep = nh / kv;
  const int qi = (blockIdx.z % nzq) * 4 + wave;
  const bool active = qi < rep;
  const int hq = g * rep + min(qi, rep - 1);
  const int kd = kv * HD;
  qa += (size_t)sq * nh * 16 * HD;
  kb += (size_t)sq * 16 * 2 * kd;
  vb += (size_t)sq * 16 * 2 * kd;
  pacc += (size_t)sq * nh * (kAttnMaxChunks + 1) * 16 * HD;
  pml += (size_t)sq * nh * (kAttnMaxChunks + 1) * 16;
  const bool blk = c == nchunks;
  const int k_first = blk ? 0 : c * chunk;
  const int count = blk ? B : min(chunk, n - k_first);
  // kv head g's rows: its ring of cap rows in the store, or the block's 16
  const f16* kbase = blk ? kb + (size_t)g * 16 * 2 * HD : sk + (size_t)g * cap * 2 * HD;
  const f16* vbase = blk ? vb + (size_t)g * 16 * 2 * HD : sv + (size_t)g * cap * 2 * HD;
  // ring row of the chunk's first key (s0 < cap and k_first < n ≤ cap)
  const long wrap = blk ? LONG_MAX : cap;
  long row_first = blk ? 0 : s0 + k_first;
  if (row_first >= wrap) row_first -= wrap;
  const long pos_base = lo_pos + k_first;

  h8 qf[HD / 32], ql[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s) {
    const size_t off = (size_t)hq * 16 * HD + ((size_t)s * 64 + lane) * 8;
    qf[s] = *reinterpret_cast<const h8*>(qa + off);
    ql[s] = *reinterpret_cast<const h8*>(qa + qps + off);
  }

  const int r = lane & 15, j = lane >> 4;
  // row r sees chunk key idx iff idx ≥ lim (the window's first position,
  // relative to this chunk's first key, clamped into int range)
  const long lim_abs = window > 0 ? a + r + 1 - window - pos_base : LONG_MIN;
  const int lim = (blk || window == 0) ? INT_MIN
                  : (int)std::max<long>(INT_MIN, std::min<long>(INT_MAX, lim_abs));
  // softmax in base 2: scores carry log2(e), exp2 is one v_exp_f32
  const float scale2 = scale * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.f;
  f4 acc[HD / 16];
#pragma unroll
  for (int d = 0; d < HD / 16; ++d) acc[d] = (f4){0.f, 0.f, 0.f, 0.f};

  // Staging: a kv head's row is 2·HD halves (hi, then lo), NPL 16-byte
  // pieces a plane. Thread t stages piece jp of key pairs q, q + QP, ..:
  // q = lane mod QP, jp = lane / QP + (64 / QP)·wave, so a load instruction
  // covers whole 128-byte runs of QP rows, and for a V^T dims row the lanes
  // with one jp write consecutive key pairs. NSET register sets (set entry
  // 2·pass + key of the pair) hold the next NSET 32-key steps while one is
  // computed.
  constexpr int QP = 1024 / HD;   // key pairs a pass: 16 pairs (32 keys) in HD / 64 passes
  constexpr int NPASS = HD / 64;
  constexpr int NPL = HD / 8;
  const int q = lane % QP, jp = lane / QP + (64 / QP) * wave;
  const int spl = jp / NPL, dd = (jp % NPL) * 8;
  // Keys past the chunk's end read the chunk's last row instead (their
  // scores are masked, so they weigh 0 against finite values): no load sits
  // in a branch, and the loads of the steps ahead stay in flight across the
  // LDS-only barriers below. Each K/V byte is read once a layer: the loads
  // carry the non-temporal bit (at 131072 positions, with the staggered
  // chunks, the kernel went from 5.5 to 6.2 TB/s).
  auto fetch = [&](int k0, h8 (&kreg)[2 * NPASS], h8 (&vreg)[2 * NPASS]) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = min(k0 + 2 * (q + QP * ps) + h, count - 1);
        long row = row_first + key;
        if (row >= wrap) row -= wrap;
        const size_t off = (size_t)row * 2 * HD + spl * HD + dd;
        kreg[2 * ps + h] = __builtin_nontemporal_load(reinterpret_cast<const h8*>(kbase + off));
        vreg[2 * ps + h] = __builtin_nontemporal_load(reinterpret_cast<const h8*>(vbase + off));
      }
  };
  auto stage = [&](const h8 (&kreg)[2 * NPASS], const h8 (&vreg)[2 * NPASS], int b) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int kk = 2 * (q + QP * ps);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<h8*>(&Ks[b][spl][(kk + h) * KST + dd]) = kreg[2 * ps + h];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<h2*>(&Vt[b][spl][(dd + e) * VST + kk]) =
            (h2){vreg[2 * ps][e], vreg[2 * ps + 1][e]};
    }
    lds_barrier();
  };
  auto compute = [&](int k0, int b) {
    // scores: st[h][v] = S^T[key 16h + 4j + v][query r]
    f4 st[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      st[hb] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        const int off = (16 * hb + (lane & 15)) * KST + 32 * s + 8 * j;
        const h8 ka = *reinterpret_cast<const h8*>(&Ks[b][0][off]);
        const h8 kl = *reinterpret_cast<const h8*>(&Ks[b][1][off]);
        st[hb] = mfma16(ka, qf[s], st[hb]);
        st[hb] = mfma16(ka, ql[s], st[hb]);
        st[hb] = mfma16(kl, qf[s], st[hb]);
      }
    }
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 16 * (e >> 2) + 4 * j + (e & 3);
      const int idx = k0 + key;
      const bool ok = idx < count && idx >= lim;
      p[e] = ok ? st[e >> 2][e & 3] * scale2 : -INFINITY;
      mx = fmaxf(mx, p[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float corr = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = p[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(p[e] - m_new);
      ps += p[e];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * corr + ps;
    m_run = m_new;
    h8 pb, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f16 h, l;
      split_f16(p[e], h, l);
      pb[e] = h;
      pl[e] = l;
    }
#pragma unroll
    for (int d = 0; d < HD / 16; ++d) {
      const int off = (16 * d + (lane & 15)) * VST + 4 * j;
      const h4 v0 = *reinterpret_cast<const h4*>(&Vt[b][0][off]);
      const h4 v1 = *reinterpret_cast<const h4*>(&Vt[b][0][off + 16]);
      const h4 w0 = *reinterpret_cast<const h4*>(&Vt[b][1][off]);
      const h4 w1 = *reinterpret_cast<const h4*>(&Vt[b][1][off + 16]);
      const h8 va = (h8){v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const h8 vl = (h8){w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      f4 t = mfma16(va, pb, acc[d] * corr);
      t = mfma16(va, pl, t);
      acc[d] = mfma16(vl, pb, t);
    }
  };
  // NSET register sets of 32-key steps: each step is fetched NSET steps
  // ahead, so that NSET steps of K/V rows are in flight while one is
  // computed. Steps past the chunk's end are fetched (the clamped last row)
  // and staged but not computed. (Three sets were measured no faster.)
  // Step s is staged into LDS buffer s mod 2 and published by one barrier;
  // that buffer's last readers, step s − 2's computes, all finished before
  // the barrier that published step s − 1.
  constexpr int NSET = 2;
  static_assert(NSET == 2, "a step's LDS buffer is its set index");
  h8 kr[NSET][2 * NPASS], vr[NSET][2 * NPASS];
  if (count > 0) {
#pragma unroll
    for (int i = 0; i < NSET; ++i) fetch(32 * i, kr[i], vr[i]);
    for (int k0 = 0; k0 < count; k0 += 32 * NSET) {
#pragma unroll
      for (int i = 0; i < NSET; ++i) {
        stage(kr[i], vr[i], i);  // step k0/32 + i, its parity i (k0 a multiple of 64)
        fetch(k0 + 32 * (i + NSET), kr[i], vr[i]);
        if (k0 + 32 * i < count) compute(k0 + 32 * i, i);
      }
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

// Softmax-merge of the chunks of one (q head, row) → y in A-layout f16:
// y = Σ_c acc_c·2^{m_c − M} / Σ_c l_c·2^{m_c − M}, M the largest chunk max
// (the chunk states are kept in base 2).
// Thread t forms chunk t's weight, then 256 / hd groups of hd threads each
// sum a strided share of the chunks.
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ pacc,
                                                    const float2* __restrict__ pml, int nh,
                                                    int kv, int hd, SeqChunks sc,
                                                    f16* __restrict__ ya, long ps) {
  __shared__ float fw[kAttnMaxChunks + 1], red[4], redl[4];
  const int hq = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  // sequence sq (blockIdx.z): its chunk states and its A-layout block of y
  const int sq = blockIdx.z, nchunks = sc.n[sq];
  pacc += (size_t)sq * nh * (kAttnMaxChunks + 1) * 16 * hd;
  pml += (size_t)sq * nh * (kAttnMaxChunks + 1) * 16;
  ya += (size_t)sq * 16 * nh * hd;
  const int lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
  const int rep = nh / kv, g = hq / rep, qi = hq % rep, nc = nchunks + 1;
  const size_t slot0 = (size_t)g * nc * rep + qi;  // chunk c is slot slot0 + c·rep
  // one chunk a thread (nc ≤ kAttnMaxChunks + 1 ≤ 256): its (m, l) is loaded
  // once, together with the first eight partial outputs this thread sums
  // below, so those loads overlap the two reductions
  static_assert(kAttnMaxChunks + 1 <= 256, "one chunk a thread");
  const float2 mlt = t < nc ? pml[(slot0 + (size_t)t * rep) * 16 + r] : make_float2(-INFINITY, 0.f);
  const int G = blockDim.x / hd, grp = t / hd, d = t - grp * hd;
  const float* pc = pacc + (slot0 * 16 + r) * hd + d;
  const size_t cs = (size_t)rep * 16 * hd;  // chunk stride
  float pre[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) pre[k] = grp + k * G < nc ? pc[(size_t)(grp + k * G) * cs] : 0.f;
  float m = mlt.x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < nw; ++w) M = fmaxf(M, red[w]);
  float l = 0.f;
  if (t < nc) {
    const float f = mlt.x != -INFINITY ? exp2f(mlt.x - M) : 0.f;
    fw[t] = f;
    l = mlt.y * f;
  }
  l = wave_sum(l);
  if (lane == 0) redl[wave] = l;
  __syncthreads();
  float L = 0.f;
  for (int w = 0; w < nw; ++w) L += redl[w];
  // thread (grp, d): dimension d of chunks grp, grp + G, … (G = blockDim / hd
  // groups), eight loads in flight; the groups' sums meet in LDS in order
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int c = grp;
  if (c + 7 * G < nc) {
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] += pre[k] * fw[c + k * G];
    c += 8 * G;
    for (; c + 7 * G < nc; c += 8 * G)
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] += pc[(size_t)(c + k * G) * cs] * fw[c + k * G];
    for (int k = 0; c < nc; c += G, ++k) y[k & 7] += pc[(size_t)c * cs] * fw[c];
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (c + k * G < nc) y[k] += pre[k] * fw[c + k * G];
  }
  const float ys = ((y[0] + y[1]) + (y[2] + y[3])) + ((y[4] + y[5]) + (y[6] + y[7]));
  __shared__ float part[256];
  part[t] = ys;
  __syncthreads();
  if (grp) return;
  float yt = part[d];
  for (int q = 1; q < G; ++q) yt += part[q * hd + d];
  put_a(ya, ps, a_idx(r, hq * hd + d), yt / L);
}

static inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }

void attention(hipStream_t st, const uint16_t* qa, long qps, const AttnSeqs& seqs, int nseq,
               const uint16_t* kb, const uint16_t* vb, int B, int nh, int kv, int hd, int window,
               float scale, float* pacc, float* pml) {
  const int rep = nh / kv, nzq = cdiv(rep, 4);
  int maxc = 0;
  for (int i = 0; i < nseq; ++i) maxc = std::max(maxc, seqs.s[i].nchunks);
  dim3 grid(kv, maxc + 1, nzq * nseq);
  const f16* q = reinterpret_cast<const f16*>(qa);
  const f16* k16 = reinterpret_cast<const f16*>(kb);
  const f16* v16 = reinterpret_cast<const f16*>(vb);
  float2* ml = reinterpret_cast<float2*>(pml);
  if (hd == 64)
    k_attn<64><<<grid, kThreads, 0, st>>>(q, qps, seqs, nzq, k16, v16, B, nh, kv, window, scale,
                                           pacc, ml);
  else if (hd == 128)
    k_attn<128><<<grid, kThreads, 0, st>>>(q, qps, seqs, nzq, k16, v16, B, nh, kv, window, scale,
                                            pacc, ml);
  else
    k_attn<256><<<grid, kThreads, 0, st>>>(q, qps, seqs, nzq, k16, v16, B, nh, kv, window, scale,
                                            pacc, ml);
}

void attn_merge(hipStream_t st, const float* pacc, const float* pml, int nh, int kv, int hd,
                const AttnSeqs& seqs, int nseq, int B, uint16_t* ya, long ps) {
  dim3 grid(nh, B, nseq);
  SeqChunks sc{};
  for (int i = 0; i < nseq; ++i) sc.n[i] = seqs.s[i].nchunks;
  k_attn_merge<<<grid, 256, 0, st>>>(pacc, reinterpret_cast<const float2*>(pml), nh, kv, hd, sc,
                                     reinterpret_cast<f16*>(ya), ps);
}

}  // namespace dfl
