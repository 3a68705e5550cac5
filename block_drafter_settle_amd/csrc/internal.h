// Shared declarations between the host orchestration (dflash.cpp) and the
// gfx950 kernels (kernels.hip). Layouts used by both sides:
//
// A-layout (activation operand of every GEMM, f16): an activation matrix of
// M rows and K columns (K % 32 == 0) is cut into 16-row blocks; inside a
// block, element (m, k) sits at half index
//     ((k/32)·64 + ((k/8)%4)·16 + m)·8 + k%8,
// so one 16x16x32 MFMA step s reads the contiguous 1 KB [s·64·8, (s+1)·64·8)
// and lane l gets row l%16, columns 32s + 8(l/16) .. +7. Rows past M are 0.
//
// Planes: an operand may carry a second A-layout array ("plane 1") at
// `ps` halves past the first, holding f16(v − f16(v)) of each value v.
// GEMMs then add both planes' products, which carries the f32 activation
// with about 22 significant bits instead of f16's 11. ps = 0 means a single
// plane. Writers of A-layout take the same ps.
//
// F16T (dense f16 weights [N][K]): 16-row tiles, each tile 32 columns at a
// time: tile t, step s, lane l holds W[16t + l%16][32s + 8(l/16) .. +7] at
// half index ((t·KS + s)·64 + l)·8, KS = K/32.
//
// I4T (int4 weights [N][K], K % 128 == 0): tile t, span p (128 columns),
// lane l owns 16 bytes at ((t·KT + p)·64 + l)·16, KT = K/128: four 32-bit
// words, word u holding row 16t + l%16, columns 128p + 32u + 8(l/16) + e for
// e = 0..7 as offset-binary nibbles (code + 8); e even at bit 2e, e odd at
// bit 16 + 2(e−1). Scales: 4 f16 per (tile, span, row) at
// ((t·KT + p)·16 + l%16)·4 + u, the scale of column group 4p + u.
//
// Tile maps: GEMM tile t (0 .. ntiles−1) reads stored tile
//     (t / seg)·seg_stride + seg_off + t % seg,
// which lets one launch walk the same rows of every layer (the settle's
// keys and values) or a row range of a fused matrix.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

struct TileMap {
  int ntiles;     // tiles in the product (output columns / 16, rounded up)
  int seg;        // tiles per segment
  long seg_stride;  // stored tiles between segments
  long seg_off;   // stored tile of the product's tile 0
};

// GEMM launches: out[split][mb·16 + m][col] partial sums (f32), col < N.
// gemm_i4: the int4 GEMM of 17–32 rows (and the debug product's): two row
// tiles a wave, a workgroup covers 8 tiles.
void gemm_i4(hipStream_t st, const uint16_t* xa, long ps, int K, int mblocks,
             const uint8_t* codes, const uint16_t* scales, TileMap map, int N, int splits,
             int spans_per_split, float* out, long split_stride);
// Many-row f16 GEMM (mblocks ≤ 16 row blocks at once, 16 weight tiles per
// block, async copies into a 3-stage LDS ring), two planes (plane 1 at
// xa + ps, ps a multiple of 8); out as gemm_i4.
void gemm_big_f16(hipStream_t st, const uint16_t* xa, long ps, int K, int mblocks,
                  const uint16_t* w, TileMap map, int N, int splits, int steps_per_split,
                  float* out, long split_stride);
// The block pass's 16-row int4 GEMM (two planes, ps ≠ 0; skinny.hip):
// splits of `ks` spans (128 columns) each, i4_block_splits(K, ks) of them;
// out as gemm_i4. R row tiles a wave, four waves a workgroup; (R, ks) is
// (2, 2) or (2, 8).
int i4_block_splits(int K, int ks);
void gemm_i4_block(hipStream_t st, const uint16_t* xa, long ps, int K, const uint8_t* codes,
                   const uint16_t* scales, TileMap map, int N, int R, int ks, float* out,
                   long split_stride);
// The block pass's 16-row f16 GEMM (two planes, ps ≠ 0): f16_block_splits(K)
// splits of 512 columns; out as gemm_i4.
int f16_block_splits(int K);
void gemm_f16_block(hipStream_t st, const uint16_t* xa, long ps, int K, const uint16_t* w,
                    TileMap map, int N, float* out, long split_stride);
// The settle's K/V at many rows straight from int4 codes (settle.hip): A the
// two-plane operand (plane 1 at xa + ps) of mblocks 16-row blocks (up to 16),
// K/V tiles through map, K splits of sps spans (128 columns) each; partial
// sums out[split][mblocks·16][N].
int kv_i4_groups(int ntiles);
void gemm_kv_i4(hipStream_t st, const uint16_t* xa, long ps, int K, int mblocks,
                const uint8_t* codes, const uint16_t* scales, TileMap map, int N, int splits,
                int sps, float* out, long ss);

// Peak probes (kernels.hip): a streaming read of `bytes` (multiple of 16) at
// p, and `workgroups` × 4 waves of `steps` rounds of 32 back-to-back MFMAs.
void probe_read(hipStream_t st, const void* p, long bytes, uint32_t* sink);
void probe_mfma(hipStream_t st, int workgroups, int steps, float* sink);

// gate/up with the SwiGLU epilogue at 16 rows, two planes in (xa, ps),
// streamed through one workgroup per tile-pair range (stream.hip), for
// K ≤ 5120 (40 spans of 128 over eight waves): gate tiles [0, ftiles), up
// tiles [ftiles, 2·ftiles) of one stored matrix; writes silu(g)·u in
// A-layout planes (ma, mps).
bool glu_stream_fits(int K);
void gemm_glu_stream(hipStream_t st, const uint16_t* xa, long ps, int K, const uint8_t* codes,
                     const uint16_t* scales, int ftiles, uint16_t* ma, long mps);
// Scratch of the selection: gmax [k][ceil(width/256)] column-group maxima,
// thr [k], counters [16], the candidate lists lv/li [k][topk_cap], and the
// score table tab [top·(1 + 15·top)].
struct SelectScratch {
  float* gmax;
  int* counters;
  float* lv;
  int* li;
  float* tab;
  int* best;  // per (row, predecessor) table row: the first candidate of the largest score
};

// Logits of rows 1..k over head tiles [0, ceil(width/16)) and the selector
// projection hp [16][rank] of all rows, in one launch; also the selection's
// column-group maxima.
void head_sel(hipStream_t st, const uint16_t* xa, long ps, int K, const uint16_t* head,
              int width, int k, float* logits, const uint16_t* sel, int rank, float* hp,
              SelectScratch sc);

// Rows 0..m of an operand taken from up to three runs of consecutive rows
// (ld floats apart): rows [0, n0) from p[0], [n0, n0 + n1) from p[1], the
// rest from p[2] (a settle's rows may wait in a ring and follow from the
// caller's buffer).
struct RowSrc {
  const float* p[3];
  int n0, n1;
  long ld;
};
void to_a(hipStream_t st, const RowSrc& x, int m, int K, uint16_t* xa, long ps);
void to_a(hipStream_t st, const float* x, long ld, int m, int K, uint16_t* xa, long ps);
// Row kernels: sqp holds partial sums of squares of each row, row_chunks(N)
// per row from rowsum_sq and embed (256 channels each), conv1_chunks(hs)
// per row from conv1; norm_apply takes the producer's count.
int row_chunks(int N);
int conv1_chunks(int hs);
// rowsum_sq: the split-summed settle rows t, their sums of squares, and
// t ⊙ w as the K/V projection's two-plane operand (plane 1 at xa + ps);
// settle_kv applies the hidden norm's per-row scale (from sqp,
// row_chunks(hs) per row).
void rowsum_sq(hipStream_t st, const float* part, int splits, long split_stride, int rows, int N,
               const float* w, uint16_t* xa, long ps, float* sqp);
// The block kernels below take `nseq` sequences' blocks at once (batched
// blocks): sequence s owns rows 16s..16s+15 of every row-major buffer
// (its `rows` block rows first), A-layout block s of every operand, and
// qa + s·nh·16·hd of the attention's queries.
constexpr int kMaxSeq = 8;
struct SeqTok {
  int t[kMaxSeq];
};
struct SeqPos {
  long a[kMaxSeq];
};
void norm_apply(hipStream_t st, const float* h, const float* sqp, int nchunk, int rows, int N,
                const float* w, float eps, float* x, uint16_t* xa, long ps, int nseq = 1);
// embed and conv1 also write u = h ⊙ w (w: the next norm's gain; conv1
// skips it for w == nullptr) as A-layout planes, the next kernel
// projection's input; conv0 applies that norm's per-row scale from sqp.
// anchors: host [nseq].
void embed(hipStream_t st, const uint16_t* emb, const int* anchors, int nseq, int mask, int rows,
           int hs, float* h, float* sqp, const float* w, uint16_t* xa, long ps);
void conv0(hipStream_t st, const float* h, const float* sqp, int nchunk, const float* w, float eps,
           const float* dpart, int splits, long split_stride, const float* base, int rows, int hs,
           int gs, int kn, uint16_t* xca, long ps, float* dsum, int nseq = 1);
void conv1(hipStream_t st, float* h, const float* opart, int splits, long split_stride,
           const float* dsum, const float* base, int rows, int hs, int gs, int kn, float* sqp,
           const float* w, uint16_t* xa, long ps, int nseq = 1);
// pos: host [nseq], each sequence's block position a
void qkv_post(hipStream_t st, const float* part, int splits, long split_stride, int rows, int nh,
              int kv, int hd, const float* q_norm, const float* k_norm, const float* inv_freq,
              const long* pos, int nseq, int rot, float eps, uint16_t* qa, long qps, uint16_t* kb,
              uint16_t* vb);
// Keys and values are kept as f16 pairs, kv head major: the head_dim f32
// values x of one kv head of one row are 2·head_dim halves, hi = f16(x) for
// all head_dim, then lo = f16(x − hi) (the bytes of the f32 values), and a
// buffer of R rows holds kv head g's rows at [g][R][2·head_dim]. A layer's
// context store is such a ring of R = cap rows for the keys and one for the
// values; position p sits at row (p − first) mod cap. The block's own rows
// (kb, vb) are R = 16 rows a sequence.
struct StoreSlot {
  uint16_t* k;
  uint16_t* v;
  long cap;
};
// Conversion between f32 rows and a ring's rows (debug reads and loads of
// the store): rows r0 .. r0+n−1 of the ring (each at row index mod cap) from
// (out = false) or to (out = true) lin, dev f32 [n][kv·hd].
void store_rows(hipStream_t st, uint16_t* ring, long cap, long r0, float* lin, long n, int kv,
                int hd, bool out);
// row0 = pos0 − first; row_end: one past the settle call's last row (rows
// below row_end − cap of a layer are not written to it); tab: the layers'
// stores (device memory).
void settle_kv(hipStream_t st, const float* part, int splits, long split_stride, int rows,
               int layers, int kv, int hd, const float* k_norm, const float* inv_freq,
               const int* rot, long pos0, float eps, const float* sqp, int hs,
               const StoreSlot* tab, long row0, long row_end);
// Context chunks per kv head of one attention call; the merge holds one
// weight per chunk (and one for the block's own rows) in LDS.
constexpr int kAttnMaxChunks = 64;
// One sequence's attention over a layer: sk, sv its ring of cap rows,
// whose n keys of positions lo.. start at ring row s0 and wrap at most
// once; a its block position; the keys in nchunks chunks of `chunk`.
struct AttnSeq {
  const uint16_t* sk;
  const uint16_t* sv;
  long cap, s0, lo, a;
  int n, chunk, nchunks;
};
struct AttnSeqs {
  AttnSeq s[kMaxSeq];
};
struct SeqChunks {
  int n[kMaxSeq];
};
// pacc, pml: nseq·nh·(kAttnMaxChunks + 1)·16 chunk states (hd floats, and a
// float pair, each)
void attention(hipStream_t st, const uint16_t* qa, long qps, const AttnSeqs& seqs, int nseq,
               const uint16_t* kb, const uint16_t* vb, int B, int nh, int kv, int hd, int window,
               float scale, float* pacc, float* pml);
void attn_merge(hipStream_t st, const float* pacc, const float* pml, int nh, int kv, int hd,
                const AttnSeqs& seqs, int nseq, int B, uint16_t* ya, long ps);
// Selection (`top_k` + `select_with`) on logits [k][width] and hp rows
// [k][rank]: cand/unary, the score table and the chain (score, chosen).
// have_gmax: the head kernel already wrote the column-group maxima.
int topk_slices(int width);
int topk_cap(int width, int top);
void select_all(hipStream_t st, const float* logits, bool have_gmax, int k, int width, int top,
                const float* hp, int rank, const uint16_t* pbook, const uint16_t* cbook,
                int vocab, int anchor, const int* forced, SelectScratch sc, int* cand,
                float* unary, float* score, int* chosen);
// nseq sequences' selections at once (batched blocks): sequence s's logits
// rows at logits + s·lseq, its projections at hp + s·hseq, its anchor
// anchors[s] (host), scratch set s of sc (sized for nseq sets: 16·ceil(
// width/256) maxima, 16 counters, 16·topk_cap lists, top·(1 + 15·top)
// table entries and 1 + 15·top best indices a set), outputs at s·k·top
// (cand, unary, score) and s·k (chosen). No forced chain when nseq > 1.
void select_batch(hipStream_t st, int nseq, const float* logits, long lseq, bool have_gmax, int k,
                  int width, int top, const float* hp, long hseq, int rank,
                  const uint16_t* pbook, const uint16_t* cbook, int vocab, const int* anchors,
                  const int* forced, SelectScratch sc, int* cand, float* unary, float* score,
                  int* chosen);
// Batched blocks (batch.hip): products of MB·16 rows (MB = 4 or 8 A-layout
// row blocks, the first `mblocks` written out) in splits of sps spans
// (int4) or steps (f16), 16 weight tiles a workgroup; out as gemm_i4.
int mb_groups(int ntiles);
void gemm_mb_i4(hipStream_t st, const uint16_t* xa, long ps, int K, int MB, int mblocks,
                const uint8_t* codes, const uint16_t* scales, TileMap map, int N, int splits,
                int sps, float* out, long split_stride);
void gemm_mb_f16(hipStream_t st, const uint16_t* xa, long ps, int K, int MB, int mblocks,
                 const uint16_t* w, TileMap map, int N, int splits, int sps, float* out,
                 long split_stride);
// silu(gate)·up of the split-summed batched gate/up product [rows of nseq
// sequences][2·ffn] into the down projection's A-layout planes
void glu_act(hipStream_t st, const float* part, int splits, long split_stride, int rows, int nseq,
             int ffn, uint16_t* ma, long mps);
void dequant_i4(hipStream_t st, const uint8_t* codes, const uint16_t* scales, TileMap map,
                int rows, int K, float* out);
void sum_rows(hipStream_t st, const float* part, int splits, long split_stride, int rows, int N,
              float* out);

// Router margin (route.hip): rows dev f32 [m][hidden], each subspace's mean
// f16 [hidden] and basis f16 [rank][hidden]; scratch coef
// [kRouteMaxRows][2][kRouteMaxRank], nrm [kRouteMaxRows][2], part
// [kRouteMaxRows][2][route_chunks(hidden)]; margin dev f32 [m].
constexpr int kRouteMaxRows = 64, kRouteMaxRank = 256, kRouteMaxHidden = 5120;
int route_chunks(int hidden);
void route_margin(hipStream_t st, const float* rows, int m, int hidden, const uint16_t* bmean,
                  const uint16_t* bbasis, int brank, const uint16_t* cmean,
                  const uint16_t* cbasis, int crank, float* coef, float* nrm, float* part,
                  float* margin);

}  // namespace dfl
