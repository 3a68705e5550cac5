/*
 * dflash.h — the DFlash 2 drafter's forward pass on one AMD MI355X (gfx950).
 *
 * The drafter and its two passes are defined on the docs.rs page
 * "cortiq_engine/dflash.rs" (cortiq-engine 0.8.78): the module overview (the
 * context, block and token formulas), `Geometry`, `settle_rows`,
 * `Drafter::block`, `block_dev` (the per-layer context ranges and the head
 * width), `select_with` and `top_k`. The device interface it replaces is the
 * CUDA block on the page "src/gpu_cuda/hyb/dflash.rs" (cortiq-engine
 * 0.8.72): `Dev::new` (the sidecar onto the card), `Dev::settle` and
 * `Dev::block`.
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative code: DFLASH_EINVAL (-1) for an
 *     invalid argument or geometry, DFLASH_ENOMEM (-2) for device memory or
 *     a layer's store capacity (max_context) exhausted, DFLASH_EHIP (-3) for
 *     a HIP runtime error. The message is kept for dflash_last_error.
 *     Arguments and capacity are checked before any launch, and a call they
 *     reject changes no state. After DFLASH_EHIP from a call that settles
 *     or moves context rows (a launch failed: the device is usually unusable
 *     then) the context is empty: span [first, first).
 *   - "dev" pointers are device memory the caller owns (e.g. torch tensors'
 *     data_ptr on the same GPU); "host" pointers are host memory.
 *   - Work is enqueued on the stream given at create and is asynchronous:
 *     outputs are valid once that stream has been synchronised
 *     (dflash_sync, or the caller's own stream sync). Calls on one handle
 *     must not overlap from several host threads.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_OK 0
#define DFLASH_EINVAL (-1)
#define DFLASH_ENOMEM (-2)
#define DFLASH_EHIP (-3)

typedef struct dflash dflash_t; /* opaque; owns every device buffer it uses */

/* A matrix of symmetric int4 weights with one f16 scale per 32 consecutive
   columns of a row: element (r, c) = q(r, c) · scale[r][c/32].
   q: [rows][cols/2] bytes, column 2j in the low nibble of byte j and column
   2j+1 in the high nibble, two's complement (−8..7).
   scale: [rows][cols/32] IEEE binary16 bit patterns. */
typedef struct {
  const uint8_t* q;
  const uint16_t* scale;
} dflash_i4;

/* One draft layer (host pointers; the names are the sidecar's tensors of
   `Drafter::new`). f16 arrays hold IEEE binary16 bit patterns. */
typedef struct {
  const float *in_norm, *post_norm; /* [hidden] input / post-attention RMSNorm gains */
  const float *q_norm, *k_norm;     /* [head_dim] per-head query / key norm gains */
  const float *attn_base, *mlp_base; /* [2][conv_kernel][hidden] conv base kernels,
                                        stage 0 (before the sub-layer) then stage 1 */
  const uint16_t *attn_kproj, *mlp_kproj; /* f16 [2*conv_kernel*(hidden/conv_group)][hidden]
                                             kernel projections; output row
                                             (stage*kn + o)*groups + g */
  dflash_i4 q, k, v; /* [heads*head_dim | kv_heads*head_dim | kv_heads*head_dim][hidden] */
  dflash_i4 o;       /* [hidden][heads*head_dim] */
  dflash_i4 gate, up; /* [intermediate][hidden] */
  dflash_i4 down;    /* [hidden][intermediate] */
} dflash_layer_w;

/* `Geometry` of the page, plus the store's capacity. Accepted when: layers
   > 0, block in [2, 16], n_taps > 0, kv_heads > 0, heads % kv_heads == 0,
   head_dim in {64, 128, 256}, conv_group > 0, hidden % conv_group == 0,
   conv_kernel in [1, block], hidden, intermediate and heads*head_dim
   multiples of 128, hidden ≤ 5120, 1 ≤ selector_top ≤ 32, selector_top ≤ vocab,
   vocab ≤ 262144, selector_rank in [1, 256], 0 ≤ mask_token < vocab, every window ≥ 0,
   max_context ≥ 1. */
typedef struct {
  int32_t hidden, intermediate, layers, heads, kv_heads, head_dim, vocab, block, mask_token,
      conv_group, conv_kernel, selector_rank, selector_top, n_taps;
  const int32_t* windows; /* host [layers]: positions a block row sees back, 0 = all */
  const uint8_t* rotary;  /* host [layers]: 1 = rotary queries and keys, 0 = `no_rope` */
  double rope_theta, eps;
  int64_t max_context; /* most context rows one layer holds: a layer without a window
                          holds every settled row, so the settled span is at most this
                          long; a windowed layer holds at most min(2·window, max_context) */
} dflash_geometry;

typedef struct {
  const uint16_t* fc;         /* f16 [hidden][n_taps*hidden] */
  const float* hidden_norm;   /* [hidden] */
  const float* norm;          /* [hidden] the final norm */
  const uint16_t* sel_proj;   /* f16 [selector_rank][hidden] selector hidden projection */
  const uint16_t* pred_book;  /* f16 [vocab][selector_rank] predecessor codebook P */
  const uint16_t* succ_book;  /* f16 [vocab][selector_rank] successor codebook C */
  const uint16_t* embed;      /* f16 [vocab][hidden] the target's embedding */
  const uint16_t* head;       /* f16 [vocab][hidden] the target's head (may equal embed) */
  const dflash_layer_w* layer; /* [layers] */
} dflash_weights;

/* Build a drafter: validate the geometry, copy every weight to device memory
   (int4 and f16 matrices repacked into the kernels' tile layouts), allocate
   each windowed layer's context ring (min(2·window, max_context) rows of
   [kv_heads][head_dim] f32 keys and values, each held as its f16 pair: the
   rows a layer holds never exceed that, see dflash_settle), the ring of waiting tap rows (see dflash_queue)
   and all scratch. A layer without a window gets its store as rows come
   (dflash_reserve). Synchronous: the caller may free every host array
   once it returns. `stream` is a hipStream_t (NULL = the null stream) that
   every later call enqueues on. On failure *out is NULL and
   dflash_last_error(NULL) has the message. */
int dflash_create(const dflash_geometry* g, const dflash_weights* w, void* stream,
                  dflash_t** out);

/* Context settle (`push_context`: `queue_context` then `settle`; the rows
   themselves as `settle_rows` and `Dev::settle` make them): n joined tap
   rows (dev f32 [n][n_taps*hidden], row r = position first_pos + r, taps in
   the order of the geometry's taps) become context, after any rows that
   wait (dflash_queue): t = rms(fc·row, hidden_norm); per layer K =
   rot(rms(Wk·t per kv head, k_norm), position) (no rotation on a no-rope
   layer), V = Wv·t, stored as f32 values (each held as its f16 pair
   hi = f16(x), lo = f16(x − hi), the form the attention multiplies).
   Position rule (`queue_context`): with first ≤ first_pos ≤ the span's end
   (waiting rows included) the context is cut at first_pos and the rows
   appended; otherwise (a gap, or first_pos < first) it restarts at
   first_pos. n = 0 only applies the rule (and settles what waits).
   The rows are settled by `settle_rows` calls, 256 rows a pass: when more
   than the waiting limit (see dflash_queue) would wait, first the oldest
   rows past it (a multiple of 64), then the rest. After each call a layer
   with window w > 0 that holds more than 2w rows keeps only the last w
   (`Ctx::dropped`): a block sees no further back than its window, so a
   block at the end of the context is unchanged by the drop. Fails with
   DFLASH_ENOMEM (nothing changed) if a layer would hold more rows than
   max_context or its store cannot grow. */
int dflash_settle(dflash_t* d, int64_t first_pos, int32_t n, const float* taps);

/* Queue rows without settling them (`queue_context`): the position rule of
   dflash_settle, then the rows wait in the library's ring (copied from the
   caller's buffer, which may be reused once the stream passes this call).
   At most 512 rows wait (`PENDING_ROWS`; when every layer is windowed,
   max(512, widest window + 256): `BLOCK_SLACK`); past that the oldest
   settle at once, as many as bring the waiting rows to the limit, rounded
   up to a multiple of 64 (`CONTEXT_CHUNK`). dflash_block fails while rows
   wait. Errors as dflash_settle; also fails with DFLASH_ENOMEM if the rows
   that would then wait could not be settled later. */
int dflash_queue(dflash_t* d, int64_t first_pos, int32_t n, const float* taps);

/* Settle every waiting row (`settle`), one `settle_rows` call. */
int dflash_flush(dflash_t* d);

/* Room for `rows` context rows in every layer without a window
   (`Dev::reserve`): a store that is too small grows to max(rows, 2·its
   rows, 4096), at most max_context, keeping what it holds (the stream is
   synchronised when a store moves). The settle calls reserve by themselves;
   a caller that knows its context length may reserve up front so that no
   later call moves a store. DFLASH_ENOMEM if rows > max_context or the
   memory cannot be had (nothing changed). */
int dflash_reserve(dflash_t* d, int64_t rows);

/* Block pass (`Drafter::block` + the head + `select_with`): rows
   [embed[anchor_token], embed[mask_token] × (block−1)] at positions a, a+1, …
   through every layer, attending to the settled context positions the
   layer's range allows (per-layer range of `block_dev`; row r also hides
   positions below a+r+1−window) and to all block rows. Rows 1..k after the
   final norm give
     logits  dev f32 [k][width], head rows 0..width−1 (NULL: not written),
   and, after the selector (top `selector_top` candidates of each row by
   logit, larger first and the smaller index first among equals, re-scored
   as logit + Σ_r (P[prev]·hp)[r]·C[cand][r], prev = anchor for row 0 and
   the chosen token of the row before otherwise):
     cand    dev int32 [k][selector_top] candidate tokens, in top-k order
     unary   dev f32   [k][selector_top] their logits
     score   dev f32   [k][selector_top] their selector scores
     chosen  dev int32 [k] the first candidate with the largest score.
   Requires 1 ≤ k < block, selector_top ≤ width ≤ vocab,
   0 ≤ anchor_token < vocab, a ≥ 0, and no waiting rows. A layer's context
   range starts at its first held position, first + dropped (`block_dev`). */
int dflash_block(dflash_t* d, int32_t anchor_token, int64_t a, int32_t k, int32_t width,
                 float* logits, int32_t* cand, float* unary, float* score, int32_t* chosen);

/* For callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid allocation): the block
   pass of dflash_block, same arguments and results, except that `logits`
   must be a caller buffer (dev f32 [k][width], not NULL). Its per-call
   scratch (activations, partial sums, attention states, candidate lists)
   comes from one static array of the library on each GPU, 48 MiB
   (`DFLASH_NOALLOC_SCRATCH_BYTES`), held until the process ends; the call
   itself allocates nothing. A geometry whose scratch exceeds it fails with
   DFLASH_EINVAL (the 27B-shaped sidecar takes about 26 MB). Every call on a
   GPU shares that GPU's array and leaves its contents behind: calls that
   overlap on one GPU (from any handle, on any stream) race, so they must be
   ordered. The dflash_debug_* reads of the last block reflect the last
   dflash_block, not this call. */
#define DFLASH_NOALLOC_SCRATCH_BYTES (48u << 20)
int dflash_block_noalloc(dflash_t* d, int32_t anchor_token, int64_t a, int32_t k, int32_t width,
                         float* logits, int32_t* cand, float* unary, float* score,
                         int32_t* chosen);

/* ---- batched blocks ------------------------------------------------------ */

/* A handle on the same weights as `model` (device memory shared, not copied)
   with a context of its own: one per sequence for dflash_block_batch. Same
   geometry except max_context; `stream` as in dflash_create. The model's
   device must be current. Weights live until the last handle that shares
   them is destroyed. On failure *out is NULL and dflash_last_error(NULL)
   has the message. */
int dflash_create_context(const dflash_t* model, int64_t max_context, void* stream,
                          dflash_t** out);

/* The block pass of dflash_block for nseq (1..8) handles that share weights
   at once, each over its own context: the rows of all their blocks go
   through every weight matrix together (16 rows a sequence, padded to 4 or
   8 sequences), so each weight is read once for the batch (the pages'
   narrow/wide split: `mm` and `many` take a block's few rows on one kernel
   and many rows on another). d: host [nseq] handles, d[0] the lead (its
   stream runs the batch; the others' streams are ordered before and after
   it by events); anchors, a: host [nseq]. k and width as dflash_block, for
   every sequence. Outputs, dev, sequence-major: logits [nseq][k][width]
   (NULL: not written; copied from the batch's own buffer), cand, unary,
   score [nseq][k][selector_top], chosen [nseq][k]. Results equal
   dflash_block's on each handle to the parity tolerance (sums run in
   another order). The lead allocates its batch scratch at the first call.
   DFLASH_EINVAL for arguments dflash_block rejects, a handle that does not
   share the lead's weights, or rows waiting on any handle. */
int dflash_block_batch(dflash_t* const* d, int32_t nseq, const int32_t* anchors, const int64_t* a,
                       int32_t k, int32_t width, float* logits, int32_t* cand, float* unary,
                       float* score, int32_t* chosen);

/* ---- router ---------------------------------------------------------------- */

/* The router margin (`Route::margin` on the docs.rs page
   "cortiq_engine/dflash.rs"): which drafter a round is for. For each of m
   target rows x at the tip (dev f32 [m][hidden], the handle's hidden),
   u = x / max(‖x‖, 1e-12); for each subspace (mean dev f16 [hidden], basis
   dev f16 [rank][hidden] row-major, as the sidecar's fit holds them)
   err = ‖d − Σ_{r<rank} ⟨d, b_r⟩ b_r‖₂ with d = u − mean (the page names
   this reconstruction error without printing it: the residual's norm after
   removing d's components along the basis rows, the distance to the affine
   subspace for orthonormal rows); margin[i] = err(chain) − err(block),
   dev f32 [m]: above zero the round is the block drafter's. Requires
   1 ≤ m ≤ 64, ranks in [0, 256] (a basis may be NULL at rank 0). Runs on
   the handle's stream with the handle's own scratch (calls on one handle
   are ordered by its stream); changes no state. DFLASH_EINVAL for null
   pointers or sizes out of range. */
int dflash_route_margin(dflash_t* d, const float* rows, int32_t m, const uint16_t* block_mean,
                        const uint16_t* block_basis, int32_t block_rank,
                        const uint16_t* chain_mean, const uint16_t* chain_basis,
                        int32_t chain_rank, float* margin);

/* Forget the context from position pos on (`truncate`), waiting rows
   included; a layer that had dropped rows past pos holds none. */
int dflash_truncate(dflash_t* d, int64_t pos);

/* The span (`span`): *first and one past the last position, waiting rows
   included (`next_position`). */
int dflash_span(const dflash_t* d, int64_t* first, int64_t* end);

/* The context's bookkeeping: first position, settled rows, waiting rows,
   and (dropped non-NULL: host int64 [layers]) each layer's dropped rows, so
   that layer l holds positions first + dropped[l] .. first + settled. */
int dflash_state(const dflash_t* d, int64_t* first, int64_t* settled, int64_t* waiting,
                 int64_t* dropped);

/* Wait for every call enqueued so far. */
int dflash_sync(dflash_t* d);

/* Release every device buffer (after finishing the enqueued work). */
void dflash_destroy(dflash_t* d);

/* The message of the handle's last failure ("" if none); NULL handle: the
   last failure of dflash_create on this thread. */
const char* dflash_last_error(const dflash_t* d);

/* ---- stage timers -------------------------------------------------------- */

/* Per-stage device time, in the manner of the page's `CMF_DFLASH_TIME`
   stage timers (`stage`, `stage_report`): with timing on, every launch of a
   settle or block call is bracketed by hipEvents on the handle's stream and
   each call waits for its last event, so the totals are exact device times
   (and the calls no longer overlap the host). Stages, in order: */
enum {
  DFLASH_ST_KPROJ = 0,  /* kernel projections (both conv sets), f16 GEMM */
  DFLASH_ST_CONV,       /* embedding, row convolutions (the norms folded in), final norm */
  DFLASH_ST_QKV,        /* q/k/v int4 GEMM */
  DFLASH_ST_QKPOST,     /* q/k norms + rotary */
  DFLASH_ST_ATTN,       /* attention chunks + merge */
  DFLASH_ST_O,          /* o int4 GEMM */
  DFLASH_ST_GLU,        /* gate/up int4 GEMM with SwiGLU */
  DFLASH_ST_DOWN,       /* down int4 GEMM */
  DFLASH_ST_HEAD,       /* head (+ selector projection) f16 GEMM */
  DFLASH_ST_SELECT,     /* top-k + selector chain */
  DFLASH_ST_S_TAPS,     /* settle: tap rows to f16 */
  DFLASH_ST_S_FC,       /* settle: fc f16 GEMM */
  DFLASH_ST_S_NORM,     /* settle: fc split sums + hidden norm input (its scale is applied by
                           the store stage) */
  DFLASH_ST_S_KV,       /* settle: all layers' K/V int4 GEMM */
  DFLASH_ST_S_STORE,    /* settle: k norm + rotary + store append */
  DFLASH_STAGES
};

/* Turn the timers on (1) or off (0); either way the totals restart. */
int dflash_set_timing(dflash_t* d, int on);

/* Totals since the last dflash_set_timing: us[s] microseconds and
   launches[s] kernel launches of stage s (arrays of DFLASH_STAGES), and the
   number of block and settle calls timed (any pointer may be NULL). */
int dflash_stage_times(const dflash_t* d, double* us, int64_t* launches, int64_t* blocks,
                       int64_t* settles);

/* Peaks this GPU sustains, to report a kernel's rate against the chip as
   measured here beside its spec sheet (8 TB/s HBM, 2.5 PFLOP/s dense f16):
   - read_gbs: a streaming read of the library's own head weights (every
     byte once a pass; each wave a contiguous chunk with eight 1 KB blocks in
     flight, non-temporal 16-byte loads, 16 workgroups per compute unit),
     `reps` passes, in GB/s;
   - mfma_tfs: back-to-back v_mfma_f32_16x16x32_f16 on register operands,
     two waves per SIMD, in TFLOP/s.
   Runs on the library stream, timed with HIP events, and synchronises it.
   reps in [1, 100]; -1 on a bad argument, -3 on a HIP error. */
int dflash_probe_peaks(dflash_t* d, int32_t reps, double* read_gbs, double* mfma_tfs);

/* ---- test entry points: each kernel on caller buffers ---------------------- */

/* Matrix ids for the debug entry points (`layer` is ignored for the
   sidecar-wide ones). */
enum {
  DFLASH_W_Q = 0, DFLASH_W_K, DFLASH_W_V, DFLASH_W_O, DFLASH_W_GATE, DFLASH_W_UP,
  DFLASH_W_DOWN, DFLASH_W_ATTN_KPROJ, DFLASH_W_MLP_KPROJ, DFLASH_W_FC, DFLASH_W_HEAD,
  DFLASH_W_SEL
};

/* The int4 matrix `which` (Q..DOWN) of `layer` as the device holds it,
   dequantised: dev f32 [rows][cols], element q·scale. */
int dflash_debug_dequant(dflash_t* d, int32_t layer, int32_t which, float* out);

/* y = W·x with the product path's GEMM kernels: x dev f32 [m][cols],
   y dev f32 [m][rows], m in [1, 256]. x enters as every operand of the
   block and settle passes does: two f16 planes, hi and the rest. */
int dflash_debug_matvec(dflash_t* d, int32_t layer, int32_t which, const float* x, int32_t m,
                        float* y);

/* Copy the rows of positions first+row0 .. first+row0+n−1 from layer's
   store (rows the layer holds: dropped ≤ row0, row0 + n ≤ settled):
   k_out, v_out dev f32 [n][kv_heads*head_dim]. The store keeps each f32
   value x as its f16 pair (hi = f16(x), lo = f16(x − hi)), the form the
   attention multiplies; a read returns hi + lo. */
int dflash_debug_read_store(dflash_t* d, int32_t layer, int64_t row0, int64_t n, float* k_out,
                            float* v_out);

/* Replace the context with `len` given rows at positions first..first+len−1,
   as if one settle had made them on an empty context (waiting rows go;
   each windowed layer then drops rows as after a settle): k[l], v[l] (host
   array of `layers` dev pointers) dev f32 [len][kv*hd], each value stored
   as its f16 pair like a settled one. */
int dflash_debug_load_store(dflash_t* d, int64_t first, int64_t len, const float* const* k,
                            const float* const* v);

/* From the last dflash_block: every row after the final norm, dev f32
   [block][hidden], and the selector projection of rows 1..k, dev f32
   [k][selector_rank] (either may be NULL). */
int dflash_debug_last_block(dflash_t* d, float* hidden, float* hp);

/* With trace non-NULL, later blocks also copy the residual rows after each
   layer into trace, dev f32 [layers][block][hidden]; NULL stops it. */
int dflash_debug_set_trace(dflash_t* d, float* trace);

/* The selector alone on given logits (dev f32 [k][width]) and projections
   hp (dev f32 [k][rank]); forced_prev (dev int32 [k] or NULL) replaces prev
   of every row j ≥ 1. Outputs as dflash_block. */
int dflash_debug_select(dflash_t* d, const float* logits, const float* hp, int32_t k,
                        int32_t width, int32_t anchor_token, const int32_t* forced_prev,
                        int32_t* cand, float* unary, float* score, int32_t* chosen);

#ifdef __cplusplus
}
#endif
#endif
