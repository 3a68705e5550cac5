// Host side of the C-ABI library: validation, the sidecar onto the card
// (repacked into the kernels' tile layouts), the context store and its
// position rule, and the launch sequences of the settle and block passes.
//
// Definitions followed (docs.rs page "cortiq_engine/dflash.rs",
// cortiq-engine 0.8.78): `Geometry::of` (what a geometry must satisfy),
// `queue_context` / `truncate` (the position rule), `settle_rows` (the
// context rows, 256 at a time as the CUDA block takes them), `block_dev`
// (each layer's context range), `Drafter::block`, `select_with`.
#include "dflash.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

#include "internal.h"

namespace {

constexpr int kSettleRows = 256;     // rows one settle pass takes
constexpr int kTargetBlocks = 512;   // workgroups a GEMM launch aims for (256 CUs)
constexpr int kR = 2;        // row tiles per wave of the skinny GEMMs (8 a workgroup)
// the block's int4 GEMMs: row tiles a wave and spans (128 columns) a split
constexpr int kRQkv = 2, kKsQkv = 8;    // q/k/v
constexpr int kRO = 2, kKsO = 2;        // o
constexpr int kRDown = 2, kKsDown = 8;  // down
constexpr int kSettleI4Blocks = 2;  // above this many 16-row blocks the settle's k/v use the many-row kernel
// `queue_context`: at most kPendingRows rows wait (as many as the widest
// window plus kBlockSlack when every layer is windowed); past that the
// oldest go through in multiples of kContextChunk rows
constexpr long kPendingRows = 512, kContextChunk = 64, kBlockSlack = 256;

thread_local std::string g_create_error;

struct Split {
  int S, per;
};

// K splits for a GEMM of `ntiles` row tiles with R tiles per wave, `steps`
// K steps (32 columns for f16, 128 for int4) and `mblocks` 16-row blocks;
// every split keeps at least `min_per` steps.
Split split_for(int ntiles, int R, int steps, int mblocks, int min_per) {
  const long groups = (ntiles + 4L * R - 1) / (4L * R);
  const long have = groups * mblocks;
  long S = (kTargetBlocks + have - 1) / have;
  S = std::max(1L, std::min<long>(S, std::max(1, steps / min_per)));
  const int per = (int)((steps + S - 1) / S);
  return {(int)((steps + per - 1) / per), per};
}

// K splits of the settle's many-row K/V kernel (16 weight tiles a block, K in
// 128-column spans): about one block per CU.
Split split_kv(int ntiles, int spans) {
  const long groups = dfl::kv_i4_groups(ntiles);
  long S = std::max(1L, std::min<long>(256 / groups, spans));
  const int per = (int)((spans + S - 1) / S);
  return {(int)((spans + per - 1) / per), per};
}

// K splits of the many-row f16 GEMM (16 weight tiles a block): about one
// block per CU, every split keeping at least 16 steps (512 columns) and an
// even number of them (the kernel takes its steps in pairs; `steps`, K/32,
// is even since K is a multiple of 128).
Split split_big(int ntiles, int steps) {
  const long groups = (ntiles + 15) / 16;
  long S = std::max(1L, std::min<long>(256 / groups, steps / 16));
  int per = (int)((steps + S - 1) / S);
  per += per & 1;
  return {(int)((steps + per - 1) / per), per};
}

// K splits of a batched product (16 weight tiles a workgroup): the count
// that finishes soonest when the workgroups run in rounds of `slots` (two a
// compute unit at 4 row blocks, one at 8: their LDS), i.e. the least
// rounds / S, the smaller S among near ties. At most 8 splits at 4 row
// blocks and 16 at 8 (each split writes a whole [rows][N] partial): with the
// int4 ring no longer drained every step, 16 at 8 blocks measured 3201 ->
// 3103 us a B = 8 pass and 16 at 4 blocks 2034 -> 2100 us for B = 4 (one box).
Split split_mb(int ntiles, int units, int MB) {
  const long groups = dfl::mb_groups(ntiles);
  const long slots = MB == 4 ? 512 : 256, cap = MB == 8 ? 16 : 8;
  long S = 1;
  double best = 1e30;
  for (long c = 1; c <= std::min<long>(cap, units); ++c) {
    const double t = (double)((groups * c + slots - 1) / slots) / c;
    if (t < best * 0.9) {
      best = t;
      S = c;
    }
  }
  const int per = (int)((units + S - 1) / S);
  return {(units + per - 1) / per, per};
}

void parallel_for(long n, const std::function<void(long)>& f) {
  unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (n < 64) nt = 1;
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (long i = t; i < n; i += nt) f(i);
    });
  for (auto& x : th) x.join();
}

// Dense f16 [N][K] → F16T with rows padded to a multiple of 16 (zeros).
std::vector<uint16_t> repack_f16(const uint16_t* src, int N, int K) {
  const int KS = K / 32, NT = (N + 15) / 16;
  std::vector<uint16_t> dst((size_t)NT * 16 * K);
  parallel_for(NT, [&](long t) {
    for (int s = 0; s < KS; ++s)
      for (int l = 0; l < 64; ++l) {
        const int j = l >> 4, n = l & 15;
        const long row = 16 * t + n;
        uint16_t* d = dst.data() + (((size_t)t * KS + s) * 64 + l) * 8;
        if (row < N)
          std::memcpy(d, src + (size_t)row * K + 32 * s + 8 * j, 16);
        else
          std::memset(d, 0, 16);
      }
  });
  return dst;
}

// int4 [N][K] → I4T tiles written at tile offset `t_off` of codes/scales.
void repack_i4(const dflash_i4& m, int N, int K, uint8_t* codes, uint16_t* scales, long t_off) {
  const int KT = K / 128, NT = N / 16;
  parallel_for(NT, [&](long t) {
    const long tt = t + t_off;
    for (int p = 0; p < KT; ++p)
      for (int l = 0; l < 64; ++l) {
        const int j = l >> 4, n = l & 15;
        const long row = 16 * t + n;
        const uint8_t* qr = m.q + (size_t)row * (K / 2);
        for (int u = 0; u < 4; ++u) {
          uint32_t word = 0;
          for (int e = 0; e < 8; ++e) {
            const int k = 128 * p + 32 * u + 8 * j + e;
            const uint32_t nib = (k & 1) ? (qr[k / 2] >> 4) : (qr[k / 2] & 15);
            const int pos = (e & 1) ? 16 + 2 * (e - 1) : 2 * e;
            word |= (nib ^ 8u) << pos;
          }
          std::memcpy(codes + (((size_t)tt * KT + p) * 64 + l) * 16 + 4 * u, &word, 4);
          if (j == 0) scales[(((size_t)tt * KT + p) * 16 + n) * 4 + u] = m.scale[(size_t)row * (K / 32) + 4 * p + u];
        }
      }
  });
}

}  // namespace

// Per-call scratch of the block pass: activations, GEMM and attention
// partial results, the selection's lists and counters.
struct BlockScratch {
  float *h = nullptr, *x = nullptr, *dsum_a = nullptr, *dsum_m = nullptr, *pacc = nullptr,
        *pml = nullptr, *part = nullptr, *logits = nullptr, *hp = nullptr, *sqp = nullptr;
  uint16_t *xa = nullptr, *xca = nullptr, *qa = nullptr, *ya = nullptr, *ma = nullptr;
  uint16_t *kb = nullptr, *vb = nullptr;  // the block's keys and values, f16-pair rows
  dfl::SelectScratch sel{};
};

struct I4Set {  // one int4 product of every layer, tiles [layer][tiles][K/128]
  uint8_t* codes = nullptr;
  uint16_t* scales = nullptr;
  int tiles = 0, K = 0;
  long layer_tiles() const { return tiles; }
};

// The device weights, shared by every handle made from them (a handle and
// the contexts made from it with dflash_create_context); freed with the last.
struct WeightOwner {
  std::vector<void*> allocs;
  ~WeightOwner() {
    for (void* p : allocs) (void)hipFree(p);
  }
};

// Scratch of batched blocks (dflash_block_batch), the lead handle's, sized
// for dfl::kMaxSeq sequences (8 A-layout row blocks) at its first batched
// call.
struct BatchScratch {
  float *h = nullptr, *dsum_a = nullptr, *dsum_m = nullptr, *pacc = nullptr, *pml = nullptr,
        *part = nullptr, *logits = nullptr, *hp = nullptr, *sqp = nullptr;
  uint16_t *xa = nullptr, *xca = nullptr, *qa = nullptr, *ya = nullptr, *ma = nullptr;
  uint16_t *kb = nullptr, *vb = nullptr;
  dfl::SelectScratch sel{};  // kMaxSeq sets (select_batch)
  long part_floats = 0;
  bool ready = false;
};

struct dflash {
  // geometry
  int hs, ffn, L, nh, kv, hd, V, B, mask, gs, kn, rank, top, ntaps, tw, qd, kd, G, P;
  std::vector<int> windows, rot;
  double theta;
  float eps;
  long maxctx;  // rows a layer may hold at most
  hipStream_t st;
  // weights
  uint16_t *fc = nullptr, *sel = nullptr, *pbook = nullptr, *cbook = nullptr, *embed = nullptr,
           *head = nullptr, *attn_kproj = nullptr, *mlp_kproj = nullptr;
  float *hidden_norm = nullptr, *norm = nullptr, *in_norm = nullptr, *post_norm = nullptr,
        *q_norm = nullptr, *k_norm = nullptr, *attn_base = nullptr, *mlp_base = nullptr,
        *inv = nullptr;
  int* rot_dev = nullptr;
  I4Set qkv, o, gu, down;
  int ptiles;  // kernel-projection row tiles
  // the context (`Ctx`): settled positions first .. first+len; per layer a
  // ring store of the rows it still holds; tap rows that wait to be settled
  long first = 0, len = 0;
  struct LayerStore {
    // rings of cap rows of f16 pairs, kv head major ([kv][cap][hi hd | lo
    // hd], 4·kd bytes a row); position p at row (p − first) mod cap
    uint16_t *k = nullptr, *v = nullptr;
    long cap = 0;
    long limit = 0;    // most rows the layer may hold (a windowed layer's ring is this big)
    long dropped = 0;  // settled rows the layer no longer holds (`Ctx::dropped`)
  };
  std::vector<LayerStore> ls;
  dfl::StoreSlot* tab = nullptr;  // every layer's (k, v, cap), for the settle's store kernel
  float* pq = nullptr;            // waiting tap rows: a ring of pcap rows from row phead
  long pcap = 0, phead = 0, pend = 0;
  int dev = 0;  // the device the handle was created on
  // block scratch (the handle's own; dflash_block_noalloc carves the same set
  // from the library's static array instead)
  BlockScratch bs;
  // settle scratch (part and sqp are shared with bs)
  float *part = nullptr, *sqp = nullptr;
  uint16_t *taps_a = nullptr, *t_a = nullptr;
  long part_floats = 0;
  int stage_cols = 0;  // widest activation the staging buffer holds
  int last_k = 0;
  float* trace = nullptr;  // per-layer residual copies (debug)
  float *rt_coef = nullptr, *rt_nrm = nullptr, *rt_part = nullptr;  // router margin scratch
  std::vector<void*> allocs;     // the handle's own device buffers (not the weights)
  std::shared_ptr<WeightOwner> wown;
  BatchScratch bb;
  hipEvent_t order = nullptr;  // orders a batched call against this handle's stream
  std::string err;
  struct Timing {
    bool on = false;
    std::vector<hipEvent_t> ev;            // event pool, grown on demand
    int used = 0;
    std::vector<std::pair<int, int>> marks;  // (stage, event) after each launch
    double us[DFLASH_STAGES] = {};
    int64_t launches[DFLASH_STAGES] = {};
    int64_t blocks = 0, settles = 0;
  } tm;
};

namespace {

int fail(dflash* d, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (d)
    d->err = buf;
  else
    g_create_error = buf;
  return code;
}

// Bytes of one store row: kd keys (or values), each as its f16 pair.
size_t store_row_bytes(const dflash* d) { return 2 * (size_t)d->kd * sizeof(uint16_t); }

int hip_check(dflash* d, hipError_t e, const char* what) {
  if (e == hipSuccess) return DFLASH_OK;
  return fail(d, e == hipErrorOutOfMemory ? DFLASH_ENOMEM : DFLASH_EHIP, "%s: %s", what,
              hipGetErrorString(e));
}

template <class T>
int dev_alloc(dflash* d, T** p, size_t count, const char* what) {
  void* q = nullptr;
  const hipError_t e = hipMalloc(&q, std::max<size_t>(count * sizeof(T), 16));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(nullptr, DFLASH_ENOMEM, "device memory for %s (%zu bytes): %s", what,
                count * sizeof(T), hipGetErrorString(e));
  }
  d->allocs.push_back(q);
  *p = static_cast<T*>(q);
  return hipMemset(q, 0, std::max<size_t>(count * sizeof(T), 16)) == hipSuccess
             ? DFLASH_OK
             : fail(nullptr, DFLASH_EHIP, "clearing %s", what);
}

template <class T>
int upload(dflash* d, T** p, const T* src, size_t count, const char* what) {
  int rc = dev_alloc(d, p, count, what);
  if (rc) return rc;
  if (hipMemcpy(*p, src, count * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
    return fail(nullptr, DFLASH_EHIP, "copying %s to the device", what);
  return DFLASH_OK;
}

int launch_check(dflash* d, const char* what) {
  return hip_check(d, hipGetLastError(), what);
}

// ---- stage timers: an event after every launch, resolved at the call's end
void tm_record(dflash* d) {
  auto& t = d->tm;
  if (t.used == (int)t.ev.size()) {
    hipEvent_t e;
    (void)hipEventCreate(&e);
    t.ev.push_back(e);
  }
  (void)hipEventRecord(t.ev[t.used++], d->st);
}

void tm_begin(dflash* d) {
  if (!d->tm.on) return;
  d->tm.used = 0;
  d->tm.marks.clear();
  tm_record(d);
}

void tm_mark(dflash* d, int stage) {
  if (!d->tm.on) return;
  tm_record(d);
  d->tm.marks.emplace_back(stage, d->tm.used - 1);
}

void tm_end(dflash* d) {
  auto& t = d->tm;
  if (!t.on || t.used == 0) return;
  (void)hipEventSynchronize(t.ev[t.used - 1]);
  int prev = 0;
  for (auto& m : t.marks) {
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, t.ev[prev], t.ev[m.second]);
    t.us[m.first] += 1000.0 * ms;
    t.launches[m.first] += 1;
    prev = m.second;
  }
}

const char* validate(const dflash_geometry* g, const dflash_weights* w) {
  if (!g || !w) return "null geometry or weights";
  if (g->layers <= 0) return "layers must be > 0";
  if (g->block < 2 || g->block > 16) return "block must be in [2, 16]";
  if (g->n_taps <= 0) return "n_taps must be > 0";
  if (g->kv_heads <= 0 || g->heads <= 0 || g->heads % g->kv_heads) return "heads % kv_heads";
  if (g->head_dim != 64 && g->head_dim != 128 && g->head_dim != 256)
    return "head_dim must be 64, 128 or 256";
  if (g->conv_group <= 0 || g->hidden % g->conv_group) return "hidden % conv_group";
  if (g->conv_kernel < 1 || g->conv_kernel > g->block) return "conv_kernel must be in [1, block]";
  if (g->hidden <= 0 || g->hidden % 128) return "hidden must be a multiple of 128";
  // gate/up streams each wave's share of K through registers: at most 40
  // spans of 128 columns over eight waves
  if (!dfl::glu_stream_fits(g->hidden)) return "hidden must be at most 5120";
  if (g->intermediate <= 0 || g->intermediate % 128) return "intermediate must be a multiple of 128";
  if ((g->heads * g->head_dim) % 128) return "heads*head_dim must be a multiple of 128";
  if (2L * g->conv_kernel * (g->hidden / g->conv_group) > 16384)
    return "2*conv_kernel*hidden/conv_group must be at most 16384";
  if (g->selector_top < 1 || g->selector_top > 32 || g->selector_top > g->vocab)
    return "selector_top must be in [1, min(32, vocab)]";
  if (g->selector_rank < 1 || g->selector_rank > 256) return "selector_rank must be in [1, 256]";
  if (g->vocab > 262144) return "vocab must be at most 262144";
  if (g->mask_token < 0 || g->mask_token >= g->vocab) return "mask_token outside the vocabulary";
  if (g->max_context < 1) return "max_context must be >= 1";
  if (!g->windows || !g->rotary) return "null windows or rotary";
  for (int l = 0; l < g->layers; ++l)
    if (g->windows[l] < 0) return "negative window";
  if (!w->fc || !w->hidden_norm || !w->norm || !w->sel_proj || !w->pred_book || !w->succ_book ||
      !w->embed || !w->head || !w->layer)
    return "null weight pointer";
  for (int l = 0; l < g->layers; ++l) {
    const dflash_layer_w& x = w->layer[l];
    if (!x.in_norm || !x.post_norm || !x.q_norm || !x.k_norm || !x.attn_base || !x.mlp_base ||
        !x.attn_kproj || !x.mlp_kproj)
      return "null layer weight pointer";
    for (const dflash_i4* m : {&x.q, &x.k, &x.v, &x.o, &x.gate, &x.up, &x.down})
      if (!m->q || !m->scale) return "null int4 matrix";
  }
  return nullptr;
}

int alloc_i4(dflash* d, I4Set& s, int tiles, int K, const char* what) {
  s.tiles = tiles;
  s.K = K;
  const size_t n = (size_t)d->L * tiles * (K / 128);
  int rc = dev_alloc(d, &s.codes, n * 64 * 16, what);
  if (!rc) rc = dev_alloc(d, &s.scales, n * 16 * 4, what);
  return rc;
}

int upload_i4(dflash* d, I4Set& s, int l, std::initializer_list<std::pair<const dflash_i4*, int>> parts) {
  const int KT = s.K / 128;
  std::vector<uint8_t> codes((size_t)s.tiles * KT * 64 * 16);
  std::vector<uint16_t> scales((size_t)s.tiles * KT * 16 * 4);
  long t_off = 0;
  for (auto& pr : parts) {
    repack_i4(*pr.first, pr.second, s.K, codes.data(), scales.data(), t_off);
    t_off += pr.second / 16;
  }
  const size_t lc = codes.size(), ls = scales.size();
  if (hipMemcpy(s.codes + (size_t)l * lc, codes.data(), lc, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(s.scales + (size_t)l * ls, scales.data(), ls * 2, hipMemcpyHostToDevice) != hipSuccess)
    return fail(nullptr, DFLASH_EHIP, "copying int4 weights to the device");
  return DFLASH_OK;
}

// Largest GEMM partial buffer (floats) any call can need.
long partial_need(const dflash* d) {
  long need = 0;
  auto i4 = [&](int N, int K, int mb, int R) {
    const Split s = split_for(N / 16, R, K / 128, mb, 4);
    need = std::max(need, (long)s.S * mb * 16 * N);
  };
  auto f16b = [&](int N, int K) {
    need = std::max(need, (long)dfl::f16_block_splits(K) * 16 * N);
  };
  f16b(d->P, d->hs);
  for (int N : {d->hs, d->P, d->rank}) f16b(N, d->hs);
  f16b(d->hs, d->tw);
  auto i4b = [&](int N, int K, int ks) {
    need = std::max(need, (long)dfl::i4_block_splits(K, ks) * 16 * N);
  };
  i4b(d->qd + 2 * d->kd, d->hs, kKsQkv);
  i4b(d->L * 2 * d->kd, d->hs, kKsQkv);  // a one-block settle's K/V
  i4b(d->hs, d->qd, kKsO);
  i4b(d->hs, d->ffn, kKsDown);
  for (int N : {d->qd, d->kd, d->ffn}) i4b(N, d->hs, 2);
  i4b(d->hs, d->qd, 2);
  i4b(d->hs, d->ffn, 2);
  for (int mb = kSettleI4Blocks + 1; mb <= kSettleRows / 16; ++mb) {
    const Split s = split_kv(d->L * 2 * d->kd / 16, d->hs / 128);
    need = std::max(need, (long)s.S * mb * 16 * d->L * 2 * d->kd);
  }
  for (int mb = 2; mb <= kSettleRows / 16; ++mb)
    for (int N : {d->hs, d->P, d->rank}) {
      const int K = N == d->hs ? d->tw : d->hs;
      const Split s = split_big((N + 15) / 16, K / 32);
      need = std::max(need, (long)s.S * mb * 16 * N);
      const Split s2 = split_big((N + 15) / 16, d->hs / 32);
      need = std::max(need, (long)s2.S * mb * 16 * N);
    }
  for (int mb = 1; mb <= kSettleRows / 16; ++mb) {
    i4(d->L * 2 * d->kd, d->hs, mb, kR);
    for (int N : {d->qd, d->kd, d->ffn}) i4(N, d->hs, mb, kR);
    i4(d->hs, d->qd, mb, kR);
    i4(d->hs, d->ffn, mb, kR);
  }
  return need;
}

void layer_range(const dflash* d, int l, long a, long* lo, long* n) {
  // `block_dev`: base = first + dropped (the layer's first held position);
  // hi = min(a, first+len), never below base; a window w > 0 starts the
  // layer at a+1−w, clamped into [base, hi].
  const long base = d->first + d->ls[l].dropped;
  long hi = std::min(a, d->first + d->len);
  hi = std::max(hi, base);
  long l0 = base;
  const int w = d->windows[l];
  if (w > 0) l0 = std::min(std::max(std::max(a + 1 - w, 0L), base), hi);
  *lo = l0;
  *n = hi - l0;
}

// ---- the context lifecycle (`queue_context`, `settle`, `settle_rows`,
// `truncate`, `Dev::reserve`)

// The device table of the layers' stores, after a store moved.
// (err: the handle that keeps the message, nullptr while creating)
int upload_tab(dflash* d, dflash* err) {
  std::vector<dfl::StoreSlot> t(d->L);
  for (int l = 0; l < d->L; ++l) t[l] = {d->ls[l].k, d->ls[l].v, std::max(1L, d->ls[l].cap)};
  return hip_check(err, hipMemcpy(d->tab, t.data(), t.size() * sizeof t[0], hipMemcpyHostToDevice),
                   "context table");
}

// The context's bookkeeping alone: the position rule and the window drop
// are worked out on a copy, checked, and only then committed.
struct CtxState {
  long first, len, pend, phead;
  std::vector<long> dropped;
};

CtxState state_of(const dflash* d) {
  CtxState s{d->first, d->len, d->pend, d->phead, {}};
  for (const auto& l : d->ls) s.dropped.push_back(l.dropped);
  return s;
}

void commit(dflash* d, const CtxState& s) {
  d->first = s.first;
  d->len = s.len;
  d->pend = s.pend;
  d->phead = s.phead;
  for (int l = 0; l < d->L; ++l) d->ls[l].dropped = s.dropped[l];
}

// `truncate`: forget positions from pos on, waiting rows included.
void truncate_state(CtxState& s, long pos) {
  s.pend = std::min(s.pend, std::max(0L, pos - (s.first + s.len)));
  const long keep = std::min(std::max(0L, pos - s.first), s.len);
  for (long& dr : s.dropped) dr = std::min(dr, keep);
  s.len = keep;
}

// The position rule of `queue_context`: rows at a held or waiting position
// cut the context there; a gap, or a position before first, restarts it.
void position_rule(CtxState& s, long pos) {
  if (pos > s.first + s.len + s.pend || pos < s.first) {
    truncate_state(s, 0);
    s.first = pos;
    s.phead = 0;
  } else {
    truncate_state(s, pos);
  }
}

// One `settle_rows` call of n rows on the bookkeeping: the rows join, then a
// windowed layer that holds more than twice its window keeps the last
// window's rows. False if a layer would hold more rows than it may (a
// windowed layer's peak inside the call is what it holds after it).
bool settle_state(const dflash* d, CtxState& s, long n) {
  s.len += n;
  for (int l = 0; l < d->L; ++l) {
    const long w = d->windows[l];
    long held = s.len - s.dropped[l];
    if (w > 0 && held > 2 * w) {
      s.dropped[l] += held - w;
      held = w;
    }
    if (held > d->ls[l].limit) return false;
  }
  return true;
}

// Room for `rows` rows in every full layer (`Dev::reserve`): a store that is
// too small grows to max(rows, 2·cap, 4096) rows, at most max_context, and
// keeps what it held. Synchronises the stream when a store moves.
int reserve(dflash* d, long rows) {
  if (rows > d->maxctx)
    return fail(d, DFLASH_ENOMEM, "%ld rows do not fit a layer's store (max_context %ld)", rows,
                d->maxctx);
  bool moved = false;
  for (int l = 0; l < d->L; ++l) {
    auto& S = d->ls[l];
    if (d->windows[l] > 0 || rows <= S.cap) continue;
    const long cap = std::min(std::max(std::max(rows, 2 * S.cap), 4096L), d->maxctx);
    const size_t bytes = (size_t)cap * store_row_bytes(d);
    uint16_t *nk = nullptr, *nv = nullptr;
    if (hipMalloc(&nk, bytes) != hipSuccess || hipMalloc(&nv, bytes) != hipSuccess) {
      (void)hipGetLastError();
      if (nk) (void)hipFree(nk);
      return fail(d, DFLASH_ENOMEM, "device memory for layer %d's context (%zu bytes)", l,
                  2 * bytes);
    }
    // a full layer holds positions first .. first+len at rows 0 .. len of
    // every kv head's ring
    const size_t hrow = store_row_bytes(d) / d->kv;  // one kv head's row
    const size_t held = (size_t)std::min(d->len, S.cap) * hrow;
    int rc = DFLASH_OK;
    if (held)
      rc = hip_check(d, hipMemcpy2DAsync(nk, cap * hrow, S.k, S.cap * hrow, held, d->kv,
                                         hipMemcpyDeviceToDevice, d->st),
                     "reserve");
    if (!rc && held)
      rc = hip_check(d, hipMemcpy2DAsync(nv, cap * hrow, S.v, S.cap * hrow, held, d->kv,
                                         hipMemcpyDeviceToDevice, d->st),
                     "reserve");
    if (!rc) rc = hip_check(d, hipStreamSynchronize(d->st), "reserve");
    if (rc) {
      (void)hipFree(nk);
      (void)hipFree(nv);
      return rc;
    }
    if (S.k) (void)hipFree(S.k);
    if (S.v) (void)hipFree(S.v);
    S.k = nk;
    S.v = nv;
    S.cap = cap;
    moved = true;
  }
  return moved ? upload_tab(d, d) : DFLASH_OK;
}

// A launch failed while rows were being settled: what the layers hold can
// no longer be told, so the context is emptied (first stays).
void lose_context(dflash* d) {
  d->len = 0;
  d->pend = 0;
  d->phead = 0;
  for (auto& l : d->ls) l.dropped = 0;
}

// The rows of one `settle_rows` call: up to three runs of consecutive tap
// rows, in order (the waiting ring's two pieces, then the caller's rows).
struct Runs {
  const float* p[3] = {nullptr, nullptr, nullptr};
  long n[3] = {0, 0, 0};
  int k = 0;
  void add(const float* q, long m) {
    if (m > 0) p[k] = q, n[k++] = m;
  }
};

// Runs of the waiting rows [from, from+count) of the ring.
void add_waiting(const dflash* d, Runs& r, long from, long count) {
  const long i = (d->phead + from) % d->pcap, a = std::min(count, d->pcap - i);
  r.add(d->pq + (size_t)i * d->tw, a);
  r.add(d->pq, count - a);
}

int attn_chunk(long n, int* nchunks) {
  if (n <= 0) {
    *nchunks = 0;
    return 32;
  }
  // at least 128 keys a chunk: shorter chunks cost more in per-chunk work and
  // merge traffic than they gain in parallelism
  long c = std::max(128L, (n + dfl::kAttnMaxChunks - 1) / dfl::kAttnMaxChunks);
  c = (c + 31) / 32 * 32;
  // Longer chunks take an odd number of 32-key steps: the workgroups walk
  // their chunks in step, and chunks a power of two of rows apart would have
  // them all at the same offset within equal-sized address blocks at once
  // (measured: a pure read of the pattern goes from 6.57 to 6.92 TB/s).
  if (c > 128 && (c / 32) % 2 == 0) c += 32;
  *nchunks = (int)((n + c - 1) / c);
  return (int)c;
}

// ---- the static scratch of dflash_block_noalloc

// Bytes of the library's static scratch on each GPU: a block pass's per-call
// scratch of the 27B-shaped sidecar takes about 26 MB of it.
constexpr size_t kNoallocScratchBytes = DFLASH_NOALLOC_SCRATCH_BYTES;

}  // namespace

// The file-scope device array dflash_block_noalloc takes its scratch from.
// In host code its name is only a stand-in: its device address is looked up
// once per device (hipGetSymbolAddress) and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
bool g_scratch_tried[kMaxDevices] = {};

// Look the array's address up on device `dev` (current), once.
void scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_tried[dev]) return;
  g_scratch_tried[dev] = true;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess)
    g_scratch[dev] = p;
  else
    (void)hipGetLastError();
}

void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[dev];
}

// Lay the block pass's scratch out from base (256-byte aligned pieces); with
// base == nullptr only count. Returns the bytes taken. The logits are the
// caller's (no scratch copy).
size_t carve_block_scratch(const dflash* d, uint8_t* base, BlockScratch* out) {
  size_t off = 0;
  auto take = [&](auto** p, size_t count) {
    using T = std::remove_pointer_t<std::remove_reference_t<decltype(*p)>>;
    off = (off + 255) / 256 * 256;
    if (base) *p = reinterpret_cast<T*>(base + off);
    off += count * sizeof(T);
  };
  BlockScratch tmp;
  BlockScratch& b = out ? *out : tmp;
  const size_t hs = d->hs;
  long part = 0;
  part = std::max(part, (long)dfl::f16_block_splits(d->hs) * 16 * d->P);
  part = std::max(part, (long)dfl::i4_block_splits(d->hs, kKsQkv) * 16 * (d->qd + 2 * d->kd));
  part = std::max(part, (long)dfl::i4_block_splits(d->qd, kKsO) * 16 * d->hs);
  part = std::max(part, (long)dfl::i4_block_splits(d->ffn, kKsDown) * 16 * d->hs);
  const size_t slots = (size_t)d->kv * (dfl::kAttnMaxChunks + 1) * (d->nh / d->kv);
  const size_t cap = (size_t)dfl::topk_cap(d->V, d->top);
  take(&b.h, 16 * hs);
  take(&b.x, 16 * hs);
  take(&b.dsum_a, 16 * (size_t)d->P);
  take(&b.dsum_m, 16 * (size_t)d->P);
  take(&b.kb, 2 * 16 * (size_t)d->kd);
  take(&b.vb, 2 * 16 * (size_t)d->kd);
  take(&b.pacc, slots * 16 * d->hd);
  take(&b.pml, slots * 16 * 2);
  take(&b.part, (size_t)part);
  take(&b.hp, 16 * (size_t)d->rank);
  take(&b.sqp, 16 * (size_t)std::max(dfl::row_chunks(d->hs), dfl::conv1_chunks(d->hs)));
  take(&b.xa, 2 * 16 * hs);
  take(&b.xca, 2 * 16 * hs);
  take(&b.qa, 2 * (size_t)d->nh * 16 * d->hd);
  take(&b.ya, 2 * 16 * (size_t)d->qd);
  take(&b.ma, 2 * 16 * (size_t)d->ffn);
  take(&b.sel.gmax, 16 * (size_t)((d->V + 255) / 256));
  take(&b.sel.counters, 16);
  take(&b.sel.lv, 16 * cap);
  take(&b.sel.li, 16 * cap);
  take(&b.sel.tab, (size_t)d->top * (1 + 15 * d->top));
  take(&b.sel.best, (size_t)(1 + 15 * d->top));
  b.logits = nullptr;
  return off;
}

}  // namespace

// ====================================================================== API

extern "C" {

const char* dflash_last_error(const dflash_t* d) {
  return d ? d->err.c_str() : g_create_error.c_str();
}

void dflash_destroy(dflash_t* d) {
  if (!d) return;
  (void)hipStreamSynchronize(d->st);
  for (hipEvent_t e : d->tm.ev) (void)hipEventDestroy(e);
  if (d->order) (void)hipEventDestroy(d->order);
  for (void* p : d->allocs) (void)hipFree(p);
  for (auto& l : d->ls) {
    if (l.k) (void)hipFree(l.k);
    if (l.v) (void)hipFree(l.v);
  }
  delete d;
}

// Everything a handle owns beyond the weights: its context stores, the
// waiting rows' ring and the scratch of both passes. Errors go to the
// create error (the handle is not out yet).
static int alloc_state(dflash* d) {
  int rc = DFLASH_OK;
  const int L = d->L, hs = d->hs;
  // ---- context: a windowed layer's ring of min(2·window, max_context) rows
  // now; a full layer's store grows as rows come (`Dev::reserve`); the
  // waiting rows' ring
  d->ls.resize(L);
  for (int l = 0; l < L && !rc; ++l) {
    auto& S = d->ls[l];
    const long w = d->windows[l];
    S.limit = w > 0 ? std::min(2 * w, d->maxctx) : d->maxctx;
    if (w > 0) {
      const size_t bytes = (size_t)S.limit * store_row_bytes(d);
      if (hipMalloc(&S.k, bytes) != hipSuccess || hipMalloc(&S.v, bytes) != hipSuccess) {
        (void)hipGetLastError();
        rc = fail(nullptr, DFLASH_ENOMEM, "device memory for layer %d's context (%zu bytes)", l,
                  2 * bytes);
      }
      S.cap = S.limit;
    }
  }
  if (!rc) rc = dev_alloc(d, &d->tab, L, "context table");
  if (!rc) rc = upload_tab(d, nullptr);
  d->pcap = kPendingRows;
  if (std::all_of(d->windows.begin(), d->windows.end(), [](int w) { return w > 0; }))
    d->pcap = std::max(kPendingRows,
                       (long)*std::max_element(d->windows.begin(), d->windows.end()) + kBlockSlack);
  if (!rc) rc = dev_alloc(d, &d->pq, (size_t)d->pcap * d->tw, "waiting rows");
  // ---- scratch
  const int rep = d->nh / d->kv;
  const size_t slots = (size_t)d->kv * (dfl::kAttnMaxChunks + 1) * rep;
  d->part_floats = partial_need(d);
  const size_t sel_cap = (size_t)dfl::topk_cap(d->V, d->top);
  BlockScratch& b = d->bs;
  if (!rc) rc = dev_alloc(d, &b.h, 16 * hs, "scratch");
  if (!rc) rc = dev_alloc(d, &b.x, 16 * hs, "scratch");
  if (!rc) rc = dev_alloc(d, &b.dsum_a, 16 * d->P, "scratch");
  if (!rc) rc = dev_alloc(d, &b.dsum_m, 16 * d->P, "scratch");
  if (!rc) rc = dev_alloc(d, &b.kb, 2 * 16 * d->kd, "scratch");
  if (!rc) rc = dev_alloc(d, &b.vb, 2 * 16 * d->kd, "scratch");
  if (!rc) rc = dev_alloc(d, &b.pacc, slots * 16 * d->hd, "attention partials");
  if (!rc) rc = dev_alloc(d, &b.pml, slots * 16 * 2, "attention partials");
  if (!rc) rc = dev_alloc(d, &d->part, d->part_floats, "GEMM partials");
  b.part = d->part;
  if (!rc) rc = dev_alloc(d, &b.logits, (size_t)16 * d->V, "logits");
  if (!rc) rc = dev_alloc(d, &b.hp, 16 * d->rank, "selector projection");
  if (!rc) rc = dev_alloc(d, &b.sel.gmax, (size_t)16 * ((d->V + 255) / 256), "selection");
  if (!rc) rc = dev_alloc(d, &b.sel.counters, 16, "selection");
  if (!rc) rc = dev_alloc(d, &b.sel.lv, 16 * sel_cap, "selection candidates");
  if (!rc) rc = dev_alloc(d, &b.sel.li, 16 * sel_cap, "selection candidates");
  // the block's activation operands, two planes each
  if (!rc) rc = dev_alloc(d, &b.xa, 2 * 16 * hs, "scratch");
  if (!rc) rc = dev_alloc(d, &b.xca, 2 * 16 * hs, "scratch");
  if (!rc) rc = dev_alloc(d, &b.qa, 2 * (size_t)d->nh * 16 * d->hd, "scratch");
  if (!rc) rc = dev_alloc(d, &b.ya, 2 * 16 * d->qd, "scratch");
  if (!rc) rc = dev_alloc(d, &b.ma, 2 * 16 * d->ffn, "scratch");
  d->stage_cols = std::max(std::max(d->tw, d->ffn), std::max(d->qd, hs));
  // the settle's operands, two planes of 256 rows each
  if (!rc) rc = dev_alloc(d, &d->taps_a, 2 * (size_t)kSettleRows * d->stage_cols, "settle scratch");
  if (!rc) rc = dev_alloc(d, &d->t_a, 2 * (size_t)kSettleRows * hs, "settle scratch");
  if (!rc)
    rc = dev_alloc(d, &d->sqp,
                   (size_t)std::max(kSettleRows * dfl::row_chunks(hs), 16 * dfl::conv1_chunks(hs)),
                   "norm scratch");
  b.sqp = d->sqp;
  if (!rc) rc = dev_alloc(d, &b.sel.tab, (size_t)d->top * (1 + 15 * d->top), "selector table");
  if (!rc) rc = dev_alloc(d, &b.sel.best, (size_t)(1 + 15 * d->top), "selector table");
  if (!rc)
    rc = dev_alloc(d, &d->rt_coef, (size_t)dfl::kRouteMaxRows * 2 * dfl::kRouteMaxRank,
                   "router scratch");
  if (!rc) rc = dev_alloc(d, &d->rt_nrm, (size_t)dfl::kRouteMaxRows * 2, "router scratch");
  if (!rc)
    rc = dev_alloc(d, &d->rt_part, (size_t)dfl::kRouteMaxRows * 2 * dfl::route_chunks(hs),
                   "router scratch");
  if (!rc) rc = hip_check(nullptr, hipDeviceSynchronize(), "create");
  if (!rc) rc = hip_check(nullptr, hipGetDevice(&d->dev), "create: current device");
  if (!rc) scratch_init(d->dev);
  return rc;
}

int dflash_create(const dflash_geometry* g, const dflash_weights* w, void* stream,
                  dflash_t** out) {
  if (!out) return fail(nullptr, DFLASH_EINVAL, "null output handle");
  *out = nullptr;
  g_create_error.clear();
  if (const char* why = validate(g, w)) return fail(nullptr, DFLASH_EINVAL, "geometry: %s", why);
  dflash* d = new dflash();
  d->hs = g->hidden;
  d->ffn = g->intermediate;
  d->L = g->layers;
  d->nh = g->heads;
  d->kv = g->kv_heads;
  d->hd = g->head_dim;
  d->V = g->vocab;
  d->B = g->block;
  d->mask = g->mask_token;
  d->gs = g->conv_group;
  d->kn = g->conv_kernel;
  d->rank = g->selector_rank;
  d->top = g->selector_top;
  d->ntaps = g->n_taps;
  d->tw = g->n_taps * g->hidden;
  d->qd = d->nh * d->hd;
  d->kd = d->kv * d->hd;
  d->G = d->hs / d->gs;
  d->P = 2 * d->kn * d->G;
  d->theta = g->rope_theta;
  d->eps = (float)g->eps;
  d->maxctx = g->max_context;
  d->st = static_cast<hipStream_t>(stream);
  d->windows.assign(g->windows, g->windows + d->L);
  for (int l = 0; l < d->L; ++l) d->rot.push_back(g->rotary[l] ? 1 : 0);
  d->ptiles = (d->P + 15) / 16;

  auto done = [&](int rc) {
    if (rc) {
      if (g_create_error.empty()) g_create_error = "create failed";
      dflash_destroy(d);
      return rc;
    }
    *out = d;
    return DFLASH_OK;
  };
  int rc = DFLASH_OK;
  const int hs = d->hs, L = d->L;
  // ---- dense f16 matrices, repacked
  {
    auto fc = repack_f16(w->fc, hs, d->tw);
    rc = upload(d, &d->fc, fc.data(), fc.size(), "fc");
  }
  if (!rc) {
    auto s = repack_f16(w->sel_proj, d->rank, hs);
    rc = upload(d, &d->sel, s.data(), s.size(), "selector projection");
  }
  if (!rc) {
    auto h = repack_f16(w->head, d->V, hs);
    rc = upload(d, &d->head, h.data(), h.size(), "head");
  }
  if (!rc) rc = upload(d, &d->embed, w->embed, (size_t)d->V * hs, "embedding");
  if (!rc) rc = upload(d, &d->pbook, w->pred_book, (size_t)d->V * d->rank, "predecessor codebook");
  if (!rc) rc = upload(d, &d->cbook, w->succ_book, (size_t)d->V * d->rank, "successor codebook");
  if (!rc) rc = upload(d, &d->hidden_norm, w->hidden_norm, hs, "hidden_norm");
  if (!rc) rc = upload(d, &d->norm, w->norm, hs, "norm");
  // ---- per-layer vectors and kernel projections, [layer][...]
  const size_t kp_layer = (size_t)d->ptiles * 16 * hs;
  if (!rc) rc = dev_alloc(d, &d->attn_kproj, L * kp_layer, "attention kernel projections");
  if (!rc) rc = dev_alloc(d, &d->mlp_kproj, L * kp_layer, "MLP kernel projections");
  std::vector<float> in_n, post_n, q_n, k_n, ab, mb;
  for (int l = 0; l < L && !rc; ++l) {
    const dflash_layer_w& x = w->layer[l];
    in_n.insert(in_n.end(), x.in_norm, x.in_norm + hs);
    post_n.insert(post_n.end(), x.post_norm, x.post_norm + hs);
    q_n.insert(q_n.end(), x.q_norm, x.q_norm + d->hd);
    k_n.insert(k_n.end(), x.k_norm, x.k_norm + d->hd);
    ab.insert(ab.end(), x.attn_base, x.attn_base + 2 * d->kn * hs);
    mb.insert(mb.end(), x.mlp_base, x.mlp_base + 2 * d->kn * hs);
    auto a = repack_f16(x.attn_kproj, d->P, hs);
    auto m = repack_f16(x.mlp_kproj, d->P, hs);
    if (hipMemcpy(d->attn_kproj + l * kp_layer, a.data(), a.size() * 2, hipMemcpyHostToDevice) ||
        hipMemcpy(d->mlp_kproj + l * kp_layer, m.data(), m.size() * 2, hipMemcpyHostToDevice))
      rc = fail(nullptr, DFLASH_EHIP, "copying kernel projections");
  }
  if (!rc) rc = upload(d, &d->in_norm, in_n.data(), in_n.size(), "input norms");
  if (!rc) rc = upload(d, &d->post_norm, post_n.data(), post_n.size(), "post-attention norms");
  if (!rc) rc = upload(d, &d->q_norm, q_n.data(), q_n.size(), "q norms");
  if (!rc) rc = upload(d, &d->k_norm, k_n.data(), k_n.size(), "k norms");
  if (!rc) rc = upload(d, &d->attn_base, ab.data(), ab.size(), "attention conv base");
  if (!rc) rc = upload(d, &d->mlp_base, mb.data(), mb.size(), "MLP conv base");
  // ---- int4 products: [q|k|v], o, [gate|up], down
  if (!rc) rc = alloc_i4(d, d->qkv, (d->qd + 2 * d->kd) / 16, hs, "q/k/v");
  if (!rc) rc = alloc_i4(d, d->o, hs / 16, d->qd, "o");
  if (!rc) rc = alloc_i4(d, d->gu, 2 * d->ffn / 16, hs, "gate/up");
  if (!rc) rc = alloc_i4(d, d->down, hs / 16, d->ffn, "down");
  for (int l = 0; l < L && !rc; ++l) {
    const dflash_layer_w& x = w->layer[l];
    rc = upload_i4(d, d->qkv, l, {{&x.q, d->qd}, {&x.k, d->kd}, {&x.v, d->kd}});
    if (!rc) rc = upload_i4(d, d->o, l, {{&x.o, hs}});
    if (!rc) rc = upload_i4(d, d->gu, l, {{&x.gate, d->ffn}, {&x.up, d->ffn}});
    if (!rc) rc = upload_i4(d, d->down, l, {{&x.down, hs}});
  }
  // ---- rotary frequencies: θ^(−2i/hd) in binary64, kept as binary32
  if (!rc) {
    std::vector<float> inv(d->hd / 2);
    for (int i = 0; i < d->hd / 2; ++i) inv[i] = (float)std::pow(d->theta, -(2.0 * i) / d->hd);
    rc = upload(d, &d->inv, inv.data(), inv.size(), "rotary frequencies");
  }
  if (!rc) rc = upload(d, &d->rot_dev, d->rot.data(), d->rot.size(), "rotary flags");
  // the weights are shared by every handle made from this one
  // (dflash_create_context): they move to their own owner
  if (!rc) {
    d->wown = std::make_shared<WeightOwner>();
    d->wown->allocs.swap(d->allocs);
  }
  if (!rc) rc = alloc_state(d);
  return done(rc);
}

int dflash_probe_peaks(dflash_t* d, int32_t reps, double* read_gbs, double* mfma_tfs) {
  if (!d) return DFLASH_EINVAL;
  if (reps < 1 || reps > 100 || !read_gbs || !mfma_tfs)
    return fail(d, DFLASH_EINVAL, "probe_peaks: reps must be in [1, 100], outputs non-null");
  hipStream_t st = d->st;
  // the sinks are written only on impossible values; any device word serves
  uint32_t* usink = reinterpret_cast<uint32_t*>(d->bs.sel.counters);
  float* fsink = reinterpret_cast<float*>(d->bs.sel.counters);
  const long bytes = (long)d->V * d->hs * 2 / 16 * 16;
  constexpr int kWgs = 512, kSteps = 4096;  // two waves on every SIMD
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = hip_check(d, hipEventCreate(&e0), "probe event");
  if (!rc) rc = hip_check(d, hipEventCreate(&e1), "probe event");
  float ms_read = 0.f, ms_mfma = 0.f;
  if (!rc) {
    dfl::probe_read(st, d->head, bytes, usink);  // warm
    (void)hipEventRecord(e0, st);
    for (int i = 0; i < reps; ++i) dfl::probe_read(st, d->head, bytes, usink);
    (void)hipEventRecord(e1, st);
    rc = hip_check(d, hipEventSynchronize(e1), "probe read");
    if (!rc) rc = hip_check(d, hipEventElapsedTime(&ms_read, e0, e1), "probe read time");
  }
  if (!rc) {
    dfl::probe_mfma(st, kWgs, kSteps, fsink);  // warm
    (void)hipEventRecord(e0, st);
    for (int i = 0; i < reps; ++i) dfl::probe_mfma(st, kWgs, kSteps, fsink);
    (void)hipEventRecord(e1, st);
    rc = hip_check(d, hipEventSynchronize(e1), "probe mfma");
    if (!rc) rc = hip_check(d, hipEventElapsedTime(&ms_mfma, e0, e1), "probe mfma time");
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (rc) return rc;
  *read_gbs = (double)bytes * reps / (ms_read * 1e-3) / 1e9;
  // 4 waves × 32 MFMAs of 16·16·32·2 flops per step
  *mfma_tfs = (double)kWgs * 4 * kSteps * 32 * 16384.0 * reps / (ms_mfma * 1e-3) / 1e12;
  return launch_check(d, "probe_peaks");
}

int dflash_set_timing(dflash_t* d, int on) {
  if (!d) return DFLASH_EINVAL;
  int rc = hip_check(d, hipStreamSynchronize(d->st), "set_timing");
  auto& t = d->tm;
  t.on = on != 0;
  t.used = 0;
  t.marks.clear();
  std::fill(t.us, t.us + DFLASH_STAGES, 0.0);
  std::fill(t.launches, t.launches + DFLASH_STAGES, 0);
  t.blocks = t.settles = 0;
  return rc;
}

int dflash_stage_times(const dflash_t* d, double* us, int64_t* launches, int64_t* blocks,
                       int64_t* settles) {
  if (!d) return DFLASH_EINVAL;
  for (int i = 0; i < DFLASH_STAGES; ++i) {
    if (us) us[i] = d->tm.us[i];
    if (launches) launches[i] = d->tm.launches[i];
  }
  if (blocks) *blocks = d->tm.blocks;
  if (settles) *settles = d->tm.settles;
  return DFLASH_OK;
}

int dflash_sync(dflash_t* d) {
  if (!d) return DFLASH_EINVAL;
  return hip_check(d, hipStreamSynchronize(d->st), "stream synchronize");
}

int dflash_span(const dflash_t* d, int64_t* first, int64_t* end) {
  if (!d || !first || !end) return DFLASH_EINVAL;
  *first = d->first;
  *end = d->first + d->len + d->pend;
  return DFLASH_OK;
}

int dflash_state(const dflash_t* d, int64_t* first, int64_t* settled, int64_t* waiting,
                 int64_t* dropped) {
  if (!d || !first || !settled || !waiting) return DFLASH_EINVAL;
  *first = d->first;
  *settled = d->len;
  *waiting = d->pend;
  if (dropped)
    for (int l = 0; l < d->L; ++l) dropped[l] = d->ls[l].dropped;
  return DFLASH_OK;
}

int dflash_truncate(dflash_t* d, int64_t pos) {
  if (!d) return DFLASH_EINVAL;
  CtxState s = state_of(d);
  truncate_state(s, std::max<int64_t>(pos, 0));
  commit(d, s);
  return DFLASH_OK;
}

int dflash_reserve(dflash_t* d, int64_t rows) {
  if (!d) return DFLASH_EINVAL;
  if (rows < 0) return fail(d, DFLASH_EINVAL, "reserve: rows must be >= 0");
  return reserve(d, rows);
}

// One settle pass of m ≤ 256 rows at positions pos0.. (store rows
// pos0 − first ..) of a settle call that ends at store row row_end.
static int settle_pass(dflash* d, const dfl::RowSrc& taps, int m, long pos0, long row_end) {
  hipStream_t st = d->st;
  const int mb = (m + 15) / 16;
  // every activation operand carries two f16 planes (hi and the rest): the
  // settled keys and values feed every later block, whose layers amplify
  // their error, so single-plane f16 rounding (1e-3 of the largest K/V
  // entry) is not enough end to end
  const long pst = (long)kSettleRows * d->tw, psh = (long)kSettleRows * d->hs;
  dfl::to_a(st, taps, m, d->tw, d->taps_a, pst);
  tm_mark(d, DFLASH_ST_S_TAPS);
  // t = fc · taps (f32 partials), then rms by hidden_norm into A-layout
  const dfl::TileMap fmap{d->hs / 16, d->hs / 16, 0, 0};
  // one 16-row block (the stream's few-row settles): the block pass's
  // 16-row kernels, every weight load of a workgroup issued at once
  const Split sf = mb > 1 ? split_big(d->hs / 16, d->tw / 32)
                          : Split{dfl::f16_block_splits(d->tw), 0};
  const long ssf = (long)mb * 16 * d->hs;
  if (mb > 1)
    dfl::gemm_big_f16(st, d->taps_a, pst, d->tw, mb, d->fc, fmap, d->hs, sf.S, sf.per, d->part,
                      ssf);
  else
    dfl::gemm_f16_block(st, d->taps_a, pst, d->tw, d->fc, fmap, d->hs, d->part, ssf);
  tm_mark(d, DFLASH_ST_S_FC);
  // the hidden norm folded: t ⊙ hidden_norm feeds the K/V projection, and
  // settle_kv applies each row's rms scale to its output
  dfl::rowsum_sq(st, d->part, sf.S, ssf, m, d->hs, d->hidden_norm, d->t_a, psh, d->sqp);
  tm_mark(d, DFLASH_ST_S_NORM);
  // K and V of every layer: the k and v tiles of each layer's q/k/v set
  const int kvt = 2 * d->kd / 16;
  const int N = d->L * 2 * d->kd;
  const long ssk = (long)mb * 16 * N;
  const dfl::TileMap map{d->L * kvt, kvt, d->qkv.tiles, d->qd / 16};
  Split sk;
  if (mb > kSettleI4Blocks) {
    sk = split_kv(d->L * kvt, d->hs / 128);
    dfl::gemm_kv_i4(st, d->t_a, psh, d->hs, mb, d->qkv.codes, d->qkv.scales, map, N, sk.S, sk.per,
                    d->part, ssk);
  } else if (mb > 1) {
    sk = split_for(d->L * kvt, kR, d->hs / 128, mb, 4);
    dfl::gemm_i4(st, d->t_a, psh, d->hs, mb, d->qkv.codes, d->qkv.scales, map, N, sk.S, sk.per,
                 d->part, ssk);
  } else {
    sk = {dfl::i4_block_splits(d->hs, kKsQkv), 0};
    dfl::gemm_i4_block(st, d->t_a, psh, d->hs, d->qkv.codes, d->qkv.scales, map, N, 2, kKsQkv,
                       d->part, ssk);
  }
  tm_mark(d, DFLASH_ST_S_KV);
  dfl::settle_kv(st, d->part, sk.S, ssk, m, d->L, d->kv, d->hd, d->k_norm, d->inv, d->rot_dev,
                 pos0, d->eps, d->sqp, d->hs, d->tab, pos0 - d->first,
                 row_end);
  tm_mark(d, DFLASH_ST_S_STORE);
  return launch_check(d, "settle");
}

// One `settle_rows` call: the rows at positions first+len.., 256 a pass,
// then the window drop.
static int settle_call(dflash* d, const Runs& r) {
  const long n = r.n[0] + r.n[1] + r.n[2];
  if (n == 0) return DFLASH_OK;
  tm_begin(d);
  for (long done = 0; done < n; done += kSettleRows) {
    const int m = (int)std::min<long>(kSettleRows, n - done);
    // this pass's rows, as runs of r
    const float* p[3] = {nullptr, nullptr, nullptr};
    long c[3] = {0, 0, 0};
    int k = 0;
    long skip = done, need = m;
    for (int i = 0; i < r.k && need > 0; ++i) {
      if (skip >= r.n[i]) {
        skip -= r.n[i];
        continue;
      }
      const long take = std::min(r.n[i] - skip, need);
      p[k] = r.p[i] + (size_t)skip * d->tw;
      c[k++] = take;
      need -= take;
      skip = 0;
    }
    const dfl::RowSrc src{{p[0], k > 1 ? p[1] : p[0], k > 2 ? p[2] : p[0]}, (int)c[0], (int)c[1],
                          (long)d->tw};
    const int rc = settle_pass(d, src, m, d->first + d->len + done, d->len + n);
    if (rc) {
      lose_context(d);
      return rc;
    }
  }
  tm_end(d);
  d->tm.settles += d->tm.on;
  CtxState s = state_of(d);
  settle_state(d, s, n);
  commit(d, s);
  return DFLASH_OK;
}

// `queue_context` (all = false: the rows past the waiting limit settle, the
// rest wait) and `push_context` (all = true: every row settles).
static int push_rows(dflash* d, int64_t pos, int32_t n, const float* taps, bool all,
                     const char* what) {
  if (n < 0 || pos < 0) return fail(d, DFLASH_EINVAL, "%s: n and first_pos must be >= 0", what);
  if (n > 0 && !taps) return fail(d, DFLASH_EINVAL, "%s: null taps", what);
  CtxState s = state_of(d);
  position_rule(s, pos);
  const long total = s.pend + n;
  const long over =
      total > d->pcap
          ? std::min((total - d->pcap + kContextChunk - 1) / kContextChunk * kContextChunk, total)
          : 0;
  // what the layers hold after the calls this makes (for a queue, also after
  // the later settle of what waits) must fit them
  CtxState t = s;
  if ((over && !settle_state(d, t, over)) || (total > over && !settle_state(d, t, total - over)))
    return fail(d, DFLASH_ENOMEM,
                "%s: the context would hold more rows than a layer's store (max_context %ld)", what,
                d->maxctx);
  if (int rc = reserve(d, t.len)) return rc;
  commit(d, s);
  long used = 0;  // caller rows settled so far
  if (over) {
    Runs r;
    const long a = std::min(over, d->pend);
    add_waiting(d, r, 0, a);
    r.add(taps, over - a);
    d->phead = (d->phead + a) % d->pcap;
    d->pend -= a;
    used = over - a;
    if (int rc = settle_call(d, r)) return rc;
  }
  if (all) {
    Runs r;
    add_waiting(d, r, 0, d->pend);
    r.add(taps + (size_t)used * d->tw, n - used);
    d->pend = 0;
    d->phead = 0;
    return settle_call(d, r);
  }
  // the caller's other rows wait: into the ring after the waiting ones
  long left = n - used;
  const float* src = taps + (size_t)used * d->tw;
  while (left > 0) {
    const long i = (d->phead + d->pend) % d->pcap, c = std::min(left, d->pcap - i);
    const int rc = hip_check(d,
                             hipMemcpyAsync(d->pq + (size_t)i * d->tw, src, (size_t)c * d->tw * 4,
                                            hipMemcpyDeviceToDevice, d->st),
                             what);
    if (rc) {
      lose_context(d);
      return rc;
    }
    d->pend += c;
    src += (size_t)c * d->tw;
    left -= c;
  }
  return DFLASH_OK;
}

int dflash_settle(dflash_t* d, int64_t first_pos, int32_t n, const float* taps) {
  if (!d) return DFLASH_EINVAL;
  return push_rows(d, first_pos, n, taps, true, "settle");
}

int dflash_queue(dflash_t* d, int64_t first_pos, int32_t n, const float* taps) {
  if (!d) return DFLASH_EINVAL;
  return push_rows(d, first_pos, n, taps, false, "queue");
}

int dflash_flush(dflash_t* d) {
  if (!d) return DFLASH_EINVAL;
  if (d->pend == 0) return DFLASH_OK;
  CtxState t = state_of(d);
  if (!settle_state(d, t, d->pend))
    return fail(d, DFLASH_ENOMEM, "flush: the context would not fit a layer's store");
  if (int rc = reserve(d, t.len)) return rc;
  Runs r;
  add_waiting(d, r, 0, d->pend);
  d->pend = 0;
  d->phead = 0;
  return settle_call(d, r);
}

// Argument checks shared by the block entry points.
static int block_args(dflash* d, int32_t anchor, int64_t a, int32_t k, int32_t width,
                      const int32_t* cand, const float* unary, const float* score,
                      const int32_t* chosen) {
  if (k < 1 || k >= d->B) return fail(d, DFLASH_EINVAL, "block: k must be in [1, block)");
  if (width < d->top || width > d->V)
    return fail(d, DFLASH_EINVAL, "block: width must be in [selector_top, vocab]");
  if (anchor < 0 || anchor >= d->V) return fail(d, DFLASH_EINVAL, "block: anchor outside the vocabulary");
  if (a < 0) return fail(d, DFLASH_EINVAL, "block: a must be >= 0");
  if (!cand || !unary || !score || !chosen) return fail(d, DFLASH_EINVAL, "block: null output");
  if (d->pend)
    return fail(d, DFLASH_EINVAL, "block: %ld rows wait to become context (dflash_flush first)",
                d->pend);
  return DFLASH_OK;
}

// The block pass on the scratch set b (arguments already checked).
static int block_pass(dflash* d, const BlockScratch& b, int32_t anchor, int64_t a, int32_t k,
                      int32_t width, float* logits, int32_t* cand, float* unary, float* score,
                      int32_t* chosen) {
  hipStream_t st = d->st;
  const int hs = d->hs, B = d->B;
  const float scale = std::pow((float)d->hd, -0.5f);
  const long ssd = 16L * d->P, ssq = 16L * (d->qd + 2 * d->kd), ssh = 16L * hs;
  const Split spk = {dfl::f16_block_splits(hs), 0};
  const Split sqk = {dfl::i4_block_splits(hs, kKsQkv), kKsQkv};
  const Split so = {dfl::i4_block_splits(d->qd, kKsO), kKsO};
  const Split sdn = {dfl::i4_block_splits(d->ffn, kKsDown), kKsDown};
  const size_t kp_layer = (size_t)d->ptiles * 16 * hs;
  const size_t i4l_qkv = (size_t)d->qkv.tiles * (hs / 128);
  const size_t i4l_o = (size_t)d->o.tiles * (d->qd / 128);
  const size_t i4l_gu = (size_t)d->gu.tiles * (hs / 128);
  const size_t i4l_dn = (size_t)d->down.tiles * (d->ffn / 128);
  // plane strides (halves) of the two-plane operands
  const int nc1 = dfl::conv1_chunks(hs);  // sums of squares per row after conv1
  const long psh = 16L * hs, psq = 16L * d->nh * d->hd, psy = 16L * d->qd, psm = 16L * d->ffn;

  tm_begin(d);
  // Each sub-layer's rms is folded into its neighbours: the producer of h
  // (embed, conv1) writes h, its partial sums of squares and h ⊙ gain as the
  // kernel projection's input; conv0 applies the per-row scale.
  const int anchors[1] = {anchor};
  const long apos[1] = {(long)a};
  dfl::embed(st, d->embed, anchors, 1, d->mask, B, hs, b.h, b.sqp, d->in_norm, b.xa, psh);
  tm_mark(d, DFLASH_ST_CONV);
  int nch = dfl::row_chunks(hs);  // sums of squares per row: embed's, then conv1's
  for (int l = 0; l < d->L; ++l) {
    const float* ab = d->attn_base + (size_t)l * 2 * d->kn * hs;
    const float* mbase = d->mlp_base + (size_t)l * 2 * d->kn * hs;
    const float* post = d->post_norm + (size_t)l * hs;
    // attention: conv_in, q/k/v, norms + rotary
    dfl::gemm_f16_block(st, b.xa, psh, hs, d->attn_kproj + l * kp_layer,
                        dfl::TileMap{d->ptiles, d->ptiles, 0, 0}, d->P, b.part, ssd);
    tm_mark(d, DFLASH_ST_KPROJ);
    dfl::conv0(st, b.h, b.sqp, nch, d->in_norm + (size_t)l * hs, d->eps, b.part, spk.S, ssd, ab,
               B, hs, d->gs, d->kn, b.xca, psh, b.dsum_a);
    tm_mark(d, DFLASH_ST_CONV);
    dfl::gemm_i4_block(st, b.xca, psh, hs, d->qkv.codes + i4l_qkv * 1024 * l,
                       d->qkv.scales + i4l_qkv * 64 * l,
                       dfl::TileMap{d->qkv.tiles, d->qkv.tiles, 0, 0}, d->qd + 2 * d->kd, kRQkv,
                       sqk.per, b.part, ssq);
    tm_mark(d, DFLASH_ST_QKV);
    dfl::qkv_post(st, b.part, sqk.S, ssq, B, d->nh, d->kv, d->hd, d->q_norm + (size_t)l * d->hd,
                  d->k_norm + (size_t)l * d->hd, d->inv, apos, 1, d->rot[l], d->eps, b.qa, psq,
                  b.kb, b.vb);
    tm_mark(d, DFLASH_ST_QKPOST);
    // attention over the layer's context range and the block's rows
    long lo, n;
    layer_range(d, l, a, &lo, &n);
    int nchunks = 0;
    const int chunk = attn_chunk(n, &nchunks);
    const auto& S = d->ls[l];
    dfl::AttnSeqs as{};
    as.s[0] = {S.k, S.v, S.cap, S.cap ? (lo - d->first) % S.cap : 0, lo, (long)a, (int)n, chunk,
               nchunks};
    dfl::attention(st, b.qa, psq, as, 1, b.kb, b.vb, B, d->nh, d->kv, d->hd, d->windows[l], scale,
                   b.pacc, b.pml);
    tm_mark(d, DFLASH_ST_ATTN);
    dfl::attn_merge(st, b.pacc, b.pml, d->nh, d->kv, d->hd, as, 1, B, b.ya, psy);
    tm_mark(d, DFLASH_ST_ATTN);
    // o, conv_out into the residual (and the MLP norm's input)
    dfl::gemm_i4_block(st, b.ya, psy, d->qd, d->o.codes + i4l_o * 1024 * l,
                       d->o.scales + i4l_o * 64 * l, dfl::TileMap{d->o.tiles, d->o.tiles, 0, 0},
                       hs, kRO, so.per, b.part, ssh);
    tm_mark(d, DFLASH_ST_O);
    dfl::conv1(st, b.h, b.part, so.S, ssh, b.dsum_a, ab, B, hs, d->gs, d->kn, b.sqp, post,
               b.xa, psh);
    nch = nc1;
    tm_mark(d, DFLASH_ST_CONV);
    // MLP, wrapped the same way
    dfl::gemm_f16_block(st, b.xa, psh, hs, d->mlp_kproj + l * kp_layer,
                        dfl::TileMap{d->ptiles, d->ptiles, 0, 0}, d->P, b.part, ssd);
    tm_mark(d, DFLASH_ST_KPROJ);
    dfl::conv0(st, b.h, b.sqp, nch, post, d->eps, b.part, spk.S, ssd, mbase, B, hs, d->gs, d->kn,
               b.xca, psh, b.dsum_m);
    tm_mark(d, DFLASH_ST_CONV);
    dfl::gemm_glu_stream(st, b.xca, psh, hs, d->gu.codes + i4l_gu * 1024 * l,
                         d->gu.scales + i4l_gu * 64 * l, d->ffn / 16, b.ma, psm);
    tm_mark(d, DFLASH_ST_GLU);
    dfl::gemm_i4_block(st, b.ma, psm, d->ffn, d->down.codes + i4l_dn * 1024 * l,
                       d->down.scales + i4l_dn * 64 * l,
                       dfl::TileMap{d->down.tiles, d->down.tiles, 0, 0}, hs, kRDown, sdn.per, b.part,
                       ssh);
    tm_mark(d, DFLASH_ST_DOWN);
    // conv_out into the residual, and the next layer's attention-norm input
    // (the final norm runs on its own below)
    const float* next = l + 1 < d->L ? d->in_norm + (size_t)(l + 1) * hs : nullptr;
    dfl::conv1(st, b.h, b.part, sdn.S, ssh, b.dsum_m, mbase, B, hs, d->gs, d->kn, b.sqp, next,
               b.xa, psh);
    tm_mark(d, DFLASH_ST_CONV);
    if (d->trace)
      (void)hipMemcpyAsync(d->trace + (size_t)l * B * hs, b.h, sizeof(float) * B * hs,
                           hipMemcpyDeviceToDevice, st);
  }
  // the final norm (the head's input), then the head over rows 1..k and
  // the selector projection
  dfl::norm_apply(st, b.h, b.sqp, nc1, B, hs, d->norm, d->eps, b.x, b.xa, psh);
  tm_mark(d, DFLASH_ST_CONV);
  float* lg = logits ? logits : b.logits;
  dfl::head_sel(st, b.xa, psh, hs, d->head, width, k, lg, d->sel, d->rank, b.hp, b.sel);
  tm_mark(d, DFLASH_ST_HEAD);
  dfl::select_all(st, lg, true, k, width, d->top, b.hp + d->rank, d->rank, d->pbook, d->cbook,
                  d->V, anchor, nullptr, b.sel, cand, unary, score, chosen);
  tm_mark(d, DFLASH_ST_SELECT);
  const int rc = launch_check(d, "block");
  tm_end(d);
  d->tm.blocks += d->tm.on;
  return rc;
}

int dflash_block(dflash_t* d, int32_t anchor, int64_t a, int32_t k, int32_t width, float* logits,
                 int32_t* cand, float* unary, float* score, int32_t* chosen) {
  if (!d) return DFLASH_EINVAL;
  if (int rc = block_args(d, anchor, a, k, width, cand, unary, score, chosen)) return rc;
  const int rc = block_pass(d, d->bs, anchor, a, k, width, logits, cand, unary, score, chosen);
  d->last_k = k;
  return rc;
}

int dflash_block_noalloc(dflash_t* d, int32_t anchor, int64_t a, int32_t k, int32_t width,
                         float* logits, int32_t* cand, float* unary, float* score,
                         int32_t* chosen) {
  if (!d) return DFLASH_EINVAL;
  if (int rc = block_args(d, anchor, a, k, width, cand, unary, score, chosen)) return rc;
  if (!logits) return fail(d, DFLASH_EINVAL, "block_noalloc: logits must be a caller buffer");
  const size_t need = carve_block_scratch(d, nullptr, nullptr);
  if (need > kNoallocScratchBytes)
    return fail(d, DFLASH_EINVAL,
                "block_noalloc: this geometry needs %zu bytes of scratch, more than the %zu the "
                "library holds",
                need, kNoallocScratchBytes);
  void* base = scratch_ptr(d->dev);
  if (!base)
    return fail(d, DFLASH_EHIP, "block_noalloc: the static scratch of device %d is unavailable",
                d->dev);
  BlockScratch b;
  carve_block_scratch(d, static_cast<uint8_t*>(base), &b);
  return block_pass(d, b, anchor, a, k, width, logits, cand, unary, score, chosen);
}

// ------------------------------------------------------- batched blocks

int dflash_create_context(const dflash_t* model, int64_t max_context, void* stream,
                          dflash_t** out) {
  if (!out) return fail(nullptr, DFLASH_EINVAL, "null output handle");
  *out = nullptr;
  g_create_error.clear();
  if (!model) return fail(nullptr, DFLASH_EINVAL, "create_context: null model handle");
  if (max_context < 1) return fail(nullptr, DFLASH_EINVAL, "create_context: max_context must be >= 1");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != model->dev)
    return fail(nullptr, DFLASH_EINVAL, "create_context: the model's device (%d) must be current",
                model->dev);
  // the geometry and the weights (shared), then a state of its own
  dflash* d = new dflash(*model);
  d->allocs.clear();
  d->ls.clear();
  d->tab = nullptr;
  d->pq = nullptr;
  d->pcap = d->phead = d->pend = 0;
  d->first = d->len = 0;
  d->bs = BlockScratch{};
  d->part = d->sqp = nullptr;
  d->taps_a = d->t_a = nullptr;
  d->part_floats = 0;
  d->stage_cols = 0;
  d->last_k = 0;
  d->trace = nullptr;
  d->bb = BatchScratch{};
  d->order = nullptr;
  d->err.clear();
  d->tm = dflash::Timing{};
  d->st = static_cast<hipStream_t>(stream);
  d->maxctx = max_context;
  const int rc = alloc_state(d);
  if (rc) {
    if (g_create_error.empty()) g_create_error = "create_context failed";
    dflash_destroy(d);
    return rc;
  }
  *out = d;
  return DFLASH_OK;
}

// The lead handle's batch scratch, for up to dfl::kMaxSeq sequences.
static int batch_scratch(dflash* d) {
  BatchScratch& b = d->bb;
  if (b.ready) return DFLASH_OK;
  const size_t R = 16 * dfl::kMaxSeq, hs = d->hs;
  const size_t slots = (size_t)dfl::kMaxSeq * d->nh * (dfl::kAttnMaxChunks + 1);
  // the largest split partial of any batched product
  // (a pass of B sequences runs MB = 4 or 8 row blocks, 16·MB rows, with the
  // splits split_mb gives at that MB)
  long part = 0;
  auto f16p = [&](int N, int K) {
    for (int MB : {4, 8})
      part = std::max(part, (long)split_mb((N + 15) / 16, K / 32, MB).S * 16 * MB * N);
  };
  auto i4p = [&](int N, int K) {
    for (int MB : {4, 8})
      part = std::max(part, (long)split_mb(N / 16, K / 128, MB).S * 16 * MB * N);
  };
  f16p(d->P, d->hs);
  f16p(d->rank, d->hs);
  i4p(d->qd + 2 * d->kd, d->hs);
  i4p(d->hs, d->qd);
  i4p(2 * d->ffn, d->hs);
  i4p(d->hs, d->ffn);
  b.part_floats = part;
  const size_t sel_cap = (size_t)dfl::topk_cap(d->V, d->top);
  int rc = DFLASH_OK;
  auto take = [&](auto** p, size_t count, const char* what) {
    if (!rc) rc = dev_alloc(d, p, count, what);
  };
  take(&b.h, R * hs, "batch scratch");
  take(&b.sqp, R * (size_t)std::max(dfl::row_chunks(d->hs), dfl::conv1_chunks(d->hs)), "batch scratch");
  take(&b.dsum_a, R * d->P, "batch scratch");
  take(&b.dsum_m, R * d->P, "batch scratch");
  take(&b.kb, 2 * R * d->kd, "batch scratch");
  take(&b.vb, 2 * R * d->kd, "batch scratch");
  take(&b.pacc, slots * 16 * d->hd, "batch attention partials");
  take(&b.pml, slots * 16 * 2, "batch attention partials");
  take(&b.part, (size_t)part, "batch partials");
  take(&b.logits, R * d->V, "batch logits");
  take(&b.hp, R * d->rank, "batch selector projection");
  take(&b.xa, 2 * R * hs, "batch scratch");
  take(&b.xca, 2 * R * hs, "batch scratch");
  take(&b.qa, 2 * R * d->qd, "batch scratch");
  take(&b.ya, 2 * R * d->qd, "batch scratch");
  take(&b.ma, 2 * R * d->ffn, "batch scratch");
  const size_t S = dfl::kMaxSeq;
  take(&b.sel.gmax, S * 16 * ((d->V + 255) / 256), "batch selection");
  take(&b.sel.counters, S * 16, "batch selection");
  take(&b.sel.lv, S * 16 * sel_cap, "batch selection");
  take(&b.sel.li, S * 16 * sel_cap, "batch selection");
  take(&b.sel.tab, S * d->top * (1 + 15 * d->top), "batch selection");
  take(&b.sel.best, S * (1 + 15 * d->top), "batch selection");
  if (rc) return fail(d, rc, "block_batch: %s", g_create_error.c_str());
  b.ready = true;
  return DFLASH_OK;
}

// The batched pass on the lead's stream and scratch (arguments checked).
static int block_batch_pass(dflash* const* ds, int nseq, const int32_t* anchors,
                            const int64_t* apos, int32_t k, int32_t width, float* logits,
                            int32_t* cand, float* unary, float* score, int32_t* chosen) {
  dflash* d = ds[0];
  BatchScratch& b = d->bb;
  hipStream_t st = d->st;
  const int MB = nseq <= 4 ? 4 : 8, R = 16 * MB;
  const int hs = d->hs, B = d->B;
  const float scale = std::pow((float)d->hd, -0.5f);
  const long psh = (long)R * hs, psq = (long)R * d->qd, psm = (long)R * d->ffn;
  const size_t kp_layer = (size_t)d->ptiles * 16 * hs;
  const size_t i4l_qkv = (size_t)d->qkv.tiles * (hs / 128);
  const size_t i4l_o = (size_t)d->o.tiles * (d->qd / 128);
  const size_t i4l_gu = (size_t)d->gu.tiles * (hs / 128);
  const size_t i4l_dn = (size_t)d->down.tiles * (d->ffn / 128);
  const int nc1 = dfl::conv1_chunks(hs);
  int anc[dfl::kMaxSeq];
  long pos[dfl::kMaxSeq];
  for (int s = 0; s < nseq; ++s) {
    anc[s] = anchors[s];
    pos[s] = (long)apos[s];
  }
  const Split skp = split_mb(d->ptiles, hs / 32, MB);
  const Split sqk = split_mb(d->qkv.tiles, hs / 128, MB);
  const Split so = split_mb(d->o.tiles, d->qd / 128, MB);
  const Split sgu = split_mb(d->gu.tiles, hs / 128, MB);
  const Split sdn = split_mb(d->down.tiles, d->ffn / 128, MB);
  const long ssd = (long)R * d->P, ssq = (long)R * (d->qd + 2 * d->kd), ssh = (long)R * hs,
             ssg = (long)R * 2 * d->ffn;
  const dfl::TileMap kpmap{d->ptiles, d->ptiles, 0, 0};

  tm_begin(d);
  dfl::embed(st, d->embed, anc, nseq, d->mask, B, hs, b.h, b.sqp, d->in_norm, b.xa, psh);
  tm_mark(d, DFLASH_ST_CONV);
  int nch = dfl::row_chunks(hs);
  for (int l = 0; l < d->L; ++l) {
    const float* ab = d->attn_base + (size_t)l * 2 * d->kn * hs;
    const float* mbase = d->mlp_base + (size_t)l * 2 * d->kn * hs;
    const float* post = d->post_norm + (size_t)l * hs;
    dfl::gemm_mb_f16(st, b.xa, psh, hs, MB, nseq, d->attn_kproj + l * kp_layer, kpmap, d->P,
                     skp.S, skp.per, b.part, ssd);
    tm_mark(d, DFLASH_ST_KPROJ);
    dfl::conv0(st, b.h, b.sqp, nch, d->in_norm + (size_t)l * hs, d->eps, b.part, skp.S, ssd, ab, B,
               hs, d->gs, d->kn, b.xca, psh, b.dsum_a, nseq);
    tm_mark(d, DFLASH_ST_CONV);
    dfl::gemm_mb_i4(st, b.xca, psh, hs, MB, nseq, d->qkv.codes + i4l_qkv * 1024 * l,
                    d->qkv.scales + i4l_qkv * 64 * l,
                    dfl::TileMap{d->qkv.tiles, d->qkv.tiles, 0, 0}, d->qd + 2 * d->kd, sqk.S,
                    sqk.per, b.part, ssq);
    tm_mark(d, DFLASH_ST_QKV);
    dfl::qkv_post(st, b.part, sqk.S, ssq, B, d->nh, d->kv, d->hd, d->q_norm + (size_t)l * d->hd,
                  d->k_norm + (size_t)l * d->hd, d->inv, pos, nseq, d->rot[l], d->eps, b.qa, psq,
                  b.kb, b.vb);
    tm_mark(d, DFLASH_ST_QKPOST);
    // each sequence's own context range of this layer, in its own store
    dfl::AttnSeqs as{};
    for (int s = 0; s < nseq; ++s) {
      const dflash* e = ds[s];
      long lo, n;
      layer_range(e, l, pos[s], &lo, &n);
      int nchunks = 0;
      const int chunk = attn_chunk(n, &nchunks);
      const auto& S = e->ls[l];
      as.s[s] = {S.k, S.v, S.cap, S.cap ? (lo - e->first) % S.cap : 0, lo, pos[s], (int)n, chunk,
                 nchunks};
    }
    dfl::attention(st, b.qa, psq, as, nseq, b.kb, b.vb, B, d->nh, d->kv, d->hd, d->windows[l],
                   scale, b.pacc, b.pml);
    dfl::attn_merge(st, b.pacc, b.pml, d->nh, d->kv, d->hd, as, nseq, B, b.ya, psq);
    tm_mark(d, DFLASH_ST_ATTN);
    dfl::gemm_mb_i4(st, b.ya, psq, d->qd, MB, nseq, d->o.codes + i4l_o * 1024 * l,
                    d->o.scales + i4l_o * 64 * l, dfl::TileMap{d->o.tiles, d->o.tiles, 0, 0}, hs,
                    so.S, so.per, b.part, ssh);
    tm_mark(d, DFLASH_ST_O);
    dfl::conv1(st, b.h, b.part, so.S, ssh, b.dsum_a, ab, B, hs, d->gs, d->kn, b.sqp, post, b.xa,
               psh, nseq);
    nch = nc1;
    tm_mark(d, DFLASH_ST_CONV);
    dfl::gemm_mb_f16(st, b.xa, psh, hs, MB, nseq, d->mlp_kproj + l * kp_layer, kpmap, d->P, skp.S,
                     skp.per, b.part, ssd);
    tm_mark(d, DFLASH_ST_KPROJ);
    dfl::conv0(st, b.h, b.sqp, nch, post, d->eps, b.part, skp.S, ssd, mbase, B, hs, d->gs, d->kn,
               b.xca, psh, b.dsum_m, nseq);
    tm_mark(d, DFLASH_ST_CONV);
    dfl::gemm_mb_i4(st, b.xca, psh, hs, MB, nseq, d->gu.codes + i4l_gu * 1024 * l,
                    d->gu.scales + i4l_gu * 64 * l, dfl::TileMap{d->gu.tiles, d->gu.tiles, 0, 0},
                    2 * d->ffn, sgu.S, sgu.per, b.part, ssg);
    dfl::glu_act(st, b.part, sgu.S, ssg, B, nseq, d->ffn, b.ma, psm);
    tm_mark(d, DFLASH_ST_GLU);
    dfl::gemm_mb_i4(st, b.ma, psm, d->ffn, MB, nseq, d->down.codes + i4l_dn * 1024 * l,
                    d->down.scales + i4l_dn * 64 * l,
                    dfl::TileMap{d->down.tiles, d->down.tiles, 0, 0}, hs, sdn.S, sdn.per, b.part,
                    ssh);
    tm_mark(d, DFLASH_ST_DOWN);
    const float* next = l + 1 < d->L ? d->in_norm + (size_t)(l + 1) * hs : nullptr;
    dfl::conv1(st, b.h, b.part, sdn.S, ssh, b.dsum_m, mbase, B, hs, d->gs, d->kn, b.sqp, next,
               b.xa, psh, nseq);
    tm_mark(d, DFLASH_ST_CONV);
  }
  dfl::norm_apply(st, b.h, b.sqp, nc1, B, hs, d->norm, d->eps, nullptr, b.xa, psh, nseq);
  tm_mark(d, DFLASH_ST_CONV);
  // the head over every row of every block, then the selector projection
  const int wtiles = (width + 15) / 16, stiles = (d->rank + 15) / 16;
  dfl::gemm_mb_f16(st, b.xa, psh, hs, MB, nseq, d->head, dfl::TileMap{wtiles, wtiles, 0, 0}, width,
                   1, hs / 32, b.logits, (long)R * width);
  const Split ssel = split_mb(stiles, hs / 32, MB);
  dfl::gemm_mb_f16(st, b.xa, psh, hs, MB, nseq, d->sel, dfl::TileMap{stiles, stiles, 0, 0},
                   d->rank, ssel.S, ssel.per, b.part, (long)R * d->rank);
  dfl::sum_rows(st, b.part, ssel.S, (long)R * d->rank, R, d->rank, b.hp);
  tm_mark(d, DFLASH_ST_HEAD);
  // every sequence's selection on its rows 1..k, in one set of launches
  dfl::select_batch(st, nseq, b.logits + width, 16L * width, false, k, width, d->top,
                    b.hp + d->rank, 16L * d->rank, d->rank, d->pbook, d->cbook, d->V, anc,
                    nullptr, b.sel, cand, unary, score, chosen);
  if (logits)
    (void)hipMemcpy2DAsync(logits, sizeof(float) * k * width, b.logits + width,
                           sizeof(float) * 16 * width, sizeof(float) * k * width, nseq,
                           hipMemcpyDeviceToDevice, st);
  tm_mark(d, DFLASH_ST_SELECT);
  const int rc = launch_check(d, "block_batch");
  tm_end(d);
  d->tm.blocks += d->tm.on;
  return rc;
}

int dflash_block_batch(dflash_t* const* ds, int32_t nseq, const int32_t* anchors,
                       const int64_t* a, int32_t k, int32_t width, float* logits, int32_t* cand,
                       float* unary, float* score, int32_t* chosen) {
  if (!ds || !ds[0]) return DFLASH_EINVAL;
  dflash* d = ds[0];
  if (nseq < 1 || nseq > dfl::kMaxSeq)
    return fail(d, DFLASH_EINVAL, "block_batch: nseq must be in [1, %d]", dfl::kMaxSeq);
  if (!anchors || !a) return fail(d, DFLASH_EINVAL, "block_batch: null anchors or positions");
  if (int rc = block_args(d, anchors[0], a[0], k, width, cand, unary, score, chosen)) return rc;
  for (int s = 1; s < nseq; ++s) {
    const dflash* e = ds[s];
    if (!e) return fail(d, DFLASH_EINVAL, "block_batch: null handle %d", s);
    if (e->wown != d->wown)
      return fail(d, DFLASH_EINVAL, "block_batch: handle %d does not share the lead's weights", s);
    if (e->pend)
      return fail(d, DFLASH_EINVAL, "block_batch: handle %d has rows waiting (dflash_flush first)",
                  s);
    if (anchors[s] < 0 || anchors[s] >= d->V)
      return fail(d, DFLASH_EINVAL, "block_batch: anchor %d outside the vocabulary", s);
    if (a[s] < 0) return fail(d, DFLASH_EINVAL, "block_batch: a must be >= 0");
  }
  if (int rc = batch_scratch(d)) return rc;
  // the other handles' streams: the batch waits for what they enqueued,
  // and they wait for the batch
  for (int s = 1; s < nseq; ++s) {
    dflash* e = ds[s];
    if (e->st == d->st) continue;
    if (!e->order && hip_check(e, hipEventCreateWithFlags(&e->order, hipEventDisableTiming),
                               "block_batch: event"))
      return fail(d, DFLASH_EHIP, "block_batch: %s", e->err.c_str());
    if (hipEventRecord(e->order, e->st) != hipSuccess ||
        hipStreamWaitEvent(d->st, e->order, 0) != hipSuccess)
      return fail(d, DFLASH_EHIP, "block_batch: ordering against handle %d's stream", s);
  }
  const int rc = block_batch_pass(ds, nseq, anchors, a, k, width, logits, cand, unary, score,
                                  chosen);
  if (rc) return rc;
  if (!d->order && hip_check(d, hipEventCreateWithFlags(&d->order, hipEventDisableTiming),
                             "block_batch: event"))
    return DFLASH_EHIP;
  if (hipEventRecord(d->order, d->st) != hipSuccess)
    return fail(d, DFLASH_EHIP, "block_batch: recording the batch's end");
  for (int s = 1; s < nseq; ++s)
    if (ds[s]->st != d->st && hipStreamWaitEvent(ds[s]->st, d->order, 0) != hipSuccess)
      return fail(d, DFLASH_EHIP, "block_batch: ordering handle %d's stream after the batch", s);
  return DFLASH_OK;
}

int dflash_route_margin(dflash_t* d, const float* rows, int32_t m, const uint16_t* block_mean,
                        const uint16_t* block_basis, int32_t block_rank,
                        const uint16_t* chain_mean, const uint16_t* chain_basis,
                        int32_t chain_rank, float* margin) {
  if (!d) return DFLASH_EINVAL;
  if (!rows || !block_mean || !chain_mean || !margin || (block_rank && !block_basis) ||
      (chain_rank && !chain_basis))
    return fail(d, DFLASH_EINVAL, "route_margin: null pointer");
  if (m < 1 || m > dfl::kRouteMaxRows)
    return fail(d, DFLASH_EINVAL, "route_margin: m must be in [1, %d]", dfl::kRouteMaxRows);
  if (block_rank < 0 || block_rank > dfl::kRouteMaxRank || chain_rank < 0 ||
      chain_rank > dfl::kRouteMaxRank)
    return fail(d, DFLASH_EINVAL, "route_margin: ranks must be in [0, %d]", dfl::kRouteMaxRank);
  dfl::route_margin(d->st, rows, m, d->hs, block_mean, block_basis, block_rank, chain_mean,
                    chain_basis, chain_rank, d->rt_coef, d->rt_nrm, d->rt_part, margin);
  return launch_check(d, "route_margin");
}

// --------------------------------------------------------------- debug

static int matrix_of(dflash* d, int layer, int which, bool* is_i4, const void** codes,
                     const uint16_t** scales, dfl::TileMap* map, int* rows, int* cols) {
  if (which < DFLASH_W_FC && (layer < 0 || layer >= d->L))
    return fail(d, DFLASH_EINVAL, "debug: layer out of range");
  const int hs = d->hs;
  auto i4 = [&](const I4Set& s, int K, int t_off, int ntiles) {
    const size_t per_layer = (size_t)s.tiles * (K / 128);
    *is_i4 = true;
    *codes = s.codes + per_layer * 1024 * layer;
    *scales = s.scales + per_layer * 64 * layer;
    *map = dfl::TileMap{ntiles, ntiles, 0, t_off};
    *rows = ntiles * 16;
    *cols = K;
  };
  auto f16 = [&](const uint16_t* w, int N, int K) {
    *is_i4 = false;
    *codes = w;
    *scales = nullptr;
    *map = dfl::TileMap{(N + 15) / 16, (N + 15) / 16, 0, 0};
    *rows = N;
    *cols = K;
  };
  const size_t kp_layer = (size_t)d->ptiles * 16 * hs;
  switch (which) {
    case DFLASH_W_Q: i4(d->qkv, hs, 0, d->qd / 16); break;
    case DFLASH_W_K: i4(d->qkv, hs, d->qd / 16, d->kd / 16); break;
    case DFLASH_W_V: i4(d->qkv, hs, (d->qd + d->kd) / 16, d->kd / 16); break;
    case DFLASH_W_O: i4(d->o, d->qd, 0, hs / 16); break;
    case DFLASH_W_GATE: i4(d->gu, hs, 0, d->ffn / 16); break;
    case DFLASH_W_UP: i4(d->gu, hs, d->ffn / 16, d->ffn / 16); break;
    case DFLASH_W_DOWN: i4(d->down, d->ffn, 0, hs / 16); break;
    case DFLASH_W_ATTN_KPROJ: f16(d->attn_kproj + kp_layer * layer, d->P, hs); break;
    case DFLASH_W_MLP_KPROJ: f16(d->mlp_kproj + kp_layer * layer, d->P, hs); break;
    case DFLASH_W_FC: f16(d->fc, hs, d->tw); break;
    case DFLASH_W_HEAD: f16(d->head, d->V, hs); break;
    case DFLASH_W_SEL: f16(d->sel, d->rank, hs); break;
    default: return fail(d, DFLASH_EINVAL, "debug: unknown matrix id %d", which);
  }
  return DFLASH_OK;
}

int dflash_debug_dequant(dflash_t* d, int32_t layer, int32_t which, float* out) {
  if (!d || !out) return DFLASH_EINVAL;
  if (which > DFLASH_W_DOWN) return fail(d, DFLASH_EINVAL, "dequant: not an int4 matrix");
  bool is_i4;
  const void* codes;
  const uint16_t* scales;
  dfl::TileMap map;
  int rows, cols;
  int rc = matrix_of(d, layer, which, &is_i4, &codes, &scales, &map, &rows, &cols);
  if (rc) return rc;
  dfl::dequant_i4(d->st, static_cast<const uint8_t*>(codes), scales, map, rows, cols, out);
  return launch_check(d, "dequant");
}

int dflash_debug_matvec(dflash_t* d, int32_t layer, int32_t which, const float* x, int32_t m,
                        float* y) {
  if (!d || !x || !y) return DFLASH_EINVAL;
  if (m < 1 || m > kSettleRows) return fail(d, DFLASH_EINVAL, "matvec: m must be in [1, 256]");
  bool is_i4;
  const void* codes;
  const uint16_t* scales;
  dfl::TileMap map;
  int rows, cols;
  int rc = matrix_of(d, layer, which, &is_i4, &codes, &scales, &map, &rows, &cols);
  if (rc) return rc;
  if (cols > d->stage_cols) return fail(d, DFLASH_EINVAL, "matvec: matrix wider than the staging buffer");
  const int mb = (m + 15) / 16;
  // two planes, as every operand of the block and the settle
  const long ps = (long)kSettleRows * cols;
  dfl::to_a(d->st, x, cols, m, cols, d->taps_a, ps);
  // at m ≤ 16 an int4 matrix takes the block pass's kernel (two-span splits)
  const Split s = is_i4 && mb == 1 ? Split{dfl::i4_block_splits(cols, 2), 2}
                  : mb == 1        ? Split{dfl::f16_block_splits(cols), 0}
                  : is_i4          ? split_for(map.ntiles, kR, cols / 128, mb, 4)
                                   : split_big(map.ntiles, cols / 32);
  const long ss = (long)mb * 16 * rows;
  if ((long)s.S * ss > d->part_floats) return fail(d, DFLASH_EINVAL, "matvec: partials too large");
  if (is_i4 && mb == 1)
    dfl::gemm_i4_block(d->st, d->taps_a, ps, cols, static_cast<const uint8_t*>(codes), scales, map,
                       rows, 2, 2, d->part, ss);
  else if (is_i4)
    dfl::gemm_i4(d->st, d->taps_a, ps, cols, mb, static_cast<const uint8_t*>(codes), scales, map, rows,
                 s.S, s.per, d->part, ss);
  else if (mb > 1)
    dfl::gemm_big_f16(d->st, d->taps_a, ps, cols, mb, static_cast<const uint16_t*>(codes), map, rows,
                      s.S, s.per, d->part, ss);
  else
    dfl::gemm_f16_block(d->st, d->taps_a, ps, cols, static_cast<const uint16_t*>(codes), map, rows,
                        d->part, ss);
  dfl::sum_rows(d->st, d->part, s.S, ss, m, rows, y);
  return launch_check(d, "matvec");
}

// f32 rows lin [n][kd] to (out = false) or from (out = true) rows r0 .. of
// a layer's ring (wrapping)
static int ring_copy(dflash* d, uint16_t* ring, long cap, long r0, float* lin, long n, bool out,
                     const char* what) {
  dfl::store_rows(d->st, ring, cap, r0, lin, n, d->kv, d->hd, out);
  return hip_check(d, hipGetLastError(), what);
}

int dflash_debug_read_store(dflash_t* d, int32_t layer, int64_t row0, int64_t n, float* k_out,
                            float* v_out) {
  if (!d || !k_out || !v_out) return DFLASH_EINVAL;
  if (layer < 0 || layer >= d->L || n < 0 || row0 < d->ls[layer].dropped || row0 + n > d->len)
    return fail(d, DFLASH_EINVAL, "read_store: rows the layer does not hold");
  auto& S = d->ls[layer];
  int rc = ring_copy(d, S.k, S.cap, row0, k_out, n, true, "read_store");
  if (!rc) rc = ring_copy(d, S.v, S.cap, row0, v_out, n, true, "read_store");
  return rc;
}

int dflash_debug_load_store(dflash_t* d, int64_t first, int64_t len, const float* const* k,
                            const float* const* v) {
  if (!d || !k || !v) return DFLASH_EINVAL;
  if (first < 0 || len < 0) return fail(d, DFLASH_EINVAL, "load_store: bad range");
  for (int l = 0; l < d->L; ++l) {
    if (len && (!k[l] || !v[l])) return fail(d, DFLASH_EINVAL, "load_store: null layer pointer");
  }
  // as one settle_rows call of len rows on an empty context at first
  CtxState s{first, 0, 0, 0, std::vector<long>(d->L, 0)};
  if (!settle_state(d, s, len))
    return fail(d, DFLASH_ENOMEM, "load_store: %ld rows do not fit a layer's store", (long)len);
  if (int rc = reserve(d, s.len)) return rc;
  commit(d, s);
  for (int l = 0; l < d->L; ++l) {
    auto& S = d->ls[l];
    const long dr = S.dropped, held = len - dr;
    int rc = ring_copy(d, S.k, S.cap, dr, const_cast<float*>(k[l]) + (size_t)dr * d->kd, held,
                       false, "load_store");
    if (!rc)
      rc = ring_copy(d, S.v, S.cap, dr, const_cast<float*>(v[l]) + (size_t)dr * d->kd, held, false,
                     "load_store");
    if (rc) {
      lose_context(d);
      return rc;
    }
  }
  return DFLASH_OK;
}

int dflash_debug_last_block(dflash_t* d, float* hidden, float* hp) {
  if (!d) return DFLASH_EINVAL;
  int rc = DFLASH_OK;
  if (hidden)
    rc = hip_check(d, hipMemcpyAsync(hidden, d->bs.x, (size_t)d->B * d->hs * 4, hipMemcpyDeviceToDevice,
                                     d->st),
                   "last_block");
  if (!rc && hp && d->last_k)
    rc = hip_check(d, hipMemcpyAsync(hp, d->bs.hp + d->rank, (size_t)d->last_k * d->rank * 4,
                                     hipMemcpyDeviceToDevice, d->st),
                   "last_block");
  return rc;
}

int dflash_debug_set_trace(dflash_t* d, float* trace) {
  if (!d) return DFLASH_EINVAL;
  d->trace = trace;
  return DFLASH_OK;
}

int dflash_debug_select(dflash_t* d, const float* logits, const float* hp, int32_t k,
                        int32_t width, int32_t anchor, const int32_t* forced_prev, int32_t* cand,
                        float* unary, float* score, int32_t* chosen) {
  if (!d || !logits || !hp || !cand || !unary || !score || !chosen) return DFLASH_EINVAL;
  if (k < 1 || k >= 16) return fail(d, DFLASH_EINVAL, "select: k must be in [1, 15]");
  if (width < d->top || width > d->V) return fail(d, DFLASH_EINVAL, "select: bad width");
  if (anchor < 0 || anchor >= d->V) return fail(d, DFLASH_EINVAL, "select: bad anchor");
  dfl::select_all(d->st, logits, false, k, width, d->top, hp, d->rank, d->pbook, d->cbook, d->V,
                  anchor, forced_prev, d->bs.sel, cand, unary, score, chosen);
  return launch_check(d, "select");
}

}  // extern "C"
