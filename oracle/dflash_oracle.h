/*
 * DFlash 2 drafter, CPU oracle — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow restatement of what the drafter computes, written from the
 * host definitions on the docs.rs page "cortiq_engine/dflash.rs" (cortiq-engine
 * 0.8.78): `rms`, `rotate`, `conv`, `Drafter::block`, `settle_rows`,
 * `select_with`, `top_k`, and the page's module overview. Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may call it; the
 * product path never does.
 *
 * Arithmetic: every product and sum is carried in binary64 (weights are
 * widened exactly from f16 / int4), except where the page fixes a precision:
 *   - the rotary angle is the binary32 product (float)pos * inv_freq[i],
 *     inv_freq[i] = (float)pow(theta, -2i/hd) computed in binary64;
 *   - eps enters as its binary32 value;
 *   - the context store holds binary32 keys and values.
 * Every output element is computed by one thread in one fixed order, so the
 * results do not depend on the OpenMP thread count.
 *
 * Shares no source, header, table or helper with the HIP library.
 */
#ifndef DFLASH_ORACLE_H
#define DFLASH_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symmetric int4, one f16 scale per 32 consecutive columns of a row.
   q: [rows][cols/2] bytes, column 2j in the low nibble of byte j and column
   2j+1 in the high nibble, two's complement. s: [rows][cols/32] f16 bits. */
typedef struct {
  const uint8_t* q;
  const uint16_t* s;
} orc_q4;

typedef struct {
  const float *in_norm, *post_norm; /* [hidden] */
  const float *q_norm, *k_norm;     /* [head_dim] */
  const float *attn_base, *mlp_base; /* [2][conv_kernel][hidden] */
  const uint16_t *attn_kproj, *mlp_kproj; /* f16 [2*kn*(hidden/conv_group)][hidden] */
  orc_q4 q, k, v, o, gate, up, down;
} orc_layer;

typedef struct {
  int hidden, intermediate, layers, heads, kv_heads, head_dim, vocab, block,
      mask_token, conv_group, conv_kernel, selector_rank, selector_top, n_taps;
  const int* windows;     /* [layers], 0 = every position */
  const uint8_t* rotary;  /* [layers], 0 = the layer carries no rotary position */
  double rope_theta, eps;
  const uint16_t* fc;        /* f16 [hidden][n_taps*hidden] */
  const float* hidden_norm;  /* [hidden] */
  const float* norm;         /* [hidden] */
  const uint16_t* sel_proj;  /* f16 [rank][hidden] */
  const uint16_t* pred_book; /* f16 [vocab][rank] */
  const uint16_t* succ_book; /* f16 [vocab][rank] */
  const uint16_t* embed;     /* f16 [vocab][hidden] */
  const uint16_t* head;      /* f16 [vocab][hidden] */
  const orc_layer* layer;    /* [layers] */
} orc_model;

double orc_f16(uint16_t h);
void orc_dequant_q4(const orc_q4* w, int rows, int cols, double* out);
void orc_inv_freq(double theta, int hd, float* out);
void orc_rms(const double* x, long rows, int len, const float* w, double eps, double* y);
void orc_rotate(double* x, long rows, int heads, int hd, const long* pos, const float* inv_freq);
void orc_conv(int rows, int hidden, int conv_group, int conv_kernel, int stage,
              const float* base, const double* d, const double* x, double* y);
void orc_apply_f16(const uint16_t* w, int rows, int cols, const double* x, int m, double* y);
void orc_apply_q4(const orc_q4* w, int rows, int cols, const double* x, int m, double* y);
void orc_attention(int rows, int heads, int kv_heads, int hd, const double* q, const double* k,
                   const double* v, const float* store_k, const float* store_v, long first,
                   long len, long dropped, long a, int window, double* y);
int orc_settle(const orc_model* m, const float* taps, int n, long pos0, float* k_out, float* v_out);
int orc_block(const orc_model* m, const float* const* store_k, const float* const* store_v,
              long first, long len, const long* dropped, int anchor, long a, int k, int width,
              double* logits, double* hp, double* hidden, double* trace);
void orc_top_k(const double* x, long n, int k, double* val, int* idx);
void orc_select(const orc_model* m, const double* logits, int width, const double* hp, int k,
                int anchor, const int* forced_prev, int* cand, double* unary, double* score,
                int* chosen, int* plain);

#ifdef __cplusplus
}
#endif
#endif
