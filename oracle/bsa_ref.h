/*
 * bsa_ref.h -- CPU oracle for block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY. This library defines what the GPU library must
 * compute; it is slow and obviously correct, and it shares no code, header,
 * table or helper with the GPU path. Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.
 *
 * What it computes (Tessera, "Decoupling Logical Masks from GPU Execution
 * for Dynamic Block-Sparse Attention", abstract): block-sparse attention that
 * computes only the blocks a logical mask selects, i.e. exact softmax
 * attention restricted to the selected (query-block, key-block) pairs. A
 * fully masked query row has output 0 and log-sum-exp -inf. Under the GQA
 * union reading (CompactAttention, summary: the block mask is a KV selection
 * signal, unioned over the query blocks of a chunk and over the query heads
 * of a group), every query head of a group attends to the union of the
 * group's selected key blocks.
 *
 * It also holds a reference planner: the keep / merge / subdivide mapping of
 * logical blocks to physical tiles, the per-tile key-tile lists, the GQA
 * union tables and paged tables, and the work list (Tessera, abstract:
 * physical mapping layer, task organization layer, regime lookup table),
 * written out plainly from the plan specification.
 */
#ifndef BSA_REF_H
#define BSA_REF_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, hq, hkv;
  int64_t sq, skv;
  int32_t d;
  int32_t dtype;          /* 0: Q/K/V are bf16 bit patterns (uint16); 1: fp32 */
  const int32_t *bq, *bk; /* [hq] logical block sizes */
  int32_t mask_broadcast; /* 1: one mask per head shared by every batch */
  int32_t causal;
  int64_t causal_offset;  /* key j allowed only if j <= i + causal_offset */
  int32_t gqa_union;
  int32_t paged, page_size, pages_per_seq, num_pages;
  double scale;           /* 0 => 1/sqrt(d) */
} ref_problem;

/* Forward. Q is [batch][hq][sq][d]; K and V are [batch][hkv][skv][d], or,
 * when paged, pools [num_pages][page_size][hkv][d] read through
 * page_table[batch][pages_per_seq]. rows holds nrows (b, h, i) triples to
 * compute (NULL: every row, in (b, h, i) order). Outputs o[nrows][d] and
 * lse[nrows] in double. mode 0 builds each full score row with -inf at masked
 * keys; mode 1 visits only allowed keys, in the same ascending order.
 * Returns 0, or -1 for an invalid problem. */
int ref_forward(const ref_problem *p, const uint8_t *mask, const int32_t *page_table,
                const void *q, const void *k, const void *v, int mode, const int64_t *rows,
                int64_t nrows, double *o, double *lse, int nthreads);

/* Forward with K and V stored as OCP FP8 E4M3 bytes (same layouts as
 * ref_forward, one byte per element) and one fp32 scale per kv head: the
 * attention reads K = k_scale[g] * e4m3(k), V = v_scale[g] * e4m3(v). Q is
 * bf16 (p->dtype must be 0). Returns 0, or -1 for invalid arguments. */
int ref_forward_kv8(const ref_problem *p, const uint8_t *mask, const int32_t *page_table,
                    const void *q, const uint8_t *k, const uint8_t *v, const float *k_scale,
                    const float *v_scale, int mode, const int64_t *rows, int64_t nrows, double *o,
                    double *lse, int nthreads);

/* Value of an OCP FP8 E4M3 byte (bias 7, subnormals, NaN at S.1111.111, no
 * infinities). */
double ref_e4m3(uint8_t b);

/* Backward (dense K/V only): gradients of a scalar loss L given dout =
 * dL/dO ([batch][hq][sq][d], same dtype as Q), by the chain rule through the
 * softmax over each row's allowed keys (see bsa_ref.c). dq receives nqrows
 * rows (qrows as in ref_forward; NULL: every row) as [nqrows][d]; dk and dv
 * receive the keys [klo, khi) of every (batch, kv head) as
 * [batch][hkv][khi-klo][d]. dq, or dk and dv, may be NULL to skip them.
 * Returns 0, or -1 for an invalid or paged problem. */
int ref_backward(const ref_problem *p, const uint8_t *mask, const void *q, const void *k,
                 const void *v, const void *dout, const int64_t *qrows, int64_t nqrows,
                 int64_t klo, int64_t khi, double *dq, double *dk, double *dv, int nthreads);

/* Per (mask batch, head): nnz, max row popcount, empty rows, effective blocks
 * (selected and causally feasible, after the union in union mode).
 * out has mask_batches * hq * 4 entries. */
int ref_features(const ref_problem *p, const uint8_t *mask, int64_t *out);

/* Reference planner. Writes the canonical plan image to image (capacity
 * *bytes); with image == NULL only reports the size. lut_text NULL selects the
 * built-in rule set; force, when not NULL, is {Tq, Tk, sched, split, pack} and
 * replaces the table's choice. Returns 0, -1 invalid problem, -2 bad table,
 * -3 unsupported geometry, -4 capacity too small. */
int ref_plan(const ref_problem *p, const uint8_t *mask, const int32_t *page_table,
             const char *lut_text, const int32_t *force, uint8_t *image, size_t *bytes);

/* Block selection from pooled scores (mask producer): for every batch b,
 * query head h and query block, the mean of the block's query rows is scored
 * against the mean of every causally feasible key block of h's kv group (fp32,
 * fixed order: see bsa_ref.c), and the best min(top_k, n) blocks (top_k > 0)
 * or ceil(n * keep_tenths / 10) blocks are kept, ties to the lower block.
 * Writes the uint8 mask in the layout ref_forward reads, one mask per batch
 * (mask_broadcast must be 0). Returns 0, or -1 for invalid arguments. */
int ref_select(const ref_problem *p, const int32_t *page_table, const void *q, const void *k,
               int32_t keep_tenths, int32_t top_k, uint8_t *mask);

#ifdef __cplusplus
}
#endif
#endif
