/*
 * bsa.h -- libbsa: block-sparse scaled-dot-product attention for AMD MI355X
 * (gfx950), C ABI.
 *
 * The operation (Tessera, "Decoupling Logical Masks from GPU Execution for
 * Dynamic Block-Sparse Attention", abstract): block-sparse attention computes
 * only the blocks that a logical mask selects; the mask specifies which
 * attention interactions are computed. For query head h, query row i and key
 * j, key j is allowed iff the head's logical mask selects the block pair
 * (i / block_q[h], j / block_k[h]) and, when causal, j <= i + causal_kv_offset.
 * The result is exact softmax attention over the allowed keys:
 *   O[i]   = sum_j softmax_j(scale * q_i . k_j) v_j
 *   LSE[i] = ln sum_j exp(scale * q_i . k_j)
 * and a row with no allowed key gets O[i] = 0 and LSE[i] = -inf.
 *
 * With gqa_union set (CompactAttention, summary: the 2-D block mask is a KV
 * selection signal; a query-block union plus an intra-group union give a
 * per-group KV block table), every query head of a kv group attends to the
 * union, over the group's heads and over all query blocks, of the selected
 * key blocks (then the causal bound).
 *
 * The work is split in two calls, as the decoupling asks:
 *   bsa_plan     maps the logical mask to a physical tile plan for gfx950 --
 *                keeping, merging or subdividing logical blocks into physical
 *                tiles, building per-query-tile key-tile lists, the GQA union
 *                tables and paged tables, and the work list -- with the tile
 *                shape and schedule picked by a lookup table built offline
 *                (Tessera, abstract: physical mapping layer, task organization
 *                layer, profile-guided regime selection).
 *   bsa_forward  runs attention over Q/K/V with a plan and writes O and LSE.
 *
 * Conventions for every call:
 *   - Functions never throw; they return a bsa_status. On failure a
 *     thread-local message is available from bsa_last_error().
 *   - Every argument is checked before any device work is queued, so an
 *     error status means nothing was launched.
 *   - "device pointer" means memory allocated on the current HIP device; the
 *     caller owns it. "stream" is a hipStream_t passed as void* (NULL: the
 *     null stream). Work is queued on that stream; bsa_forward never
 *     synchronises.
 *   - Diagnostics go to stderr, under two environment variables read at each
 *     call. BSA_LOG=n (0..3, default 0): 1 prints every error and warning
 *     status with its message, 2 also each new plan's regime and sizes and
 *     each loaded table, 3 also each forward and backward launch.
 *     BSA_TRACE=1 prints the phases of each bsa_plan, bsa_plan_acsr,
 *     bsa_forward and bsa_backward call with their host wall time and the
 *     stream's time between events recorded at the phase boundaries; a
 *     traced call waits for its last event (synchronous with its stream, so
 *     not for use under graph capture). Neither changes any result.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 2

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1,    /* null pointer, bad value, misaligned tensor */
  BSA_ERR_UNSUPPORTED = 2,    /* valid but outside what this build supports */
  BSA_ERR_SHAPE_MISMATCH = 3, /* tensors or dtype disagree with the plan */
  BSA_ERR_OUT_OF_MEMORY = 4,  /* a device or host allocation failed */
  BSA_ERR_HIP = 5,            /* a HIP runtime call failed (message names it) */
  BSA_ERR_LUT = 6,            /* lookup table text malformed */
  BSA_WARN_LUT_DEFAULT = 7    /* not a failure: bsa_lut_load could not use the file it
                                 was given (missing or malformed) and returned the
                                 built-in default table instead (message says why) */
} bsa_status;

typedef enum { BSA_BF16 = 0, BSA_F32 = 1 } bsa_dtype;

typedef struct bsa_plan_s *bsa_plan_t;
typedef struct bsa_lut_s *bsa_lut_t;

/* Problem description. Host memory; bsa_plan copies what it needs. */
typedef struct {
  int32_t batch;         /* >= 1 */
  int32_t num_q_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0; q head h reads kv head h / (Hq/Hkv) */
  int64_t seqlen_q;      /* Sq >= 0, need not be a block multiple */
  int64_t seqlen_kv;     /* Skv >= 0 */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t dtype;         /* bsa_dtype of Q, K, V and O; LSE is always fp32 */
  const int32_t *block_q; /* [Hq] logical query block size per head: 16..512, power of 2 */
  const int32_t *block_k; /* [Hq] logical key block size per head: 16..512, power of 2 */
  int32_t mask_batch_broadcast; /* 1: one mask per head shared by every batch */
  int32_t causal;        /* 1: key j allowed only if j <= i + causal_kv_offset */
  int64_t causal_kv_offset;
  int32_t gqa_union;     /* 1: union semantics above; heads of a group share block_k */
  int32_t paged;         /* 1: K/V are page pools read through a page table */
  int32_t page_size;     /* tokens per page; a multiple of 64 when paged */
  int32_t pages_per_seq; /* page-table row length; page_size * pages_per_seq >= Skv */
  int32_t num_pages;     /* pages in each pool; every table entry must be < num_pages */
  float softmax_scale;   /* 0 => 1 / sqrt(head_dim) */
} bsa_problem;

/* A strided tensor whose last (head_dim) axis is contiguous. Strides count
 * elements. data and every stride must be 16-byte aligned.
 *   Q, O:  [batch][Hq][Sq][D]  -> stride_b, stride_h, stride_s
 *   K, V:  [batch][Hkv][Skv][D], or when paged a pool [num_pages][page_size][Hkv][D]
 *          with stride_b = page stride, stride_s = token stride within a page,
 *          stride_h = kv-head stride. */
typedef struct {
  void *data;
  int64_t stride_b, stride_h, stride_s;
} bsa_tensor;

/* Plan statistics, filled by bsa_plan_stats. */
typedef struct {
  int32_t tile_q, tile_k;   /* physical tile shape */
  int32_t sched;            /* 0 = row order (locality), 1 = longest first,
                               2 = row order dealt to the XCDs in blocks of 64 */
  int32_t split;            /* key tiles per work item before a row is split; 0 = never */
  int32_t pack;             /* 1: a group's heads share each task, head after head;
                               2: the same tasks with the heads interleaved row by row
                               (the few rows of a decode step sit in one wave) */
  int32_t reserved;
  int64_t rows, entries, items, partial_slots, combines;
  int64_t logical_nnz;      /* selected logical blocks in the mask (before any union) */
  int64_t logical_blocks;   /* all logical blocks of the mask */
  int64_t density_pm;       /* 1000 * logical_nnz / logical_blocks */
  int64_t imbalance16;      /* 16 * heaviest row / mean row, worst head */
  int64_t effective_blocks; /* blocks computed: after the union, causally feasible, all batches */
  double effective_flops;   /* sum over effective blocks of 4 * bq * bk * D */
  int64_t tile_live_subblocks; /* live (query sub-block, key sub-block) pairs over all entries */
  int64_t executed_tiles;   /* (query tile, key tile) pairs the forward computes, over all work
                               items: executed_tiles * tile_q * tile_k / (effective area) is the
                               merge waste of the plan (1 = none) */
  int64_t partial_slot_bound; /* partial slots a forward call's scratch is sized for, a bound
                                 computed on the host before the plan exists (>= partial_slots) */
} bsa_plan_info;

/* ABI version of the library (BSA_ABI_VERSION it was built with). */
int bsa_abi_version(void);

/* Static text for a status code. */
const char *bsa_status_str(bsa_status s);

/* Message of the last failure on the calling thread ("" if none). */
const char *bsa_last_error(void);

/* Lookup table of execution regimes (Tessera, abstract: plan selection through
 * a lookup table built from offline profiling). Text format:
 *   bsa-lut 1
 *   rule D dtype union paged bq_lo bq_hi bk_lo bk_hi dens_lo dens_hi imb_lo imb_hi
 *        -> Tq Tk sched split pack
 * or, with a fifth range on the query length seqlen_q (decode and short
 * chunks want their own regime):
 *   bsa-lut 2
 *   rule D dtype union paged bq_lo bq_hi bk_lo bk_hi dens_lo dens_hi imb_lo imb_hi
 *        sq_lo sq_hi -> Tq Tk sched split pack
 * pack is 0, 1 or 2 (see bsa_plan_info.pack; packing applies to union plans
 * with 2 or 4 query heads per kv head, else it is 0).
 * D, dtype (bf16|f32), union and paged (0|1) may be '*'; ranges are inclusive
 * and match the smallest block_q, smallest block_k, density per mille and
 * imbalance x16 of the mask (and seqlen_q); sched is local|lpt|dealt; the first
 * matching rule wins; with no match the built-in default applies
 * (128, 64, local, 0, 1).
 * bsa_lut_load reads a file. path NULL gives the built-in default table (the
 * packaged gfx950 table, compiled into the library). A file that cannot be
 * opened or does not parse also gives the built-in table, with status
 * BSA_WARN_LUT_DEFAULT (not an error: *out is set and must be freed; the
 * reason is in bsa_last_error). bsa_lut_parse reads text and returns
 * BSA_ERR_LUT on malformed text (no fallback). The table is host memory owned
 * by the library, immutable, and may be shared by threads; free it with
 * bsa_lut_free. */
bsa_status bsa_lut_load(const char *path, bsa_lut_t *out);
bsa_status bsa_lut_parse(const char *text, bsa_lut_t *out);
void bsa_lut_free(bsa_lut_t lut);

/* Build a plan for one mask (Tessera, abstract: physical mapping layer and
 * task organization layer; CompactAttention, summary: per-group KV block
 * tables over a paged cache).
 *   mask        device pointer, uint8, nonzero = selected. For each mask batch
 *               bm (1 if mask_batch_broadcast, else batch) and head h, a
 *               row-major [ceil(Sq/bq_h)][ceil(Skv/bk_h)] block, concatenated
 *               in (bm, h) order. Read only during the call.
 *   page_table  device pointer, int32 [batch][pages_per_seq] when paged, else
 *               ignored. Read only during the call; entries are validated.
 *   lut         regime table (NULL: built-in default).
 *   stream      stream for the planning kernels.
 * The call blocks once, on one small device-to-host read of the mask
 * features; all other planning work is queued on the stream, so the plan is
 * ready for any work queued on the same stream afterwards (work on another
 * stream must first wait for an event recorded on this one). The plan owns its
 * device memory and can be used by any number of bsa_forward calls with
 * matching tensors; its tile lists are immutable and are only read by those
 * calls. Everything a forward call writes besides O and LSE (work-queue
 * counters, split-KV partial results) lives in scratch that the call takes
 * from the device's stream-ordered pool on its own stream and returns there,
 * so any number of calls on one plan may be in flight at once, on any
 * streams, with any inputs. Free it with bsa_plan_free. */
bsa_status bsa_plan(const bsa_problem *problem, const uint8_t *mask, const int32_t *page_table,
                    bsa_lut_t lut, void *stream, bsa_plan_t *out);

/* Attention forward over a plan (Tessera, abstract: compute only the blocks
 * the logical mask selects). q, k, v, o: device tensors as described at
 * bsa_tensor, in the plan's dtype; lse: device pointer, fp32 [batch][Hq][Sq].
 * Every O row and LSE entry is written exactly once (empty rows included), so
 * O need not be cleared. Queued on stream; never synchronises. O and LSE must
 * not overlap Q, K or V. Work items are taken from per-XCD queues in the
 * order the plan's schedule gives, so which workgroup computes a row varies
 * from call to call; the values written do not. Scratch: one set of queue
 * counters plus, when the plan splits rows, partial O and LSE of
 * partial_slots capacity (fp32, Tq x (D + 1) per slot), from the device's
 * stream-ordered pool on this stream, returned in stream order after the
 * combine; BSA_ERR_OUT_OF_MEMORY if the pool cannot provide it. */
bsa_status bsa_forward(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                       const bsa_tensor *v, bsa_tensor *o, float *lse, void *stream);

/* bsa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, arguments, errors and results as bsa_forward, but the
 * call's scratch (work-queue counters and split-KV partials) is a static
 * device array of 64 MiB that the library holds on each device it runs on
 * until the process ends, so the call allocates nothing. A plan whose
 * scratch needs more (many split rows: see bsa_plan_info.partial_slot_bound,
 * 4 * tile_q * (head_dim + 1) bytes per slot, plus 256) is rejected with
 * BSA_ERR_UNSUPPORTED before anything is queued. Every call on a device
 * shares that device's array: calls that overlap in time on one device (on
 * any streams, any plans) race and must be serialised by the caller. Unlike
 * bsa_forward, a call on a stream other than the plan's records no event for
 * bsa_plan_free: order the plan's release after it yourself. */
bsa_status bsa_forward_noalloc(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                               const bsa_tensor *v, bsa_tensor *o, float *lse, void *stream);

/* Attention forward with K and V stored as OCP FP8 E4M3 bytes (one byte per
 * element: sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities), the low-precision KV cache of serving (CompactAttention
 * summary: zero-copy execution over the paged cache; the quantized-attention
 * line of the related-work page). The attention reads
 *   K = k_scale[g] * e4m3(k),  V = v_scale[g] * e4m3(v)
 * for kv head g, and is otherwise bsa_forward: same plan (bf16 dtype: Q and O
 * bf16), same layouts for k and v (dense or paged pool) with strides counted
 * in bytes (multiples of 16), k_scale and v_scale device pointers to fp32
 * [Hkv]. Every e4m3 value is exact in bf16, so the products are bf16 MFMAs on
 * the exact K and V values. BSA_ERR_UNSUPPORTED for fp32 plans. */
bsa_status bsa_forward_kv8(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                           const bsa_tensor *v, const float *k_scale, const float *v_scale,
                           bsa_tensor *o, float *lse, void *stream);

/* Backward of bsa_forward over the same plan: for a scalar loss with
 * dout = dL/dO, writes dq = dL/dQ, dk = dL/dK and dv = dL/dV. By the chain
 * rule through the softmax over each query row's allowed keys (Tessera,
 * abstract: only the selected blocks are computed, in training as in
 * inference):
 *   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . V_j - dO_i . O_i),
 *   dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i,
 * with P_ij = exp(scale Q_i . K_j - LSE_i) recomputed over the allowed keys.
 *   q, k, v:  the forward's inputs (bf16, dense K/V: paged plans are not
 *             supported);
 *   o, lse:   the forward's outputs for those inputs (lse fp32 [batch][Hq][Sq]);
 *   dout:     bf16, Q's shape [batch][Hq][Sq][D];
 *   dq:       bf16, Q's shape; dk, dv: bf16, K's shape [batch][Hkv][Skv][D].
 * Every element of dq, dk and dv is written exactly once (zero for rows
 * without keys and keys no query sees), by one workgroup in a fixed order,
 * so the results are the same bit for bit on every call. Outputs must not
 * overlap the inputs. Queued on stream; never synchronises; uses
 * batch * Hq * Sq * 4 bytes of scratch from the device's stream-ordered
 * pool, returned in stream order. BSA_ERR_UNSUPPORTED for fp32 or paged
 * plans. */
bsa_status bsa_backward(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                        const bsa_tensor *v, const bsa_tensor *o, const float *lse,
                        const bsa_tensor *dout, bsa_tensor *dq, bsa_tensor *dk, bsa_tensor *dv,
                        void *stream);

/* Canonical byte image of a plan (header; block sizes and the query- and
 * key-block interleave of each head; features, lists, entries, rows, work
 * list), for comparison with the reference planner. With host_buf NULL
 * only *bytes is set to the size needed; otherwise *bytes is the capacity on
 * input and the size on output. Synchronises with the plan's stream. */
bsa_status bsa_plan_export(bsa_plan_t plan, void *host_buf, size_t *bytes);

/* Plan statistics. Synchronises with the plan's stream. */
bsa_status bsa_plan_stats(bsa_plan_t plan, bsa_plan_info *out);

/* Parameters of block selection. */
typedef struct {
  int32_t keep_tenths; /* keep ceil(n * keep_tenths / 10) of a query block's n candidates (1..10) */
  int32_t top_k;       /* > 0: keep min(top_k, n) candidates instead; 0: use keep_tenths */
} bsa_select_params;

/* Block selection from pooled scores: writes the logical mask that bsa_plan
 * reads, from Q and K on the GPU. Hierarchical sparse attention selects the
 * key/value blocks with the best coarse attention scores (DashAttention page,
 * summary of NSA and InfLLMv2); CompactAttention (summary) treats the chunked-
 * prefill block mask as a KV selection signal; Sol-Attn (summary) thresholds
 * per query. Here, for batch b, query head h and query block qb, the coarse
 * score of key block kb (of h's kv group) is the dot product of the mean of
 * the query block's rows with the mean of the key block's rows; among the key
 * blocks that are causally feasible (first key <= last query of qb +
 * causal_kv_offset, or all blocks without causal masking) the best are kept
 * (params), ties to the lower block. All of it is fp32 in a fixed order (row
 * sums in ascending order, one division per mean, fused multiply-adds over d
 * ascending), so the mask is reproducible bit for bit.
 *   problem: shapes, block sizes, causal flag and offset, paging, dtype
 *            (mask_batch_broadcast must be 0: one mask per batch).
 *   q, k:    device tensors as for bsa_forward (k may be a paged pool read
 *            through page_table; pool entries outside [0, num_pages) are not
 *            followed).
 *   mask:    device pointer, uint8 [batch][per head: nqb_h x nkb_h], every
 *            byte written (0 or 1).
 * Up to 64 query heads and 8192 key blocks per head. Queued on stream; uses
 * scratch from the device's stream-ordered pool, returned in stream order. */
bsa_status bsa_select_blocks(const bsa_problem *problem, const bsa_select_params *params,
                             const bsa_tensor *q, const bsa_tensor *k, const int32_t *page_table,
                             uint8_t *mask, void *stream);

/* Affine-compressed sparse rows (SPLAT, abstract: the masks of common sparse
 * attention patterns have regular geometric properties, and its ACSR format
 * stores such a mask by an affine function of the row instead of per-row
 * column lists). Here a head's logical mask is given by up to
 * BSA_ACSR_MAX_RUNS runs; run j selects, in logical query block r, the key
 * blocks
 *   c = floor(row_num_j * r / row_den_j) + offset_j + stride_j * i,
 *       0 <= i < count_j,  kept when 0 <= c < ceil(Skv / block_k[h]),
 * and the row's selection is the union of its runs (runs may overlap). A
 * sliding window of w blocks is one run (1, 1, -w, 1, 2w + 1); a dilated
 * pattern (key block = query block mod s) is one run of stride s; global
 * columns are a run with row_num 0. */
#define BSA_ACSR_MAX_RUNS 4
typedef struct {
  int64_t row_num;  /* |row_num| <= 2^20 */
  int64_t row_den;  /* 1 .. 2^20 */
  int64_t offset;   /* |offset| <= 2^40 */
  int64_t stride;   /* 1 .. 2^31 */
  int64_t count;    /* 0 .. 2^40, and stride * count <= 2^50 */
} bsa_acsr_run;

typedef struct {
  int32_t num_runs; /* 0 .. BSA_ACSR_MAX_RUNS; 0 selects nothing */
  int32_t reserved; /* 0 */
  bsa_acsr_run runs[BSA_ACSR_MAX_RUNS];
} bsa_acsr_head;

/* Build a plan from affine row descriptors instead of a mask: the plan (and
 * its bsa_plan_export image) is the one bsa_plan builds from the mask the
 * descriptors expand to, but no mask exists anywhere and the call does not
 * block: the mask features are counted on the host from the runs (inclusion
 * and exclusion over the runs, congruences combined by the Chinese remainder
 * theorem), so there is no device-to-host read, and the planning kernels
 * evaluate the runs where bsa_plan reads mask bytes.
 *   problem: as for bsa_plan, with mask_batch_broadcast = 1 (one pattern for
 *            every batch), gqa_union = 0 and paged = 0 (BSA_ERR_UNSUPPORTED
 *            otherwise).
 *   heads:   host pointer, [Hq] descriptors; copied during the call.
 *   lut, stream, out: as for bsa_plan.
 * Every argument is checked before any device work is queued. */
bsa_status bsa_plan_acsr(const bsa_problem *problem, const bsa_acsr_head *heads, bsa_lut_t lut,
                         void *stream, bsa_plan_t *out);

/* The mask features that bsa_plan_acsr counts on the host, without a device:
 * for each head h, out[4h..4h+3] = selected logical blocks, the largest row
 * count, the number of empty rows, and the blocks that the causal bound
 * leaves reachable (every selected block when not causal) -- the per-head
 * values bsa_plan computes from the expanded mask. Same argument rules as
 * bsa_plan_acsr; out is host memory of 4 * Hq int64. */
bsa_status bsa_acsr_features(const bsa_problem *problem, const bsa_acsr_head *heads, int64_t *out);

/* Release a plan. Its device memory is returned in stream order on the plan's
 * stream, so the call may follow the last bsa_forward queued on that stream
 * directly. Forward and backward calls queued on other streams record an
 * event there after their kernels, and the release first makes the plan's
 * stream wait for those events, so it may also follow them directly (the
 * streams may be destroyed in between). NULL is ignored. */
void bsa_plan_free(bsa_plan_t plan);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
