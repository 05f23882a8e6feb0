// Internal declarations shared by the libbsa sources (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <atomic>
#include <mutex>
#include <vector>

#include "bsa.h"
#include "bsa_lut.h"

namespace bsa {

// Per query head, device resident. Live-bit decoding for a score at query
// offset qloc within its physical tile and key offset kloc within its key
// tile: bit = (qloc >> lq) * mk + (kloc >> lk).
struct HeadMeta {
  int64_t mask_off;  // offset of this head's [nqb][nkb] mask within one mask batch
  int64_t row_off;   // number of logical rows of the heads before this one
  int64_t bits_off;  // 64-bit words of the row bitmaps of the heads before this one
  int32_t nqb, nkb, bq, bk;
  int32_t lq, lk, mk;
  int32_t lqil;      // log2 of the query-block interleave (0: consecutive blocks)
  int32_t lkil;      // log2 of the key-block interleave (0: consecutive blocks)
};

// Query-block interleave candidates: s = 1, 2, 4, 8 for 128-row tiles that
// merge query blocks of 32 or 64 rows (non-union plans).
constexpr int kQilCands = 4;
// Key-block interleave candidates: s = 1, 2, 4, 8 for 64-key tiles that merge
// two 32-key blocks (non-union, non-paged plans without a causal bound).
constexpr int kKilCands = 4;

// Logical query block of sub-block iq of physical tile t when a tile merges
// 2^lm blocks with interleave 2^ls: in each full group of 2^(ls+lm) blocks,
// tile t takes the blocks t mod 2^ls apart by 2^ls; blocks past the last
// full group are merged consecutively. A partition of the head's nq blocks.
__host__ __device__ inline int64_t qblock_of(int64_t t, int64_t iq, int ls, int lm, int64_t nq) {
  const int lg = ls + lm;
  const int64_t full = nq >> lg;
  if (t < (full << ls)) return ((t >> ls) << lg) + (iq << ls) + (t & ((int64_t(1) << ls) - 1));
  return (full << lg) + ((t - (full << ls)) << lm) + iq;
}

// Query position of row R (0 .. tq-1) of physical tile qt of a non-packed
// row of the head with metadata m (ltq = log2 tq).
__host__ __device__ inline int64_t tile_query(const HeadMeta &m, int ltq, int64_t qt, int R) {
  if (m.lqil == 0) return (qt << ltq) + R;
  const int64_t qb = qblock_of(qt, R >> m.lq, m.lqil, ltq - m.lq, m.nqb);
  return (qb << m.lq) + (R & ((1 << m.lq) - 1));
}

// Key block of key sub-block ik of key tile kt of the head with metadata m
// when its tiles merge 2^lmk key blocks (the same partition as qblock_of).
__host__ __device__ inline int64_t tile_key_block(const HeadMeta &m, int lmk, int64_t kt, int ik) {
  return qblock_of(kt, ik, m.lkil, lmk, m.nkb);
}

// Key tile kt of 64 keys over two 32-key blocks of the head with metadata m:
// (x, y) such that key column c of the tile is key x + c, plus y when
// c >= 32 (y = 0 unless the head's key blocks are interleaved, then the
// tile's blocks lie s apart in each full group of 2s blocks).
__host__ __device__ inline int2 key_tile_span(const HeadMeta &m, int kt) {
  const int ls = m.lkil;
  if (ls == 0) return make_int2(kt * 64, 0);
  const int lg = ls + 1, full = m.nkb >> lg;
  if (kt < (full << ls)) return make_int2((((kt >> ls) << lg) + (kt & ((1 << ls) - 1))) * 32, ((1 << ls) - 1) * 32);
  return make_int2(((full << lg) + ((kt - (full << ls)) << 1)) * 32, 0);
}

// Counters written on the device by the planner.
enum { CNT_ENT = 0, CNT_ITEMS = 1, CNT_SLOTS = 2, CNT_COMB = 3, CNT_BADPAGE = 4, CNT_N = 8 };
// Work-queue counters of the attention kernel: one per XCD (8). Each forward
// call has its own set, in the call's scratch (with its split-KV partials),
// so calls that overlap in time never share counters or partials.
constexpr int kQueuesPerSet = 8;

// Host-side plan object. All device arrays live in two allocations.
struct Plan {
  // problem
  int32_t B, Hq, Hkv, G, D, dtype;
  int64_t Sq, Skv;
  int32_t causal;
  int64_t off;
  int32_t uni, paged, P, pps, npages, bcast;
  float scale;
  std::vector<int32_t> bq, bk;
  std::vector<int32_t> qil;          // query-block interleave per head (1 = consecutive)
  std::vector<int64_t> qil_cost;     // [Hq][kQilCands] key blocks listed per candidate
  std::vector<int32_t> kil;          // key-block interleave per head (1 = consecutive)
  bool key_interleaved = false;      // some head has kil > 1
  std::vector<int64_t> kil_cost;     // [Hq][kQilCands][kKilCands] key tiles listed
  // regime and geometry
  Regime rg;
  int32_t tr;  // query positions per physical row
  int64_t nqt, nkt, nlists, nrows, nlb, nbm, unkb;
  int64_t ent_cap, item_cap, slot_cap, comb_cap;
  int64_t part_slots;  // bound on the partial slots a forward writes (sizes its scratch)
  // mask features (host copy) and aggregates
  std::vector<int64_t> feat;  // [nbm][Hq][4]: nnz, max row, empty rows, effective blocks
  int64_t total_nnz, total_blocks, density_pm, imb16, min_bq, min_bk;
  // device memory
  std::vector<HeadMeta> hmeta_host;  // host copy kept alive for the asynchronous uploads
  void *pre = nullptr;    // features, counters, head metadata, union bits
  void *arena = nullptr;  // lists, entries, rows, work list, partials, scratch
  size_t pre_bytes = 0, arena_bytes = 0;
  HeadMeta *hmeta;
  unsigned long long *feat_dev;
  unsigned long long *qil_dev;  // [Hq][kQilCands] interleave costs (mask plans)
  int32_t *row_feat;  // per logical row: selected blocks, effective blocks
  unsigned long long *row_bits;  // per logical row: its selected key blocks, one bit each
  int64_t bits_per_bm = 0;       // words of row bitmaps per mask batch (0: none kept)
  int32_t *counters;
  uint8_t *uni_bits;
  const bsa_acsr_head *acsr = nullptr;  // device copy of the affine row descriptors (ACSR plans)
  int32_t *list_off, *ent_kt, *ent_page;
  uint32_t *ent_live;
  int32_t *row_ent, *items, *comb;
  hipStream_t stream;
  int device;
  // Streams other than the plan's that forward or backward calls used, each
  // with an event recorded after the call's last kernel: bsa_plan_free makes
  // the plan's stream wait for them before the memory is returned.
  mutable std::mutex use_mu;
  mutable std::vector<std::pair<hipStream_t, hipEvent_t>> used_on;
};
// Records that a call on stream s used the plan (no-op on the plan's stream).
bsa_status note_stream_use(const Plan &p, hipStream_t s);

struct AttnArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, v_sb, v_sh, v_ss, o_sb, o_sh, o_ss;
  const int32_t *items, *counters, *ent_kt, *ent_page;
  int32_t *queue;  // this call's kQueuesPerSet work-queue counters
  const uint32_t *ent_live;
  const HeadMeta *hm;
  float *part_o, *part_lse;
  int64_t Sq, Skv, off, nqt;
  int32_t Hq, Hkv, G, tq, tr, pack, causal, paged, P, sched;
  float scale_log2;  // softmax scale * log2(e)
  int32_t kv8;       // K and V are OCP FP8 E4M3 bytes scaled per kv head by k_scale, v_scale
  const float *k_scale, *v_scale;
  int32_t part_slots;  // partial slots the scratch holds (writes beyond are dropped)
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  float *delta;  // [B][Hq][Sq]: dO . O per query row, written by the dQ kernel
  float *lse2;   // [B][Hq][Sq]: LSE * log2(e) (+inf for rows without keys), written by the dQ kernel
  void *dq, *dk, *dv;
  int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss, do_sb, do_sh, do_ss, dq_sb, dq_sh, dq_ss;
  int64_t dk_sb, dk_sh, dk_ss, dv_sb, dv_sh, dv_ss;
  const int32_t *row_ent, *list_off, *ent_kt;
  const uint32_t *ent_live;
  const int32_t *t_off, *t_q0, *t_meta;  // key-major chunk index
  const uint32_t *t_live;
  const HeadMeta *hm;
  int64_t Sq, Skv, off, nqt, nkt;
  int32_t Hq, Hkv, G, tq, tr, tk, pack, uni, causal, nlb;
  float scale, scale_log2;
  // grp32: every element offset of Q and dO within one kv group's heads
  // ((G-1) * head stride + (Sq-1) * row stride + D) and G * Sq fit in 31
  // bits, so the dK/dV kernel forms its chunk addresses in 32-bit arithmetic
  // from these stride copies (checked on the host; 0 otherwise).
  int32_t grp32, q_sh32, q_ss32, do_sh32, do_ss32;
};

// Device allocations of plans and per-call scratch: stream-ordered (the
// device's default pool), on the stream that uses them, so repeated requests
// reuse freed blocks without waiting. With BSA_TEST_FAIL_ALLOC=n set, the
// n-th allocation (device or pinned host) counted from when the variable
// took that value fails, for tests of the out-of-memory paths (the variable
// is read at each allocation; a value change is seen there).
// Diagnostics to stderr, both read from the environment at each call.
// BSA_LOG=n (0..3, default 0): 1 prints every error and warning status with
// its message, 2 also each plan's regime and sizes, 3 also each forward and
// backward launch. BSA_TRACE=1 prints per-phase times of each plan, forward
// and backward call (host wall time, and the stream's time between events
// recorded at the phase boundaries); it waits for the call's last event, so
// a traced call is synchronous with its stream.
int log_level();
bool trace_on();
void log_msg(int level, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

hipError_t plan_alloc(void **ptr, size_t bytes, int device, hipStream_t stream);
void plan_release(void *ptr, hipStream_t stream);
bool alloc_fault_injected();

// Per-call scratch of a forward call: one set of work-queue counters, then
// the split-KV partial O (fp32 [slot][Tq][D]) and LSE (fp32 [slot][Tq]).
struct FwdScratch {
  size_t queue_off, part_o_off, part_lse_off, bytes;
};
FwdScratch fwd_scratch_layout(const Plan &p);

// Planner entry points (bsa_planner.hip). Each returns BSA_OK or BSA_ERR_HIP.
bsa_status plan_features(Plan &p, const uint8_t *mask, const int32_t *page_table);
bsa_status plan_build(Plan &p, const uint8_t *mask, const int32_t *page_table, void *scratch,
                      size_t scratch_bytes);
size_t plan_scratch_bytes(const Plan &p);

// Affine-compressed rows (bsa_acsr.hip). floor(a / b) for b > 0.
__host__ __device__ inline int64_t floor_div(int64_t a, int64_t b) {
  const int64_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}
// First key block of run u in logical query block r.
__host__ __device__ inline int64_t acsr_first(const bsa_acsr_run &u, int64_t r) {
  return (u.row_den == 1 ? u.row_num * r : floor_div(u.row_num * r, u.row_den)) + u.offset;
}
// Whether key block kb is one of run u's blocks in a row whose first block is f.
__host__ __device__ inline bool acsr_in_run(const bsa_acsr_run &u, int64_t f, int64_t kb) {
  const int64_t d = kb - f;
  if (d < 0) return false;
  if (u.stride == 1) return d < u.count;
  if (d < (int64_t(1) << 32) && u.stride < (int64_t(1) << 32)) {
    const uint32_t qq = (uint32_t)d / (uint32_t)u.stride;
    return (uint32_t)d == qq * (uint32_t)u.stride && qq < u.count;
  }
  return d % u.stride == 0 && d / u.stride < u.count;
}
// Argument checks of bsa_plan_acsr / bsa_acsr_features (host only, no device
// work), and the per-head mask features [Hq][4] counted from the runs.
bsa_status acsr_check(const bsa_problem &pr, const bsa_acsr_head *heads);
void acsr_features(const bsa_problem &pr, const bsa_acsr_head *heads, int64_t *out);
// Query-block interleave costs [Hq][kQilCands] counted from the runs.
void acsr_qil_costs(const bsa_problem &pr, const bsa_acsr_head *heads, int64_t *out, int64_t *kout);
// Planner side of an ACSR plan: head metadata and descriptors to the device
// through kernel arguments (no host buffer has to outlive the call), features
// on the host.
bsa_status plan_features_acsr(Plan &p, const bsa_acsr_head *heads, bsa_acsr_head *dev_heads,
                              const bsa_problem &pr);

// Key-major chunk index of a plan for the backward pass: for every (list
// batch, kv head, group of nkt_per consecutive key tiles = 128 keys), the
// 32-query chunks that may see one of its keys, in (head, query) order: first
// query, a packed word (head within the group | chunk index within its plan
// row << 8 | lq << 11 | lk << 16 | mk << 21) and nkt_per live words. Built
// into caller-provided scratch.
struct KvIndex {
  const int32_t *off, *q0, *meta;
  const uint32_t *live;
  int64_t nkp;
};
size_t plan_kv_index_bytes(const Plan &p, int nkt_per);
bsa_status plan_kv_index(const Plan &p, int nkt_per, void *scratch, KvIndex *out, hipStream_t s);

// Block selection from pooled scores (bsa_select.hip).
bsa_status select_blocks(const bsa_problem &pr, int keep_tenths, int top_k, const bsa_tensor &q,
                         const bsa_tensor &k, const int32_t *page_table, uint8_t *mask, hipStream_t s);

// Attention entry point (bsa_attention.hip).
bsa_status attention_launch(const Plan &p, const AttnArgs &a, hipStream_t stream);

// Backward entry point (bsa_backward.hip).
bsa_status backward_launch(const Plan &p, const BwdArgs &a, hipStream_t stream);

}  // namespace bsa

// The opaque plan handle of the C ABI.
struct bsa_plan_s : public bsa::Plan {};
