// libbsa C ABI: argument checking, regime lookup table, plan object, forward
// launch, plan export and statistics.
#include <algorithm>
#include <chrono>
#include <cstdarg>
#include <cstdlib>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <mutex>
#include <sstream>

#include "bsa_internal.h"

#include <climits>

namespace bsa {

static thread_local std::string g_err;

int log_level() {
  const char *v = std::getenv("BSA_LOG");
  return v ? std::max(0, std::min(3, std::atoi(v))) : 0;
}

bool trace_on() {
  const char *v = std::getenv("BSA_TRACE");
  return v && std::atoi(v) > 0;
}

void log_msg(int level, const char *fmt, ...) {
  if (level > log_level()) return;
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[bsa] %s\n", buf);
}

bsa_status fail(bsa_status s, const std::string &msg) {
  g_err = msg;
  log_msg(1, "%s: %s", bsa_status_str(s), msg.c_str());
  return s;
}

// Phase timers of one call (BSA_TRACE=1); inert otherwise. mark() closes the
// phase that began at the previous mark: it takes the host clock and records
// an event on the call's stream. report() waits for the last event and prints
// each phase's host and stream time.
class Trace {
 public:
  Trace(const char *what, hipStream_t s) : what_(what), s_(s), on_(trace_on()) {
    if (on_) t0_ = std::chrono::steady_clock::now(), mark("start");
  }
  ~Trace() {
    for (auto &m : marks_)
      if (m.ev) (void)hipEventDestroy(m.ev);
  }
  Trace(const Trace &) = delete;
  Trace &operator=(const Trace &) = delete;

  void mark(const char *phase) {
    if (!on_) return;
    Mark m{phase, nullptr, std::chrono::duration<double, std::milli>(
                               std::chrono::steady_clock::now() - t0_).count()};
    if (hipEventCreate(&m.ev) != hipSuccess) m.ev = nullptr;
    if (m.ev && hipEventRecord(m.ev, s_) != hipSuccess) {
      (void)hipEventDestroy(m.ev);
      m.ev = nullptr;
    }
    marks_.push_back(m);
  }

  void report(const std::string &detail = "") {
    if (!on_ || marks_.size() < 2) return;
    const bool synced = marks_.back().ev && hipEventSynchronize(marks_.back().ev) == hipSuccess;
    std::string line = std::string("[bsa trace] ") + what_ + (detail.empty() ? "" : " (" + detail + ")") + ":";
    char buf[160];
    for (size_t i = 1; i < marks_.size(); ++i) {
      float ms = -1.f;
      if (!synced || !marks_[i - 1].ev || !marks_[i].ev ||
          hipEventElapsedTime(&ms, marks_[i - 1].ev, marks_[i].ev) != hipSuccess)
        ms = -1.f;
      std::snprintf(buf, sizeof buf, " %s %.3f ms stream / %.3f ms host;", marks_[i].phase, ms,
                    marks_[i].host_ms - marks_[i - 1].host_ms);
      line += buf;
    }
    std::snprintf(buf, sizeof buf, " total %.3f ms host",
                  std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0_).count());
    std::fprintf(stderr, "%s%s\n", line.c_str(), buf);
  }

 private:
  struct Mark {
    const char *phase;
    hipEvent_t ev;
    double host_ms;
  };
  const char *what_;
  hipStream_t s_;
  bool on_;
  std::chrono::steady_clock::time_point t0_;
  std::vector<Mark> marks_;
};

#define HIP_TRY(expr)                                                          \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess)                                                      \
      return fail(BSA_ERR_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static bool is_block(int32_t x) { return x >= 16 && x <= 512 && (x & (x - 1)) == 0; }
static int ilog2(int64_t x) {
  int r = 0;
  while ((int64_t(1) << (r + 1)) <= x) ++r;
  return r;
}
static size_t aligned(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Problem checks (all before any device work)
// ---------------------------------------------------------------------------
// need_mask = false: an ACSR plan, which reads neither a mask nor a page table.
static bsa_status check_problem(const bsa_problem *p, const uint8_t *mask, const int32_t *table,
                                bool need_mask = true) {
  if (!p) return fail(BSA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(BSA_ERR_INVALID_ARG, "batch and head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(BSA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (p->seqlen_q < 0 || p->seqlen_kv < 0) return fail(BSA_ERR_INVALID_ARG, "negative sequence length");
  if (p->seqlen_q > (int64_t(1) << 31) || p->seqlen_kv > (int64_t(1) << 31))
    return fail(BSA_ERR_UNSUPPORTED, "sequence length above 2^31");
  if (p->head_dim != 64 && p->head_dim != 128) return fail(BSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->dtype != BSA_BF16 && p->dtype != BSA_F32) return fail(BSA_ERR_INVALID_ARG, "unknown dtype");
  if (!p->block_q || !p->block_k) return fail(BSA_ERR_INVALID_ARG, "block_q / block_k is NULL");
  for (int h = 0; h < p->num_q_heads; ++h)
    if (!is_block(p->block_q[h]) || !is_block(p->block_k[h]))
      return fail(BSA_ERR_UNSUPPORTED, "block sizes must be powers of two in [16, 512] (head " +
                                           std::to_string(h) + ")");
  if ((p->mask_batch_broadcast | p->causal | p->gqa_union | p->paged) & ~1)
    return fail(BSA_ERR_INVALID_ARG, "flags must be 0 or 1");
  if (!(p->softmax_scale >= 0.f) || std::isinf(p->softmax_scale))
    return fail(BSA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (p->gqa_union) {
    const int gs = p->num_q_heads / p->num_kv_heads;
    for (int h = 0; h < p->num_q_heads; ++h)
      if (p->block_k[h] != p->block_k[(h / gs) * gs])
        return fail(BSA_ERR_INVALID_ARG, "gqa_union needs equal block_k within each kv group");
  }
  if (p->paged) {
    if (p->page_size < 64 || p->page_size % 64)
      return fail(BSA_ERR_UNSUPPORTED, "page_size must be a positive multiple of 64");
    if (p->pages_per_seq < 1 || p->num_pages < 1)
      return fail(BSA_ERR_INVALID_ARG, "pages_per_seq and num_pages must be >= 1");
    if ((int64_t)p->page_size * p->pages_per_seq < p->seqlen_kv)
      return fail(BSA_ERR_INVALID_ARG, "page table too short for seqlen_kv");
    if (need_mask && !table) return fail(BSA_ERR_INVALID_ARG, "paged problem needs a page table");
  }
  int64_t msize = 0;
  for (int h = 0; h < p->num_q_heads; ++h)
    msize += cdiv(p->seqlen_q, p->block_q[h]) * cdiv(p->seqlen_kv, p->block_k[h]);
  if (need_mask && msize > 0 && !mask) return fail(BSA_ERR_INVALID_ARG, "mask is NULL");
  return BSA_OK;
}

// ---------------------------------------------------------------------------
// Plan memory comes from the device's default stream-ordered pool
// (hipMallocAsync / hipFreeAsync on the plan's stream). A block freed by one
// plan is reused by the next plan built on the same stream without waiting:
// stream order already places the new plan's kernels after the work that
// used the old one. The pool keeps freed memory (release threshold raised
// once per device) instead of returning it to the driver at each
// synchronisation.
// ---------------------------------------------------------------------------
namespace {
std::mutex g_pool_mu;
std::vector<int> g_pool_ready;  // devices whose pool threshold is set

// Pinned host blocks for the planner's read-back, kept for reuse (one per
// concurrently planning thread at most).
std::mutex g_pin_mu;
std::vector<std::pair<void *, size_t>> g_pin_free;

struct PinnedBuf {
  void *p = nullptr;
  size_t n = 0;
  explicit PinnedBuf(size_t bytes) {
    if (alloc_fault_injected()) return;
    {
      std::lock_guard<std::mutex> lk(g_pin_mu);
      for (size_t i = 0; i < g_pin_free.size(); ++i)
        if (g_pin_free[i].second >= bytes) {
          p = g_pin_free[i].first, n = g_pin_free[i].second;
          g_pin_free.erase(g_pin_free.begin() + i);
          return;
        }
    }
    n = std::max<size_t>(bytes, size_t(64) << 10);
    if (hipHostMalloc(&p, n, hipHostMallocDefault) != hipSuccess) p = nullptr, n = 0;
  }
  ~PinnedBuf() {
    if (!p) return;
    std::lock_guard<std::mutex> lk(g_pin_mu);
    g_pin_free.emplace_back(p, n);
  }
  PinnedBuf(const PinnedBuf &) = delete;
  PinnedBuf &operator=(const PinnedBuf &) = delete;
};
}  // namespace

// Allocation-failure injection (BSA_TEST_FAIL_ALLOC=n): the countdown is
// reset whenever the variable's value changes, and the allocation that brings
// it to zero fails; later ones succeed until the value changes again.
bool alloc_fault_injected() {
  static std::mutex mu;
  static std::string last;
  static long countdown = 0;
  const char *v = std::getenv("BSA_TEST_FAIL_ALLOC");
  std::lock_guard<std::mutex> lk(mu);
  const std::string cur = v ? v : "";
  if (cur != last) {
    last = cur;
    countdown = v ? std::strtol(v, nullptr, 10) : 0;
  }
  if (countdown <= 0) return false;
  return --countdown == 0;
}

hipError_t plan_alloc(void **ptr, size_t bytes, int device, hipStream_t stream) {
  if (alloc_fault_injected()) {
    *ptr = nullptr;
    return hipErrorOutOfMemory;
  }
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    if (std::find(g_pool_ready.begin(), g_pool_ready.end(), device) == g_pool_ready.end()) {
      hipMemPool_t pool;
      if (hipDeviceGetDefaultMemPool(&pool, device) == hipSuccess) {
        uint64_t keep = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
      }
      g_pool_ready.push_back(device);
    }
  }
  return hipMallocAsync(ptr, bytes, stream);
}

void plan_release(void *ptr, hipStream_t stream) {
  if (ptr) (void)hipFreeAsync(ptr, stream);
}

bsa_status note_stream_use(const Plan &p, hipStream_t s) {
  if (s == p.stream) return BSA_OK;
  std::lock_guard<std::mutex> lk(p.use_mu);
  hipEvent_t ev = nullptr;
  for (auto &u : p.used_on)
    if (u.first == s) ev = u.second;
  if (!ev) {
    HIP_TRY(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    p.used_on.emplace_back(s, ev);
  }
  HIP_TRY(hipEventRecord(ev, s));
  return BSA_OK;
}

static void free_plan(bsa_plan_s *p) {
  if (!p) return;
  // Work queued on other streams that reads the plan comes first.
  for (auto &u : p->used_on) {
    (void)hipStreamWaitEvent(p->stream, u.second, 0);
    (void)hipEventDestroy(u.second);
  }
  p->used_on.clear();
  plan_release(p->pre, p->stream);
  plan_release(p->arena, p->stream);
  delete p;
}

// Regime: forced by the table's first matching rule, then made valid.
static bsa_status choose_regime(Plan &p, const bsa_lut_s *lut) {
  Regime rg;
  if (lut) {
    const int64_t key[4] = {p.D, p.dtype, p.uni, p.paged};
    const int64_t val[5] = {p.min_bq, p.min_bk, p.density_pm, p.imb16, p.Sq};
    (void)lut_match(*lut, key, val, &rg);
  }
  if (!(p.uni && (p.G == 2 || p.G == 4))) rg.pack = 0;
  if (p.dtype == BSA_F32) rg.tq = 128, rg.tk = 64;  // fp32 tiles are 128 x 64
  if (rg.tq == 256) rg.tk = 64;                      // 256-row tiles use 64 keys
  if (p.paged && p.P % rg.tk) {
    if (rg.tk == 128 && p.P % 64 == 0) rg.tk = 64;
    else return fail(BSA_ERR_UNSUPPORTED, "page_size not a multiple of the key tile");
  }
  // At most 32 live bits per tile: shrink Tk to 64, then Tq to 128.
  for (;;) {
    bool bad = false;
    for (int h = 0; h < p.Hq; ++h) {
      const int mq = (!p.uni && p.bq[h] < rg.tq) ? rg.tq / p.bq[h] : 1;
      const int mk = p.bk[h] < rg.tk ? rg.tk / p.bk[h] : 1;
      if (mq * mk > 32) bad = true;
    }
    if (!bad) break;
    if (rg.tk == 128) rg.tk = 64;
    else if (rg.tq == 256) rg.tq = 128;
    else return fail(BSA_ERR_UNSUPPORTED, "block sizes too small for the tile (more than 32 sub-blocks)");
  }
  p.rg = rg;
  return BSA_OK;
}

FwdScratch fwd_scratch_layout(const Plan &P) {
  FwdScratch f;
  f.queue_off = 0;
  f.part_o_off = aligned(sizeof(int32_t) * kQueuesPerSet);
  f.part_lse_off = f.part_o_off + aligned(sizeof(float) * (size_t)P.part_slots * P.rg.tq * P.D);
  f.bytes = f.part_lse_off + aligned(sizeof(float) * (size_t)P.part_slots * P.rg.tq);
  return f;
}

// Static forward scratch for bsa_forward_noalloc: one array per device,
// allocated with the code object and held until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory, so its device
// address is looked up once per device (with that device current) and only
// that address is handed to kernels.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

static std::mutex g_static_mu;
static std::vector<std::pair<int, void *>> g_static_addr;  // (device, address)

static bsa_status static_scratch(int device, void **out) {
  std::lock_guard<std::mutex> lk(g_static_mu);
  for (auto &d : g_static_addr)
    if (d.first == device) {
      *out = d.second;
      return BSA_OK;
    }
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(BSA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  g_static_addr.emplace_back(device, ptr);
  *out = ptr;
  return BSA_OK;
}

}  // namespace bsa

using namespace bsa;

extern "C" {

int bsa_abi_version(void) { return BSA_ABI_VERSION; }

const char *bsa_status_str(bsa_status s) {
  switch (s) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported";
    case BSA_ERR_SHAPE_MISMATCH: return "shape mismatch";
    case BSA_ERR_OUT_OF_MEMORY: return "out of memory";
    case BSA_ERR_HIP: return "HIP error";
    case BSA_ERR_LUT: return "lookup table error";
    case BSA_WARN_LUT_DEFAULT: return "warning: lookup table replaced by the built-in default";
  }
  return "unknown status";
}

const char *bsa_last_error(void) { return g_err.c_str(); }

bsa_status bsa_lut_parse(const char *text, bsa_lut_t *out) {
  if (!text || !out) return fail(BSA_ERR_INVALID_ARG, "text or out is NULL");
  *out = nullptr;
  auto *l = new bsa_lut_s;
  if (bsa_status s = parse_lut(text, l)) {
    delete l;
    return s;
  }
  *out = l;
  return BSA_OK;
}

bsa_status bsa_lut_load(const char *path, bsa_lut_t *out) {
  if (!out) return fail(BSA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  // The built-in default: the packaged table compiled into the library.
  auto builtin = [&]() -> bsa_status {
    auto *l = new bsa_lut_s;
    if (bsa_status s = parse_lut(kDefaultLutText, l)) {
      delete l;
      return s;
    }
    *out = l;
    return BSA_OK;
  };
  if (!path) return builtin();
  std::ifstream f(path);
  std::string why;
  if (!f) {
    why = std::string("cannot open lookup table ") + path;
  } else {
    std::stringstream ss;
    ss << f.rdbuf();
    auto *l = new bsa_lut_s;
    if (parse_lut(ss.str().c_str(), l) == BSA_OK) {
      log_msg(2, "lookup table %s: %zu rules", path, l->rules.size());
      *out = l;
      return BSA_OK;
    }
    delete l;
    why = std::string("malformed lookup table ") + path + ": " + g_err;
  }
  // Missing or malformed file: the built-in table, with a warning status.
  if (bsa_status s = builtin()) return s;
  g_err = why + "; using the built-in default table";
  log_msg(1, "%s: %s", bsa_status_str(BSA_WARN_LUT_DEFAULT), g_err.c_str());
  return BSA_WARN_LUT_DEFAULT;
}

void bsa_lut_free(bsa_lut_t lut) { delete lut; }

// The plan object of a checked problem (host fields only).
static bsa_plan_s *new_plan(const bsa_problem *pr, void *stream) {
  bsa_plan_s *p = new bsa_plan_s();
  Plan &P = *p;
  P.B = pr->batch, P.Hq = pr->num_q_heads, P.Hkv = pr->num_kv_heads, P.G = P.Hq / P.Hkv;
  P.D = pr->head_dim, P.dtype = pr->dtype, P.Sq = pr->seqlen_q, P.Skv = pr->seqlen_kv;
  P.causal = pr->causal, P.off = pr->causal_kv_offset, P.uni = pr->gqa_union;
  P.paged = pr->paged, P.P = pr->paged ? pr->page_size : 0, P.pps = pr->paged ? pr->pages_per_seq : 0;
  P.npages = pr->paged ? pr->num_pages : 0, P.bcast = pr->mask_batch_broadcast;
  P.scale = pr->softmax_scale > 0.f ? pr->softmax_scale : 1.f / std::sqrt((float)P.D);
  P.bq.assign(pr->block_q, pr->block_q + P.Hq);
  P.bk.assign(pr->block_k, pr->block_k + P.Hq);
  P.nbm = P.bcast ? 1 : P.B;
  P.nlb = (P.paged || !P.bcast) ? P.B : 1;
  P.stream = (hipStream_t)stream;
  P.unkb = 0;
  for (int h = 0; h < P.Hq; ++h) P.unkb = std::max<int64_t>(P.unkb, cdiv(P.Skv, P.bk[h]));
  return p;
}

// Device header of a plan: counters, features, head metadata,
// union bits, per-row features and (ACSR plans) the affine descriptors.
// Returns the descriptors' device address in *acsr_dev when acsr is set.
static bsa_status alloc_header(Plan &P, bool acsr, bsa_acsr_head **acsr_dev) {
  const size_t feat_bytes = sizeof(int64_t) * 4 * P.nbm * P.Hq;
  int64_t rows_per_bm = 0;
  for (int h = 0; h < P.Hq; ++h) rows_per_bm += cdiv(P.Sq, P.bq[h]);
  // Row bitmaps (mask plans without union: the interleave costs read them).
  P.bits_per_bm = 0;
  if (!acsr && !P.uni)
    for (int h = 0; h < P.Hq; ++h) P.bits_per_bm += cdiv(P.Sq, P.bq[h]) * cdiv(cdiv(P.Skv, P.bk[h]), 64);
  const size_t bits_bytes = sizeof(unsigned long long) * P.nbm * P.bits_per_bm;
  const size_t acsr_bytes = acsr ? sizeof(bsa_acsr_head) * P.Hq : 0;
  // query-interleave costs [Hq][kQilCands], then key-interleave costs
  // [Hq][kQilCands][kKilCands]
  const size_t cost_bytes = sizeof(unsigned long long) * kQilCands * (1 + kKilCands) * P.Hq;
  const size_t pre_bytes = aligned(sizeof(int32_t) * CNT_N) + aligned(feat_bytes) + aligned(cost_bytes) +
                           aligned(sizeof(int64_t) * (kQilCands * P.Hq + 1)) +
                           aligned(sizeof(HeadMeta) * P.Hq) +
                           aligned((size_t)P.nbm * P.Hkv * std::max<int64_t>(P.unkb, 1)) +
                           aligned(sizeof(int32_t) * 2 * std::max<int64_t>(acsr ? 1 : P.nbm * rows_per_bm, 1)) +
                           aligned(acsr_bytes) + aligned(bits_bytes);
  if (plan_alloc(&P.pre, pre_bytes, P.device, P.stream) != hipSuccess)
    return fail(BSA_ERR_OUT_OF_MEMORY, "device allocation of plan header failed");
  P.pre_bytes = pre_bytes;
  uint8_t *pb = (uint8_t *)P.pre;
  // Counters and features are adjacent: the one read-back copies both.
  P.counters = (int32_t *)pb;
  pb += aligned(sizeof(int32_t) * CNT_N);
  P.feat_dev = (unsigned long long *)pb;
  pb += aligned(feat_bytes);
  P.qil_dev = (unsigned long long *)pb;  // costs, then the cost kernel's wave offsets
  pb += aligned(cost_bytes) + aligned(sizeof(int64_t) * (kQilCands * P.Hq + 1));
  P.hmeta = (HeadMeta *)pb;
  pb += aligned(sizeof(HeadMeta) * P.Hq);
  P.uni_bits = pb;
  pb += aligned((size_t)P.nbm * P.Hkv * std::max<int64_t>(P.unkb, 1));
  P.row_feat = (int32_t *)pb;
  pb += aligned(sizeof(int32_t) * 2 * std::max<int64_t>(acsr ? 1 : P.nbm * rows_per_bm, 1));
  if (acsr_dev) *acsr_dev = acsr ? (bsa_acsr_head *)pb : nullptr;
  pb += aligned(acsr_bytes);
  P.row_bits = bits_bytes ? (unsigned long long *)pb : nullptr;
  if (hipMemsetAsync(P.counters, 0, sizeof(int32_t) * CNT_N, P.stream) != hipSuccess ||
      hipMemsetAsync(P.qil_dev, 0, cost_bytes, P.stream) != hipSuccess)
    return fail(BSA_ERR_HIP, "hipMemsetAsync failed");
  return BSA_OK;
}

// Everything after the features (host copy in P.feat): aggregates, regime,
// geometry and capacities, the arena, and the planning kernels.
static bsa_status finish_plan(Plan &P, bsa_lut_t lut, const uint8_t *mask, const int32_t *page_table,
                              Trace &tr) {
  // ---- aggregates and regime ----
  P.total_nnz = P.total_blocks = P.imb16 = 0;
  P.min_bq = P.min_bk = 1 << 30;
  for (int64_t bm = 0; bm < P.nbm; ++bm)
    for (int h = 0; h < P.Hq; ++h) {
      const int64_t nq = cdiv(P.Sq, P.bq[h]), nk = cdiv(P.Skv, P.bk[h]);
      const int64_t *f = &P.feat[(bm * P.Hq + h) * 4];
      P.total_nnz += f[0];
      P.total_blocks += nq * nk;
      if (f[0] > 0) P.imb16 = std::max(P.imb16, 16 * f[1] * nq / f[0]);
    }
  for (int h = 0; h < P.Hq; ++h) {
    P.min_bq = std::min<int64_t>(P.min_bq, P.bq[h]);
    P.min_bk = std::min<int64_t>(P.min_bk, P.bk[h]);
  }
  P.density_pm = P.total_blocks ? 1000 * P.total_nnz / P.total_blocks : 0;
  if (bsa_status s = choose_regime(P, lut)) return s;
  // Query-block interleave per head (128-row tiles merging 32- or 64-row
  // blocks, no union): the candidate s = 2^c with s * mq <= nq whose tiles
  // list the fewest key blocks, the smallest on ties.
  P.qil.assign(P.Hq, 1);
  for (int h = 0; h < P.Hq; ++h) {
    const int64_t bq = P.bq[h], nq = cdiv(P.Sq, bq);
    if (P.uni || P.rg.tq != 128 || bq >= 128 || bq < 32 || P.qil_cost.empty()) continue;
    const int64_t mq = 128 / bq;
    int64_t best = P.qil_cost[h * kQilCands];
    for (int c = 1; c < kQilCands && (int64_t(1) << c) * mq <= nq; ++c)
      if (P.qil_cost[h * kQilCands + c] < best) best = P.qil_cost[h * kQilCands + c], P.qil[h] = 1 << c;
  }
  // Key-block interleave per head (64-key tiles merging two 32-key blocks,
  // 128-row tiles merging 32- or 64-row blocks, bf16, one query head per kv
  // head, no union, paging or causal bound): given the head's query
  // interleave, the candidate s = 2^c with 2 s <= nk whose query tiles list
  // the fewest key tiles, the smallest on ties.
  P.kil.assign(P.Hq, 1);
  for (int h = 0; h < P.Hq; ++h) {
    const int64_t bq = P.bq[h], nk = cdiv(P.Skv, P.bk[h]);
    if (P.uni || P.paged || P.causal || P.dtype != BSA_BF16 || P.G != 1 || P.rg.tq != 128 ||
        P.rg.tk != 64 || P.bk[h] != 32 || bq >= 128 || bq < 32 || P.kil_cost.empty())
      continue;
    const int64_t *kc = &P.kil_cost[((size_t)h * kQilCands + __builtin_ctz(P.qil[h])) * kKilCands];
    int64_t best = kc[0];
    for (int c = 1; c < kKilCands && (int64_t(2) << c) <= nk; ++c)
      if (kc[c] < best) best = kc[c], P.kil[h] = 1 << c;
  }
  P.key_interleaved = false;
  for (int k : P.kil) P.key_interleaved |= k > 1;

  // ---- geometry and capacities ----
  const int tq = P.rg.tq, tk = P.rg.tk;
  P.tr = P.rg.pack ? tq / P.G : tq;
  P.nqt = cdiv(P.Sq, P.tr);
  P.nkt = cdiv(P.Skv, tk);
  P.nlists = P.uni ? P.nlb * P.Hkv : P.nlb * P.Hq * P.nqt;
  P.nrows = (int64_t)P.B * (P.rg.pack ? P.Hkv : P.Hq) * P.nqt;
  int64_t row_total;  // upper bound on the sum of row lengths
  if (P.uni) {
    P.ent_cap = P.nlists * P.nkt;
    row_total = P.nrows * P.nkt;
  } else {
    P.ent_cap = 0;
    for (int64_t lb = 0; lb < P.nlb; ++lb)
      for (int h = 0; h < P.Hq; ++h) {
        const int64_t bm = P.nbm == 1 ? 0 : lb;
        const int64_t sq = P.bq[h] > tq ? P.bq[h] / tq : 1, sk = P.bk[h] > tk ? P.bk[h] / tk : 1;
        P.ent_cap += std::min(P.nqt * P.nkt, P.feat[(bm * P.Hq + h) * 4] * sq * sk);
      }
    row_total = P.ent_cap * (P.B / P.nlb);
  }
  const int64_t split = P.rg.split;
  P.slot_cap = split > 0 ? std::min(2 * row_total / split + 1, P.nrows * cdiv(P.nkt, split)) : 0;
  P.comb_cap = split > 0 ? std::min(P.nrows, row_total / (split + 1) + 1) : 0;
  P.item_cap = P.nrows + P.slot_cap;
  // A tighter bound on the slots, from the longest row a head can have: a
  // split row of n entries takes ceil(n / split) slots, and a row of head h
  // has at most min(nkt, mq * (largest logical row of h) * sk) entries (mq
  // query blocks merged into the tile, each selected block covering sk key
  // tiles); a union row at most nkt. Sizes the forward's partial buffers.
  P.part_slots = 0;
  if (split > 0) {
    int64_t bound = 0;
    for (int h = 0; h < P.Hq; ++h) {
      if (P.uni && P.rg.pack && h % P.G) continue;  // a packed row serves the whole group
      int64_t maxlen = P.nkt;
      if (!P.uni) {
        int64_t maxrow = 0;
        for (int64_t bm = 0; bm < P.nbm; ++bm) maxrow = std::max(maxrow, P.feat[(bm * P.Hq + h) * 4 + 1]);
        const int64_t mq = P.bq[h] < tq ? tq / P.bq[h] : 1, sk = P.bk[h] > tk ? P.bk[h] / tk : 1;
        maxlen = std::min(P.nkt, mq * maxrow * sk);
      }
      if (maxlen > split) bound += (int64_t)P.B * P.nqt * cdiv(maxlen, split);
    }
    P.part_slots = std::min(P.slot_cap, bound);
  }
  const int64_t lim = (int64_t(1) << 31) - 2;
  if (P.ent_cap > lim || P.item_cap > lim || P.nrows > lim || P.nlists > lim)
    return fail(BSA_ERR_UNSUPPORTED, "plan too large (more than 2^31 entries or rows)");
  const size_t part_bytes = (size_t)P.slot_cap * tq * (P.D + 1) * sizeof(float);
  if (part_bytes > (size_t(64) << 30))
    return fail(BSA_ERR_UNSUPPORTED, "split threshold too small: partial buffers above 64 GiB");

  // ---- the arena, then the rest of the planning on the stream ----
  std::vector<std::pair<void **, size_t>> parts = {
      {(void **)&P.list_off, sizeof(int32_t) * (P.nlists + 1)},
      {(void **)&P.ent_kt, sizeof(int32_t) * std::max<int64_t>(P.ent_cap, 1)},
      {(void **)&P.ent_page, P.paged ? sizeof(int32_t) * std::max<int64_t>(P.ent_cap, 1) : 0},
      {(void **)&P.ent_live, sizeof(uint32_t) * std::max<int64_t>(P.ent_cap, 1)},
      {(void **)&P.row_ent, sizeof(int32_t) * 2 * std::max<int64_t>(P.nrows, 1)},
      {(void **)&P.items, sizeof(int32_t) * 4 * std::max<int64_t>(P.item_cap, 1)},
      {(void **)&P.comb, sizeof(int32_t) * 3 * std::max<int64_t>(P.comb_cap, 1)},
  };
  size_t total = 0;
  for (auto &pt : parts) total += aligned(pt.second);
  const size_t scratch = plan_scratch_bytes(P);
  total += scratch;
  if (plan_alloc(&P.arena, total, P.device, P.stream) != hipSuccess)
    return fail(BSA_ERR_OUT_OF_MEMORY, "device allocation of " + std::to_string(total) + " plan bytes failed");
  P.arena_bytes = total;
  uint8_t *ap = (uint8_t *)P.arena;
  for (auto &pt : parts) {
    *pt.first = pt.second ? ap : nullptr;
    ap += aligned(pt.second);
  }
  tr.mark("host planning");
  const bsa_status st = plan_build(P, mask, page_table, ap, scratch);
  if (st == BSA_OK) tr.mark("build");
  return st;
}

// BSA_LOG >= 2: the regime and the sizes of a new plan.
static void log_plan(const Plan &P, const char *how) {
  if (log_level() < 2) return;
  static const char *const kSched[] = {"local", "lpt", "dealt"};
  int interleaved = 0, key_interleaved = 0;
  for (int q : P.qil) interleaved += q > 1;
  for (int k : P.kil) key_interleaved += k > 1;
  log_msg(2,
          "plan (%s): B=%d Hq=%d Hkv=%d Sq=%lld Skv=%lld D=%d density %lld/1000 -> Tq=%d Tk=%d %s "
          "split=%d pack=%d; %lld rows, at most %lld items and %lld entries, %lld partial slots, "
          "%d heads interleaved (%d on the key side), %zu bytes",
          how, P.B, P.Hq, P.Hkv, (long long)P.Sq, (long long)P.Skv, P.D, (long long)P.density_pm, P.rg.tq,
          P.rg.tk, kSched[std::min(2, std::max(0, P.rg.sched))], P.rg.split, P.rg.pack, (long long)P.nrows,
          (long long)P.item_cap, (long long)P.ent_cap, (long long)P.part_slots, interleaved, key_interleaved, P.arena_bytes);
}

bsa_status bsa_plan(const bsa_problem *pr, const uint8_t *mask, const int32_t *page_table,
                    bsa_lut_t lut, void *stream, bsa_plan_t *out) {
  if (!out) return fail(BSA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (bsa_status s = check_problem(pr, mask, page_table)) return s;

  bsa_plan_s *p = new_plan(pr, stream);
  Plan &P = *p;
  auto bail = [&](bsa_status s) {
    free_plan(p);
    return s;
  };
  if (hipGetDevice(&P.device) != hipSuccess) return bail(fail(BSA_ERR_HIP, "hipGetDevice failed"));
  Trace tr("plan", P.stream);

  // ---- phase 1: features (one device-to-host read) ----
  if (bsa_status s = alloc_header(P, false, nullptr)) return bail(s);
  if (bsa_status s = plan_features(P, mask, page_table)) return bail(s);
  tr.mark("features");
  // The one read-back of planning: counters and mask features, into pinned
  // host memory (a direct DMA, no staging through pageable memory).
  const size_t feat_bytes = sizeof(int64_t) * 4 * P.nbm * P.Hq;
  const size_t cost_bytes = sizeof(int64_t) * kQilCands * (1 + kKilCands) * P.Hq;
  const size_t head_bytes = aligned(sizeof(int32_t) * CNT_N) + aligned(feat_bytes) + cost_bytes;
  PinnedBuf pin(head_bytes);
  if (!pin.p) return bail(fail(BSA_ERR_OUT_OF_MEMORY, "pinned host allocation failed"));
  if (hipMemcpyAsync(pin.p, P.counters, head_bytes, hipMemcpyDeviceToHost, P.stream) != hipSuccess ||
      hipStreamSynchronize(P.stream) != hipSuccess)
    return bail(fail(BSA_ERR_HIP, std::string("reading mask features failed: ") +
                                      hipGetErrorString(hipGetLastError())));
  const int32_t *hc = (const int32_t *)pin.p;
  const int64_t *hf = (const int64_t *)((const uint8_t *)pin.p + aligned(sizeof(int32_t) * CNT_N));
  P.feat.assign(hf, hf + feat_bytes / 8);
  const int64_t *hcost = (const int64_t *)((const uint8_t *)hf + aligned(feat_bytes));
  P.qil_cost.assign(hcost, hcost + kQilCands * P.Hq);
  P.kil_cost.assign(hcost + kQilCands * P.Hq, hcost + kQilCands * (1 + kKilCands) * P.Hq);
  if (hc[CNT_BADPAGE]) return bail(fail(BSA_ERR_INVALID_ARG, "page table entry outside [0, num_pages)"));
  tr.mark("read-back");

  if (bsa_status s = finish_plan(P, lut, mask, page_table, tr)) return bail(s);
  log_plan(P, "mask");
  tr.report("mask");
  *out = p;
  return BSA_OK;
}

bsa_status bsa_acsr_features(const bsa_problem *pr, const bsa_acsr_head *heads, int64_t *out) {
  if (!out) return fail(BSA_ERR_INVALID_ARG, "out is NULL");
  if (bsa_status s = check_problem(pr, nullptr, nullptr, false)) return s;
  if (bsa_status s = acsr_check(*pr, heads)) return s;
  acsr_features(*pr, heads, out);
  return BSA_OK;
}

bsa_status bsa_plan_acsr(const bsa_problem *pr, const bsa_acsr_head *heads, bsa_lut_t lut,
                         void *stream, bsa_plan_t *out) {
  if (!out) return fail(BSA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (bsa_status s = check_problem(pr, nullptr, nullptr, false)) return s;
  if (bsa_status s = acsr_check(*pr, heads)) return s;

  bsa_plan_s *p = new_plan(pr, stream);
  Plan &P = *p;
  auto bail = [&](bsa_status s) {
    free_plan(p);
    return s;
  };
  if (hipGetDevice(&P.device) != hipSuccess) return bail(fail(BSA_ERR_HIP, "hipGetDevice failed"));
  Trace tr("plan", P.stream);
  bsa_acsr_head *dev_heads = nullptr;
  if (bsa_status s = alloc_header(P, true, &dev_heads)) return bail(s);
  // features from the runs on the host: no read-back, so nothing blocks
  if (bsa_status s = plan_features_acsr(P, heads, dev_heads, *pr)) return bail(s);
  tr.mark("features");
  if (bsa_status s = finish_plan(P, lut, nullptr, nullptr, tr)) return bail(s);
  log_plan(P, "affine runs");
  tr.report("affine runs");
  *out = p;
  return BSA_OK;
}

static bsa_status forward_common(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                                 const bsa_tensor *v, bsa_tensor *o, float *lse, const float *k_scale,
                                 const float *v_scale, void *stream, bool no_alloc = false);

bsa_status bsa_forward(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                       bsa_tensor *o, float *lse, void *stream) {
  return forward_common(plan, q, k, v, o, lse, nullptr, nullptr, stream);
}

bsa_status bsa_forward_noalloc(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                               const bsa_tensor *v, bsa_tensor *o, float *lse, void *stream) {
  return forward_common(plan, q, k, v, o, lse, nullptr, nullptr, stream, true);
}

bsa_status bsa_forward_kv8(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                           const bsa_tensor *v, const float *k_scale, const float *v_scale,
                           bsa_tensor *o, float *lse, void *stream) {
  if (!plan) return fail(BSA_ERR_INVALID_ARG, "NULL plan or tensor");
  if (plan->dtype != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "FP8 K/V needs a bf16 plan (bf16 Q and O)");
  const bool any = plan->B * (int64_t)plan->Hq * plan->Sq > 0 && plan->Skv > 0;
  if (any && (!k_scale || !v_scale)) return fail(BSA_ERR_INVALID_ARG, "NULL k_scale or v_scale");
  return forward_common(plan, q, k, v, o, lse, k_scale, v_scale, stream);
}

static bsa_status forward_common(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                                 const bsa_tensor *v, bsa_tensor *o, float *lse, const float *k_scale,
                                 const float *v_scale, void *stream, bool no_alloc) {
  if (!plan || !q || !k || !v || !o) return fail(BSA_ERR_INVALID_ARG, "NULL plan or tensor");
  const Plan &P = *plan;
  const bool kv8 = k_scale != nullptr;
  const bool any_q = P.B * (int64_t)P.Hq * P.Sq > 0;
  if (any_q && (!q->data || !o->data || !lse)) return fail(BSA_ERR_INVALID_ARG, "NULL Q, O or LSE data");
  if (any_q && P.Skv > 0 && (!k->data || !v->data)) return fail(BSA_ERR_INVALID_ARG, "NULL K or V data");
  const int64_t esz = P.dtype == BSA_BF16 ? 2 : 4, vec = 16 / esz;
  for (const bsa_tensor *t : {q, k, v, (const bsa_tensor *)o}) {
    const int64_t tv = (kv8 && (t == k || t == v)) ? 16 : vec;  // e4m3: one byte per element
    if (((uintptr_t)t->data) % 16)
      return fail(BSA_ERR_INVALID_ARG, "tensor data must be 16-byte aligned");
    if (t->stride_b % tv || t->stride_h % tv || t->stride_s % tv)
      return fail(BSA_ERR_INVALID_ARG, "tensor strides must be multiples of 16 bytes");
    if (t->stride_b < 0 || t->stride_h < 0 || t->stride_s < 0)
      return fail(BSA_ERR_INVALID_ARG, "negative stride");
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != P.device)
    return fail(BSA_ERR_INVALID_ARG, "current device differs from the plan's device");
  AttnArgs a{};
  a.q = q->data, a.k = k->data, a.v = v->data, a.o = o->data, a.lse = lse;
  a.q_sb = q->stride_b, a.q_sh = q->stride_h, a.q_ss = q->stride_s;
  a.k_sb = k->stride_b, a.k_sh = k->stride_h, a.k_ss = k->stride_s;
  a.v_sb = v->stride_b, a.v_sh = v->stride_h, a.v_ss = v->stride_s;
  a.o_sb = o->stride_b, a.o_sh = o->stride_h, a.o_ss = o->stride_s;
  a.items = P.items, a.counters = P.counters, a.ent_kt = P.ent_kt, a.ent_page = P.ent_page;
  a.ent_live = P.ent_live, a.hm = P.hmeta;
  a.Sq = P.Sq, a.Skv = P.Skv, a.off = P.off, a.nqt = P.nqt;
  a.Hq = P.Hq, a.Hkv = P.Hkv, a.G = P.G, a.tq = P.rg.tq, a.tr = P.tr, a.pack = P.rg.pack;
  // The fp32 kernel lays packed tiles out head after head only (its combine
  // reads the same layout).
  if (P.dtype == BSA_F32 && a.pack) a.pack = 1;
  a.causal = P.causal, a.paged = P.paged, a.P = P.P, a.sched = P.rg.sched;
  a.scale_log2 = P.scale * 1.4426950408889634f;
  a.kv8 = kv8 ? 1 : 0, a.k_scale = k_scale, a.v_scale = v_scale;
  if (P.nrows == 0) return BSA_OK;
  // This call's scratch (work-queue counters, split-KV partials), taken from
  // the stream-ordered pool on the call's stream and returned after the
  // combine in stream order: calls on one plan that overlap in time (on any
  // streams) never share it.
  const FwdScratch fs = fwd_scratch_layout(P);
  hipStream_t s = (hipStream_t)stream;
  log_msg(3, "forward%s: plan %p, %lld rows, %zu scratch bytes, stream %p",
          no_alloc ? " (static scratch)" : kv8 ? " (fp8 K/V)" : "", (const void *)plan,
          (long long)P.nrows, fs.bytes, stream);
  Trace tr("forward", s);
  void *scratch = nullptr;
  if (no_alloc) {
    // The device's static scratch array instead of the pool.
    if (fs.bytes > kStaticScratchBytes)
      return fail(BSA_ERR_UNSUPPORTED, "this plan's forward needs " + std::to_string(fs.bytes) +
                                           " bytes of scratch; the static scratch holds " +
                                           std::to_string(kStaticScratchBytes));
    if (bsa_status st = static_scratch(P.device, &scratch)) return st;
    a.queue = (int32_t *)((uint8_t *)scratch + fs.queue_off);
    a.part_o = fs.part_o_off != fs.part_lse_off ? (float *)((uint8_t *)scratch + fs.part_o_off) : nullptr;
    a.part_lse = fs.part_lse_off != fs.bytes ? (float *)((uint8_t *)scratch + fs.part_lse_off) : nullptr;
    a.part_slots = P.part_slots;
    const bsa_status st = attention_launch(P, a, s);
    if (st == BSA_OK) tr.mark("attention"), tr.report("static scratch");
    return st;
  }
  const hipError_t e = plan_alloc(&scratch, fs.bytes, P.device, s);
  if (e != hipSuccess)
    return fail(BSA_ERR_OUT_OF_MEMORY, "forward scratch of " + std::to_string(fs.bytes) +
                                           " bytes: " + hipGetErrorString(e));
  uint8_t *sb = (uint8_t *)scratch;
  a.queue = (int32_t *)(sb + fs.queue_off);
  a.part_o = fs.part_o_off != fs.part_lse_off ? (float *)(sb + fs.part_o_off) : nullptr;
  a.part_lse = fs.part_lse_off != fs.bytes ? (float *)(sb + fs.part_lse_off) : nullptr;
  a.part_slots = P.part_slots;
  bsa_status st = attention_launch(P, a, s);
  plan_release(scratch, s);
  if (st == BSA_OK) st = note_stream_use(P, s);
  if (st == BSA_OK) tr.mark("attention"), tr.report(kv8 ? "fp8 K/V" : "");
  return st;
}

bsa_status bsa_backward(bsa_plan_t plan, const bsa_tensor *q, const bsa_tensor *k,
                        const bsa_tensor *v, const bsa_tensor *o, const float *lse,
                        const bsa_tensor *dout, bsa_tensor *dq, bsa_tensor *dk, bsa_tensor *dv,
                        void *stream) {
  if (!plan || !q || !k || !v || !o || !dout || !dq || !dk || !dv)
    return fail(BSA_ERR_INVALID_ARG, "NULL plan or tensor");
  const Plan &P = *plan;
  if (P.dtype != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "backward supports bf16 only");
  if (P.paged) return fail(BSA_ERR_UNSUPPORTED, "backward needs dense K/V (paged plans are not supported)");
  const bool any_q = P.B * (int64_t)P.Hq * P.Sq > 0, any_k = P.B * (int64_t)P.Hkv * P.Skv > 0;
  if (any_q && (!q->data || !o->data || !dout->data || !dq->data || !lse))
    return fail(BSA_ERR_INVALID_ARG, "NULL Q, O, dO, dQ or LSE data");
  if (any_k && (!k->data || !v->data || !dk->data || !dv->data))
    return fail(BSA_ERR_INVALID_ARG, "NULL K, V, dK or dV data");
  for (const bsa_tensor *t : {q, k, v, o, dout, (const bsa_tensor *)dq, (const bsa_tensor *)dk,
                              (const bsa_tensor *)dv}) {
    if (((uintptr_t)t->data) % 16)
      return fail(BSA_ERR_INVALID_ARG, "tensor data must be 16-byte aligned");
    if (t->stride_b % 8 || t->stride_h % 8 || t->stride_s % 8)
      return fail(BSA_ERR_INVALID_ARG, "tensor strides must be multiples of 16 bytes");
    if (t->stride_b < 0 || t->stride_h < 0 || t->stride_s < 0)
      return fail(BSA_ERR_INVALID_ARG, "negative stride");
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != P.device)
    return fail(BSA_ERR_INVALID_ARG, "current device differs from the plan's device");
  if (!any_q && !any_k) return BSA_OK;
  hipStream_t s = (hipStream_t)stream;
  BwdArgs a{};
  a.q = q->data, a.k = k->data, a.v = v->data, a.o = o->data, a.dout = dout->data, a.lse = lse;
  a.dq = dq->data, a.dk = dk->data, a.dv = dv->data;
  a.q_sb = q->stride_b, a.q_sh = q->stride_h, a.q_ss = q->stride_s;
  a.k_sb = k->stride_b, a.k_sh = k->stride_h, a.k_ss = k->stride_s;
  a.v_sb = v->stride_b, a.v_sh = v->stride_h, a.v_ss = v->stride_s;
  a.o_sb = o->stride_b, a.o_sh = o->stride_h, a.o_ss = o->stride_s;
  a.do_sb = dout->stride_b, a.do_sh = dout->stride_h, a.do_ss = dout->stride_s;
  a.dq_sb = dq->stride_b, a.dq_sh = dq->stride_h, a.dq_ss = dq->stride_s;
  a.dk_sb = dk->stride_b, a.dk_sh = dk->stride_h, a.dk_ss = dk->stride_s;
  a.dv_sb = dv->stride_b, a.dv_sh = dv->stride_h, a.dv_ss = dv->stride_s;
  a.row_ent = P.row_ent, a.list_off = P.list_off, a.ent_kt = P.ent_kt, a.ent_live = P.ent_live;
  a.hm = P.hmeta;
  a.Sq = P.Sq, a.Skv = P.Skv, a.off = P.off, a.nqt = P.nqt, a.nkt = P.nkt;
  a.Hq = P.Hq, a.Hkv = P.Hkv, a.G = P.G, a.tq = P.rg.tq, a.tr = P.tr, a.tk = P.rg.tk;
  {
    // 32-bit chunk addressing in the dK/dV kernel when a kv group's span of
    // Q and dO (in elements) fits in 31 bits.
    const int64_t lim = (int64_t)1 << 31;
    const int64_t qspan = (int64_t)(P.G - 1) * q->stride_h + (P.Sq - 1) * q->stride_s + P.D;
    const int64_t dspan = (int64_t)(P.G - 1) * dout->stride_h + (P.Sq - 1) * dout->stride_s + P.D;
    const bool ok = qspan < lim && dspan < lim && (int64_t)P.G * P.Sq < lim && q->stride_h < lim &&
                    q->stride_s < lim && dout->stride_h < lim && dout->stride_s < lim;
    a.grp32 = ok ? 1 : 0;
    a.q_sh32 = ok ? (int32_t)q->stride_h : 0, a.q_ss32 = ok ? (int32_t)q->stride_s : 0;
    a.do_sh32 = ok ? (int32_t)dout->stride_h : 0, a.do_ss32 = ok ? (int32_t)dout->stride_s : 0;
  }
  // (an interleaved forward regime has the same rows; the backward lays
  // them out head after head)
  a.pack = P.rg.pack ? 1 : 0, a.uni = P.uni, a.causal = P.causal, a.nlb = (int)P.nlb;
  a.scale = P.scale, a.scale_log2 = P.scale * 1.4426950408889634f;
  // Scratch, stream-ordered and returned after the kernels: Delta (dO . O per
  // query row) and the LSE in log2 units, both written by the dQ kernel for
  // the dK/dV kernel, and the key-major chunk index (groups of 128 keys) that
  // the dK/dV kernel walks.
  if (P.G > 255) return fail(BSA_ERR_UNSUPPORTED, "backward supports up to 255 query heads per kv head");
  const size_t row_bytes = (sizeof(float) * (size_t)std::max<int64_t>(P.B * (int64_t)P.Hq * P.Sq, 1) + 255) & ~(size_t)255;
  const size_t delta_bytes = 2 * row_bytes;  // Delta, then LSE * log2(e)
  const int nkt_per = 128 / P.rg.tk;
  const size_t index_bytes = plan_kv_index_bytes(P, nkt_per);
  log_msg(3, "backward: plan %p, %zu scratch bytes, stream %p", (const void *)plan,
          delta_bytes + index_bytes, stream);
  Trace tr("backward", s);
  void *scratch = nullptr;
  const hipError_t e = plan_alloc(&scratch, delta_bytes + index_bytes, P.device, s);
  if (e != hipSuccess) return fail(BSA_ERR_OUT_OF_MEMORY, std::string("backward scratch: ") + hipGetErrorString(e));
  a.delta = (float *)scratch;
  a.lse2 = (float *)((uint8_t *)scratch + row_bytes);
  KvIndex ix{};
  bsa_status st = plan_kv_index(P, nkt_per, (uint8_t *)scratch + delta_bytes, &ix, s);
  a.t_off = ix.off, a.t_q0 = ix.q0, a.t_meta = ix.meta, a.t_live = ix.live;
  if (st == BSA_OK) tr.mark("key index");
  if (st == BSA_OK) st = backward_launch(P, a, s);
  plan_release(scratch, s);
  if (st == BSA_OK) st = note_stream_use(P, s);
  if (st == BSA_OK) tr.mark("delta, dQ, dK/dV"), tr.report();
  return st;
}

bsa_status bsa_select_blocks(const bsa_problem *problem, const bsa_select_params *params,
                             const bsa_tensor *q, const bsa_tensor *k, const int32_t *page_table,
                             uint8_t *mask, void *stream) {
  if (!params || !q || !k) return fail(BSA_ERR_INVALID_ARG, "NULL params or tensor");
  if (bsa_status st = check_problem(problem, mask, page_table)) return st;
  if (problem->mask_batch_broadcast)
    return fail(BSA_ERR_INVALID_ARG, "block selection writes one mask per batch (mask_batch_broadcast = 0)");
  if (params->top_k < 0 || (params->top_k == 0 && (params->keep_tenths < 1 || params->keep_tenths > 10)))
    return fail(BSA_ERR_INVALID_ARG, "keep_tenths must be in [1, 10] when top_k is 0; top_k must be >= 0");
  const bool any = problem->seqlen_q > 0;
  if (any && (!q->data || (problem->seqlen_kv > 0 && !k->data)))
    return fail(BSA_ERR_INVALID_ARG, "NULL Q or K data");
  const int64_t vec = problem->dtype == BSA_BF16 ? 8 : 4;  // elements per 16 bytes
  for (const bsa_tensor *t : {q, k}) {
    if (t->stride_b < 0 || t->stride_h < 0 || t->stride_s < 0)
      return fail(BSA_ERR_INVALID_ARG, "negative stride");
    if (((uintptr_t)t->data) % 16 || t->stride_b % vec || t->stride_h % vec || t->stride_s % vec)
      return fail(BSA_ERR_INVALID_ARG, "tensor data and strides must be 16-byte aligned");
  }
  return select_blocks(*problem, params->keep_tenths, params->top_k, *q, *k, page_table, mask,
                       (hipStream_t)stream);
}

bsa_status bsa_plan_export(bsa_plan_t plan, void *host_buf, size_t *bytes) {
  if (!plan || !bytes) return fail(BSA_ERR_INVALID_ARG, "NULL plan or bytes");
  const Plan &P = *plan;
  int32_t cnt[CNT_N];
  HIP_TRY(hipStreamSynchronize(P.stream));
  HIP_TRY(hipMemcpy(cnt, P.counters, sizeof cnt, hipMemcpyDeviceToHost));
  const int64_t nent = cnt[CNT_ENT], nitems = cnt[CNT_ITEMS], nslots = cnt[CNT_SLOTS], ncomb = cnt[CNT_COMB];
  std::vector<uint8_t> img;
  auto put = [&](const void *src, size_t n) {
    const uint8_t *s = (const uint8_t *)src;
    img.insert(img.end(), s, s + n);
  };
  auto put_dev = [&](const void *src, size_t n) -> bsa_status {
    const size_t at = img.size();
    img.resize(at + n);
    if (n) HIP_TRY(hipMemcpy(img.data() + at, src, n, hipMemcpyDeviceToHost));
    return BSA_OK;
  };
  put("BSAPLAN1", 8);
  int64_t hdr[40] = {1, P.B, P.Hq, P.Hkv, P.Sq, P.Skv, P.D, P.dtype, P.causal, P.off, P.uni, P.paged,
                     P.P, P.pps, P.bcast, P.rg.tq, P.rg.tk, P.rg.sched, P.rg.split, P.rg.pack,
                     P.nqt, P.nkt, P.nlists, nent, P.nrows, nitems, nslots, ncomb, P.total_nnz,
                     P.total_blocks, P.density_pm, P.imb16, P.min_bq, P.min_bk, P.nlb};
  put(hdr, sizeof hdr);
  put(P.bq.data(), sizeof(int32_t) * P.Hq);
  put(P.bk.data(), sizeof(int32_t) * P.Hq);
  put(P.qil.data(), sizeof(int32_t) * P.Hq);
  put(P.kil.data(), sizeof(int32_t) * P.Hq);
  put(P.feat.data(), sizeof(int64_t) * P.feat.size());
  if (bsa_status s = put_dev(P.list_off, sizeof(int32_t) * (P.nlists + 1))) return s;
  if (bsa_status s = put_dev(P.ent_kt, sizeof(int32_t) * nent)) return s;
  if (P.paged)
    if (bsa_status s = put_dev(P.ent_page, sizeof(int32_t) * nent)) return s;
  if (bsa_status s = put_dev(P.ent_live, sizeof(uint32_t) * nent)) return s;
  if (bsa_status s = put_dev(P.row_ent, sizeof(int32_t) * 2 * P.nrows)) return s;
  if (bsa_status s = put_dev(P.items, sizeof(int32_t) * 4 * nitems)) return s;
  if (bsa_status s = put_dev(P.comb, sizeof(int32_t) * 3 * ncomb)) return s;
  if (host_buf) {
    if (*bytes < img.size()) {
      *bytes = img.size();
      return fail(BSA_ERR_INVALID_ARG, "export buffer too small");
    }
    std::memcpy(host_buf, img.data(), img.size());
  }
  *bytes = img.size();
  return BSA_OK;
}

bsa_status bsa_plan_stats(bsa_plan_t plan, bsa_plan_info *out) {
  if (!plan || !out) return fail(BSA_ERR_INVALID_ARG, "NULL plan or out");
  const Plan &P = *plan;
  int32_t cnt[CNT_N];
  HIP_TRY(hipStreamSynchronize(P.stream));
  HIP_TRY(hipMemcpy(cnt, P.counters, sizeof cnt, hipMemcpyDeviceToHost));
  std::vector<uint32_t> live(cnt[CNT_ENT]);
  if (!live.empty())
    HIP_TRY(hipMemcpy(live.data(), P.ent_live, sizeof(uint32_t) * live.size(), hipMemcpyDeviceToHost));
  std::memset(out, 0, sizeof *out);
  out->tile_q = P.rg.tq, out->tile_k = P.rg.tk, out->sched = P.rg.sched, out->split = P.rg.split;
  out->pack = P.rg.pack;
  out->rows = P.nrows, out->entries = cnt[CNT_ENT], out->items = cnt[CNT_ITEMS];
  out->partial_slots = cnt[CNT_SLOTS], out->combines = cnt[CNT_COMB];
  out->logical_nnz = P.total_nnz, out->logical_blocks = P.total_blocks;
  out->density_pm = P.density_pm, out->imbalance16 = P.imb16;
  double flops = 0;
  int64_t eff = 0;
  for (int b = 0; b < P.B; ++b)
    for (int h = 0; h < P.Hq; ++h) {
      const int64_t e = P.feat[((P.nbm == 1 ? 0 : b) * (int64_t)P.Hq + h) * 4 + 3];
      eff += e;
      flops += 4.0 * P.bq[h] * P.bk[h] * P.D * (double)e;
    }
  out->effective_blocks = eff, out->effective_flops = flops;
  int64_t bits = 0;
  for (uint32_t w : live) bits += __builtin_popcount(w);
  out->tile_live_subblocks = bits;
  std::vector<int32_t> items((size_t)4 * cnt[CNT_ITEMS]);
  if (!items.empty())
    HIP_TRY(hipMemcpy(items.data(), P.items, sizeof(int32_t) * items.size(), hipMemcpyDeviceToHost));
  int64_t executed = 0;
  for (size_t i = 0; i < items.size(); i += 4) executed += items[i + 2] - items[i + 1];
  out->executed_tiles = executed;
  out->partial_slot_bound = P.part_slots;
  return BSA_OK;
}

void bsa_plan_free(bsa_plan_t plan) { free_plan(plan); }

}  // extern "C"
