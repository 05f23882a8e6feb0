// Block selection from pooled scores: the logical mask for bsa_plan, made on
// the GPU from Q and K (the step before the attention path).
//
// Hierarchical sparse attention picks the key/value blocks with the best
// coarse attention scores (DashAttention page, summary of NSA and InfLLMv2);
// CompactAttention (summary) uses the block mask of chunked prefill as a KV
// selection signal; Sol-Attn (summary) thresholds per query. Here the coarse
// score of (query block, key block) is the dot product of the two blocks'
// mean rows, and each query block keeps its best causally feasible key blocks.
//
// Floating point decides which blocks are kept, so every value is computed in
// one fixed fp32 order: a block mean sums its rows in ascending order (one
// fp32 addition each) and divides once; a score is a chain of fused
// multiply-adds over d ascending, starting from 0. Blocks are ranked by the
// total order of the scores' bit patterns, ties to the lower block index.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <string>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kSelThreads = 256;
constexpr int kMaxSelHeads = 64;
constexpr int kMaxSelKeyBlocks = 8192;

struct SelHeads {
  int32_t n;
  int32_t bq[kMaxSelHeads], bk[kMaxSelHeads], nqb[kMaxSelHeads], nkb[kMaxSelHeads];
  int32_t g[kMaxSelHeads];
  int32_t qm_off[kMaxSelHeads];  // row offset of the head's pooled query blocks (per batch)
  int32_t km_off[kMaxSelHeads];  // row offset of the pooled key blocks it reads (per batch)
  int32_t lead[kMaxSelHeads];    // 1: the head pools its group's key blocks at its block size
  int64_t mask_off[kMaxSelHeads];  // offset of the head's [nqb][nkb] mask within a batch
};

struct SelArgs {
  const void *q, *k;
  const int32_t *page_table;
  int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss;
  int64_t Sq, Skv, off;
  int32_t D, bf16, causal, paged, P, pps, npages;
  int32_t qm_rows, km_rows;  // pooled rows per batch
  int64_t mask_bytes;        // mask bytes per batch
  int32_t keep_tenths, top_k;
  int32_t kcap;  // LDS sort capacity (a power of two >= every head's key block count)
  float *qm, *km;
  uint8_t *mask;
};

__device__ __forceinline__ float load_el(const SelArgs &a, const void *base, int64_t idx) {
  if (a.bf16) return __uint_as_float((uint32_t)((const uint16_t *)base)[idx] << 16);
  return ((const float *)base)[idx];
}

// Query block x of the concatenation over heads: (head, block).
__device__ __forceinline__ int2 query_block(const SelHeads &hs, int x) {
  int h = 0;
  while (h + 1 < hs.n && x >= hs.qm_off[h] + hs.nqb[h]) ++h;
  return make_int2(h, x - hs.qm_off[h]);
}

// 8 consecutive elements (columns c0 .. c0+7 of one row) as fp32.
__device__ __forceinline__ void load8(const SelArgs &a, const void *base, int64_t idx, float (&x)[8]) {
  if (a.bf16) {
    const uint4 v = *(const uint4 *)((const uint16_t *)base + idx);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[2 * u] = __uint_as_float(w[u] << 16);
      x[2 * u + 1] = __uint_as_float(w[u] & 0xffff0000u);
    }
  } else {
    const float4 p = *(const float4 *)((const float *)base + idx);
    const float4 q = *(const float4 *)((const float *)base + idx + 4);
    x[0] = p.x, x[1] = p.y, x[2] = p.z, x[3] = p.w, x[4] = q.x, x[5] = q.y, x[6] = q.z, x[7] = q.w;
  }
}

// Block means: a lane owns 8 consecutive columns of one block and sums them
// over the block's rows in order (one fp32 addition per row and column), 4
// rows of loads in flight; a workgroup pools kSelThreads / (D / 8) blocks.
// row_at(r) gives the element index of column 0 of row r.
template <typename RowAt>
__device__ __forceinline__ void pool8(const SelArgs &a, const void *base, int64_t r0, int64_t r1, int c0,
                                      RowAt row_at, float *out) {
  float s[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) s[u] = 0.0f;
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    float x[4][8];
#pragma unroll
    for (int v = 0; v < 4; ++v) load8(a, base, row_at(r + v) + c0, x[v]);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int u = 0; u < 8; ++u) s[u] = __fadd_rn(s[u], x[v][u]);
  }
  for (; r < r1; ++r) {
    float x[8];
    load8(a, base, row_at(r) + c0, x);
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] = __fadd_rn(s[u], x[u]);
  }
  const float n = (float)(r1 - r0);
#pragma unroll
  for (int u = 0; u < 8; ++u) out[c0 + u] = __fdiv_rn(s[u], n);
}

// Query block means of one batch: block x of the concatenation over heads.
__global__ __launch_bounds__(kSelThreads) void k_pool_q(SelArgs a, SelHeads hs) {
  const int b = blockIdx.y;
  const int lanes = a.D / 8, per = kSelThreads / lanes;
  const int x = blockIdx.x * per + threadIdx.x / lanes;
  if (threadIdx.x >= per * lanes || x >= a.qm_rows) return;
  const int2 hq = query_block(hs, x);
  const int h = hq.x, qb = hq.y;
  const int64_t i0 = (int64_t)qb * hs.bq[h];
  const int64_t i1 = min<int64_t>(a.Sq, i0 + hs.bq[h]);
  const int64_t base = b * a.q_sb + h * a.q_sh;
  pool8(a, a.q, i0, i1, 8 * (threadIdx.x % lanes), [&](int64_t i) { return base + i * a.q_ss; },
        a.qm + ((int64_t)b * a.qm_rows + x) * a.D);
}

// Key block means of one batch: the key blocks of each distinct (kv group,
// block size) pair are pooled once, through the page table when K is paged.
__global__ __launch_bounds__(kSelThreads) void k_pool_k(SelArgs a, SelHeads hs) {
  const int b = blockIdx.y;
  const int lanes = a.D / 8, per = kSelThreads / lanes;
  const int row = blockIdx.x * per + threadIdx.x / lanes;
  if (threadIdx.x >= per * lanes || row >= a.km_rows) return;
  int h = 0;
  while (h < hs.n && !(hs.lead[h] && row >= hs.km_off[h] && row < hs.km_off[h] + hs.nkb[h])) ++h;
  if (h == hs.n) return;  // not reached: the rows are exactly the leaders' key blocks
  const int g = hs.g[h], bk = hs.bk[h], kb = row - hs.km_off[h];
  const int64_t j0 = (int64_t)kb * bk, j1 = min<int64_t>(a.Skv, j0 + bk);
  auto row_at = [&](int64_t j) -> int64_t {
    if (a.paged) {
      // entries outside [0, num_pages) are not followed (page 0 is read)
      int64_t page = a.page_table[(int64_t)b * a.pps + j / a.P];
      page = (page < 0 || page >= a.npages) ? 0 : page;
      return page * a.k_sb + (j % a.P) * a.k_ss + g * a.k_sh;
    }
    return b * a.k_sb + g * a.k_sh + j * a.k_ss;
  };
  pool8(a, a.k, j0, j1, 8 * (threadIdx.x % lanes), row_at, a.km + ((int64_t)b * a.km_rows + row) * a.D);
}

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per (batch, head, query block): scores of the causally
// feasible key blocks (a prefix of the block indices), a descending bitonic
// sort of (score key << 32 | ~block) in LDS, and the mask row.
__global__ __launch_bounds__(kSelThreads) void k_select(SelArgs a, SelHeads hs) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.y;
  const int2 hq = query_block(hs, blockIdx.x);
  const int h = hq.x, qb = hq.y;
  const int nkb = hs.nkb[h], bk = hs.bk[h];
  const int64_t last_q = min<int64_t>(a.Sq, (int64_t)(qb + 1) * hs.bq[h]) - 1;
  int ncand = nkb;
  if (a.causal) {
    const int64_t lim = last_q + a.off;  // a key block is feasible if its first key <= lim
    ncand = lim < 0 ? 0 : (int)min<int64_t>(nkb, lim / bk + 1);
  }
  int npow = 1;
  while (npow < ncand) npow <<= 1;
  unsigned long long *keys = (unsigned long long *)smem;
  float *qm_s = (float *)(keys + a.kcap);
  uint8_t *sel = (uint8_t *)(qm_s + 256);

  const float *qm = a.qm + ((int64_t)b * a.qm_rows + hs.qm_off[h] + qb) * a.D;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) qm_s[d] = qm[d];
  for (int i = threadIdx.x; i < nkb; i += blockDim.x) sel[i] = 0;
  __syncthreads();
  const float *km = a.km + ((int64_t)b * a.km_rows + hs.km_off[h]) * a.D;
  for (int i = threadIdx.x; i < npow; i += blockDim.x) {
    unsigned long long key = 0;  // padding sorts last
    if (i < ncand) {
      const float *kr = km + (int64_t)i * a.D;
      float sc = 0.0f;
      for (int d = 0; d < a.D; ++d) sc = __fmaf_rn(qm_s[d], kr[d], sc);
      key = ((unsigned long long)order_key(sc) << 32) | (0xffffffffu - (uint32_t)i);
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int kk = 2; kk <= npow; kk <<= 1)
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < npow; i += blockDim.x) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const unsigned long long x = keys[i], y = keys[ixj];
          const bool desc = (i & kk) == 0;
          if (desc ? (x < y) : (x > y)) keys[i] = y, keys[ixj] = x;
        }
      }
      __syncthreads();
    }
  const int keep = a.top_k > 0 ? min(a.top_k, ncand) : (int)(((int64_t)ncand * a.keep_tenths + 9) / 10);
  for (int i = threadIdx.x; i < keep; i += blockDim.x)
    sel[0xffffffffu - (uint32_t)(keys[i] & 0xffffffffull)] = 1;
  __syncthreads();
  uint8_t *row = a.mask + (int64_t)b * a.mask_bytes + hs.mask_off[h] + (int64_t)qb * nkb;
  for (int i = threadIdx.x; i < nkb; i += blockDim.x) row[i] = sel[i];
}

}  // namespace

bsa_status select_blocks(const bsa_problem &pr, int keep_tenths, int top_k, const bsa_tensor &q,
                         const bsa_tensor &k, const int32_t *page_table, uint8_t *mask,
                         hipStream_t s) {
  const int Hq = pr.num_q_heads, G = pr.num_q_heads / pr.num_kv_heads;
  if (Hq > kMaxSelHeads) return fail(BSA_ERR_UNSUPPORTED, "block selection supports up to 64 query heads");
  if (pr.head_dim > 256) return fail(BSA_ERR_UNSUPPORTED, "block selection supports head_dim <= 256");
  SelHeads hs{};
  hs.n = Hq;
  int32_t qrows = 0, krows = 0, maxk = 1;
  int64_t mbytes = 0;
  for (int h = 0; h < Hq; ++h) {
    const int64_t nq = (pr.seqlen_q + pr.block_q[h] - 1) / pr.block_q[h];
    const int64_t nk = (pr.seqlen_kv + pr.block_k[h] - 1) / pr.block_k[h];
    if (nk > kMaxSelKeyBlocks)
      return fail(BSA_ERR_UNSUPPORTED, "block selection supports up to 8192 key blocks per head");
    if ((int64_t)qrows + nq > INT32_MAX / 2 || (int64_t)krows + nk > INT32_MAX / 2)
      return fail(BSA_ERR_UNSUPPORTED, "too many blocks");
    hs.bq[h] = pr.block_q[h], hs.bk[h] = pr.block_k[h], hs.nqb[h] = (int32_t)nq, hs.nkb[h] = (int32_t)nk;
    hs.g[h] = h / G;
    hs.qm_off[h] = qrows;
    qrows += (int32_t)nq;
    hs.mask_off[h] = mbytes;
    mbytes += nq * nk;
    maxk = std::max<int32_t>(maxk, (int32_t)nk);
    // pooled key blocks are shared by the heads of a group with the same block size
    int lead = h;
    for (int h2 = (h / G) * G; h2 < h; ++h2)
      if (pr.block_k[h2] == pr.block_k[h]) {
        lead = h2;
        break;
      }
    hs.lead[h] = lead == h;
    if (lead != h) {
      hs.km_off[h] = hs.km_off[lead];
    } else {
      hs.km_off[h] = krows;
      krows += (int32_t)nk;
    }
  }
  const int64_t B = pr.batch;
  if (B == 0 || qrows == 0) return BSA_OK;
  int kcap = 1;
  while (kcap < maxk) kcap <<= 1;

  // Pooled rows live in scratch from the stream-ordered pool, freed in order.
  const size_t qm_bytes = sizeof(float) * (size_t)B * qrows * pr.head_dim;
  const size_t km_bytes = sizeof(float) * (size_t)B * std::max(krows, 1) * pr.head_dim;
  void *scratch = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BSA_ERR_HIP, "hipGetDevice failed");
  if (plan_alloc(&scratch, ((qm_bytes + 255) & ~size_t(255)) + km_bytes, dev, s) != hipSuccess)
    return fail(BSA_ERR_OUT_OF_MEMORY, "device allocation of block-selection scratch failed");
  SelArgs a{};
  a.q = q.data, a.k = k.data, a.page_table = page_table;
  a.q_sb = q.stride_b, a.q_sh = q.stride_h, a.q_ss = q.stride_s;
  a.k_sb = k.stride_b, a.k_sh = k.stride_h, a.k_ss = k.stride_s;
  a.Sq = pr.seqlen_q, a.Skv = pr.seqlen_kv, a.off = pr.causal_kv_offset;
  a.D = pr.head_dim, a.bf16 = pr.dtype == BSA_BF16, a.causal = pr.causal, a.paged = pr.paged;
  a.P = pr.page_size, a.pps = pr.pages_per_seq, a.npages = pr.num_pages;
  a.qm_rows = qrows, a.km_rows = krows, a.mask_bytes = mbytes;
  a.keep_tenths = keep_tenths, a.top_k = top_k, a.kcap = kcap;
  a.qm = (float *)scratch;
  a.km = (float *)((uint8_t *)scratch + ((qm_bytes + 255) & ~size_t(255)));
  a.mask = mask;
  const int per = kSelThreads / (pr.head_dim / 8);  // blocks pooled per workgroup
  hipLaunchKernelGGL(k_pool_q, dim3((unsigned)((qrows + per - 1) / per), (unsigned)B), dim3(kSelThreads),
                     0, s, a, hs);
  if (krows > 0 && pr.seqlen_kv > 0)
    hipLaunchKernelGGL(k_pool_k, dim3((unsigned)((krows + per - 1) / per), (unsigned)B), dim3(kSelThreads),
                       0, s, a, hs);
  const size_t lds = sizeof(unsigned long long) * kcap + sizeof(float) * 256 + ((maxk + 15) & ~15);
  hipError_t e = hipSuccess;
  if (lds > (size_t(64) << 10))
    e = hipFuncSetAttribute((const void *)k_select, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_select, dim3((unsigned)qrows, (unsigned)B), dim3(kSelThreads), lds, s, a, hs);
    e = hipGetLastError();
  }
  plan_release(scratch, s);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, std::string("block selection launch failed: ") + hipGetErrorString(e));
  return BSA_OK;
}

}  // namespace bsa
