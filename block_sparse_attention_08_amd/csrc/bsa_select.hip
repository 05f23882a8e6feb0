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
#include <type_traits>

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

constexpr int kPoolRows = 16;  // rows of loads in flight per wave

// Columns c0 .. c0 + CPL - 1 of one row as fp32 (BF: bf16 elements).
template <int CPL, bool BF>
__device__ __forceinline__ void load_cols(const void *base, int64_t idx, float (&x)[CPL]) {
  if constexpr (BF && CPL == 2) {
    const uint32_t w = *(const uint32_t *)((const uint16_t *)base + idx);
    x[0] = __uint_as_float(w << 16), x[1] = __uint_as_float(w & 0xffff0000u);
  } else if constexpr (BF) {
    x[0] = __uint_as_float((uint32_t)((const uint16_t *)base)[idx] << 16);
  } else if constexpr (CPL == 2) {
    const float2 v = *(const float2 *)((const float *)base + idx);
    x[0] = v.x, x[1] = v.y;
  } else {
    x[0] = ((const float *)base)[idx];
  }
}

// Adds rows r0 .. r1-1 (row r at element off + r * stride) to the running
// column sums s, in ascending order, one fp32 addition each. One wave per
// block: lane l owns columns CPL l .. CPL l + CPL - 1 (CPL = D / 64, so a row
// is one contiguous read of the wave). kPoolRows rows are loaded before any
// is added (rows past the end load the last row again and are not added), so
// a wave waits once per kPoolRows rows.
template <int CPL, bool BF>
__device__ __forceinline__ void pool_rows(const void *base, int64_t off, int64_t stride, int64_t r0,
                                          int64_t r1, float (&s)[CPL]) {
  const int c0 = CPL * (threadIdx.x & 63);
  for (int64_t r = r0; r < r1; r += kPoolRows) {
    float x[kPoolRows][CPL];
#pragma unroll
    for (int v = 0; v < kPoolRows; ++v) load_cols<CPL, BF>(base, off + min(r + v, r1 - 1) * stride + c0, x[v]);
#pragma unroll
    for (int v = 0; v < kPoolRows; ++v)
      if (r + v < r1)
#pragma unroll
        for (int u = 0; u < CPL; ++u) s[u] = __fadd_rn(s[u], x[v][u]);
  }
}

// The block mean from its column sums over n rows (one fp32 division).
template <int CPL>
__device__ __forceinline__ void store_mean(const float (&s)[CPL], int64_t n, float *out) {
  const int c0 = CPL * (threadIdx.x & 63);
#pragma unroll
  for (int u = 0; u < CPL; ++u) out[c0 + u] = __fdiv_rn(s[u], (float)n);
}

// Query block means of one batch: one wave per (head, query block).
template <int CPL, bool BF>
__global__ __launch_bounds__(kSelThreads) void k_pool_q(SelArgs a, SelHeads hs) {
  const int b = blockIdx.y;
  const int x = blockIdx.x * (kSelThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (x >= a.qm_rows) return;
  const int2 hq = query_block(hs, x);
  const int h = hq.x, qb = hq.y;
  const int64_t i0 = (int64_t)qb * hs.bq[h];
  const int64_t i1 = min<int64_t>(a.Sq, i0 + hs.bq[h]);
  float s[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) s[u] = 0.0f;
  pool_rows<CPL, BF>(a.q, b * a.q_sb + h * a.q_sh, a.q_ss, i0, i1, s);
  store_mean<CPL>(s, i1 - i0, a.qm + ((int64_t)b * a.qm_rows + x) * a.D);
}

// Key block means of one batch: the key blocks of each distinct (kv group,
// block size) pair are pooled once, one wave per key block; a paged K is
// walked page by page (one page-table lookup per page, the sums carried
// across pages in row order).
template <int CPL, bool BF>
__global__ __launch_bounds__(kSelThreads) void k_pool_k(SelArgs a, SelHeads hs) {
  const int b = blockIdx.y;
  const int row = blockIdx.x * (kSelThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.km_rows) return;
  int h = 0;
  while (h < hs.n && !(hs.lead[h] && row >= hs.km_off[h] && row < hs.km_off[h] + hs.nkb[h])) ++h;
  if (h == hs.n) return;  // not reached: the rows are exactly the leaders' key blocks
  const int g = hs.g[h], bk = hs.bk[h], kb = row - hs.km_off[h];
  const int64_t j0 = (int64_t)kb * bk, j1 = min<int64_t>(a.Skv, j0 + bk);
  float s[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) s[u] = 0.0f;
  if (a.paged) {
    for (int64_t j = j0; j < j1;) {
      const int64_t pi = j / a.P, jend = min<int64_t>(j1, (pi + 1) * a.P);
      // entries outside [0, num_pages) are not followed (page 0 is read)
      int64_t page = a.page_table[(int64_t)b * a.pps + pi];
      page = (page < 0 || page >= a.npages) ? 0 : page;
      // key j' of this page sits at page * k_sb + (j' - pi P) * k_ss + g * k_sh
      pool_rows<CPL, BF>(a.k, page * a.k_sb + g * a.k_sh - pi * a.P * a.k_ss, a.k_ss, j, jend, s);
      j = jend;
    }
  } else {
    pool_rows<CPL, BF>(a.k, b * a.k_sb + g * a.k_sh, a.k_ss, j0, j1, s);
  }
  store_mean<CPL>(s, j1 - j0, a.km + ((int64_t)b * a.km_rows + row) * a.D);
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
      // four columns per load (pooled rows are D floats, 16-byte aligned),
      // the multiply-adds still in ascending column order
      const float4 *kr = (const float4 *)(km + (int64_t)i * a.D);
      float sc = 0.0f;
      for (int d4 = 0; d4 < a.D / 4; ++d4) {
        const float4 x = kr[d4];
        sc = __fmaf_rn(qm_s[4 * d4], x.x, sc);
        sc = __fmaf_rn(qm_s[4 * d4 + 1], x.y, sc);
        sc = __fmaf_rn(qm_s[4 * d4 + 2], x.z, sc);
        sc = __fmaf_rn(qm_s[4 * d4 + 3], x.w, sc);
      }
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
  const int per = kSelThreads / 64;  // blocks pooled per workgroup (one wave each)
  // (head_dim is 64 or 128: one or two columns per lane; bf16 or fp32)
  auto pool = [&](auto cpl, auto bf) {
    constexpr int CPL = decltype(cpl)::value;
    constexpr bool BF = decltype(bf)::value;
    hipLaunchKernelGGL((k_pool_q<CPL, BF>), dim3((unsigned)((qrows + per - 1) / per), (unsigned)B),
                       dim3(kSelThreads), 0, s, a, hs);
    if (krows > 0 && pr.seqlen_kv > 0)
      hipLaunchKernelGGL((k_pool_k<CPL, BF>), dim3((unsigned)((krows + per - 1) / per), (unsigned)B),
                         dim3(kSelThreads), 0, s, a, hs);
  };
  using One = std::integral_constant<int, 1>;
  using Two = std::integral_constant<int, 2>;
  if (a.D == 128) {
    if (a.bf16) pool(Two{}, std::true_type{});
    else pool(Two{}, std::false_type{});
  } else {
    if (a.bf16) pool(One{}, std::true_type{});
    else pool(One{}, std::false_type{});
  }
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
