// Mask-to-tile planner kernels for gfx950.
//
// Tessera ("Decoupling Logical Masks from GPU Execution for Dynamic
// Block-Sparse Attention", abstract) splits the work of a block-sparse request
// into a physical mapping layer (keep, merge or subdivide logical blocks into
// physical tiles while preserving the selected interactions), a task
// organization layer (group and schedule tiles into GPU tasks) and a
// profile-built lookup table that picks the execution plan. CompactAttention
// (summary) builds per-group KV block tables from the union of a group's
// selections and runs them zero-copy over a paged cache.
//
// Everything here is integer work done with wave-level ballots, prefix
// popcounts and a three-phase exclusive scan, so the plan is bit-for-bit
// reproducible: integer atomics only ever produce order-independent sums and
// maxima, every list is emitted in ascending key-tile order, and the
// longest-first order is a stable counting sort.
#include "bsa_internal.h"

#include <algorithm>
#include <cstring>
#include <type_traits>

namespace bsa {
namespace {

constexpr int kThreads = 256;
constexpr int kScanBlock = 1024;  // elements per scan workgroup (4 per thread)
constexpr int kLptKeys = 1024;    // longest-first key = min(item length, 1023)
constexpr int kRowBatch = 8;      // mask loads in flight per lane (k_row_features)
constexpr int kMapBatch = 8;      // key tiles per lane tested together (k_map)

#define HIP_TRY(expr)                                                          \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess)                                                      \
      return fail(BSA_ERR_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

__device__ __forceinline__ int wave_sum(int x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int64_t lo_mask(int lane) { return (int64_t)((1ull << lane) - 1ull); }

// The n lowest bits set (none for n <= 0, all for n >= 64).
__device__ __forceinline__ unsigned long long prefix_mask(int64_t n) {
  return n <= 0 ? 0ull : (n >= 64 ? ~0ull : (1ull << n) - 1ull);
}

// Key-block bits to key-tile bits when a block spans 2^sh tiles: the low
// 64 >> sh bits of x, each repeated 2^sh times (sh >= 6: bit 0 for all 64).
__device__ __forceinline__ unsigned long long spread_bits(unsigned long long x, int sh) {
  if (sh >= 6) return (x & 1ull) ? ~0ull : 0ull;
  x &= sh == 0 ? ~0ull : (1ull << (64 >> sh)) - 1ull;
  for (int i = 0; i < sh; ++i) {  // each pass doubles every bit of the low 32
    x = (x | (x << 16)) & 0x0000FFFF0000FFFFull;
    x = (x | (x << 8)) & 0x00FF00FF00FF00FFull;
    x = (x | (x << 4)) & 0x0F0F0F0F0F0F0F0Full;
    x = (x | (x << 2)) & 0x3333333333333333ull;
    x = (x | (x << 1)) & 0x5555555555555555ull;
    x |= x << 1;
  }
  return x;
}

// -------------------------------------------------------------------------
// Mask features and group union
// -------------------------------------------------------------------------

// Group union (CompactAttention: query-block union plus intra-group union):
// U[bm][g][kb] = 1 iff some head of group g selects key block kb in some row.
__global__ void k_union(const uint8_t *__restrict__ mask, const HeadMeta *__restrict__ hm,
                        int64_t mask_bstride, int Hkv, int G, int nbm, int64_t unkb,
                        uint8_t *__restrict__ U) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nbm * Hkv * unkb) return;
  const int64_t kb = idx % unkb, bg = idx / unkb;
  const int g = (int)(bg % Hkv), bm = (int)(bg / Hkv);
  uint8_t u = 0;
  for (int hh = 0; hh < G && !u; ++hh) {
    const HeadMeta m = hm[g * G + hh];
    if (kb >= m.nkb) continue;
    const uint8_t *col = mask + bm * mask_bstride + m.mask_off + kb;
    for (int64_t qb = 0; qb < m.nqb; ++qb)
      if (col[qb * m.nkb]) {
        u = 1;
        break;
      }
  }
  U[idx] = u;
}

// One wave per logical row: popcount, and the count of effective blocks (the
// union's in union mode) that the causal bound can reach, written per row
// (no atomics, so no contention and no clearing).
__global__ void k_row_features(const uint8_t *__restrict__ mask, const HeadMeta *__restrict__ hm,
                               int Hq, int Hkv, int G, int nbm, int64_t rows_per_bm,
                               int64_t mask_bstride, const uint8_t *__restrict__ U, int64_t unkb,
                               int causal, int64_t off, int64_t Sq, int32_t *__restrict__ rowf,
                               unsigned long long *__restrict__ bits, int64_t bits_per_bm) {
  const int lane = threadIdx.x & 63;
  // one row per wave: the index is wave-uniform, so the head search, the
  // head metadata and the row's base address are scalar
  const int64_t wv = blockIdx.x * (int64_t)(blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv >= nbm * rows_per_bm) return;
  const int bm = (int)(wv / rows_per_bm);
  const int64_t r = wv % rows_per_bm;
  int lo = 0, hi = Hq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (hm[mid].row_off <= r) lo = mid;
    else hi = mid - 1;
  }
  const int h = lo;
  const HeadMeta m = hm[h];
  const int64_t qb = r - m.row_off;
  const uint8_t *row = mask + bm * mask_bstride + m.mask_off + qb * m.nkb;
  const uint8_t *urow = U ? U + ((int64_t)bm * Hkv + h / G) * unkb : nullptr;
  const int64_t qlast = min(Sq, (qb + 1) * (int64_t)m.bq) - 1;
  int64_t kbmax = m.nkb - 1;
  if (causal) kbmax = (qlast + off) < 0 ? -1 : (qlast + off) / m.bk;
  int cnt = 0, eff = 0;
  // the row as a bitmap, one 64-bit word per 64 key blocks (when kept)
  unsigned long long *brow = bits ? bits + bm * bits_per_bm + m.bits_off + qb * ((m.nkb + 63) >> 6) : nullptr;
  const int nkb = (int)m.nkb, kbm = (int)min<int64_t>(kbmax, nkb);  // key blocks are below 2^31
  // kRowBatch mask bytes per lane are loaded before any is tested, so a wave
  // waits once per 64 * kRowBatch key blocks rather than once per 64 (the
  // kernel is bound by those waits). The loads take a clamped index and are
  // tested afterwards, with no branch between them (a load under a lane
  // condition would be waited for at once); lane u stores the batch's word u.
  auto scan_row = [&](auto has_union) {
    constexpr bool HU = decltype(has_union)::value;
    for (int kb0 = 0; kb0 < nkb; kb0 += 64 * kRowBatch) {
      uint8_t v[kRowBatch], uv[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const uint32_t kc = (uint32_t)min(kb0 + 64 * u + lane, nkb - 1);
        v[u] = row[kc];
        if constexpr (HU) uv[u] = urow[kc];
      }
      unsigned long long mine = 0;
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int kb = kb0 + 64 * u + lane;
        const int sel = kb < nkb && v[u] != 0;
        cnt += sel;
        const int es = HU ? (kb < nkb && uv[u] != 0) : sel;
        eff += es && kb <= kbm;
        const unsigned long long word = __ballot(sel);
        if (lane == u) mine = word;
      }
      if (brow && lane < kRowBatch && kb0 + 64 * lane < nkb) brow[(kb0 >> 6) + lane] = mine;
    }
  };
  if (urow) scan_row(std::true_type{});
  else scan_row(std::false_type{});
  cnt = wave_sum(cnt);
  eff = wave_sum(eff);
  if (lane == 0) {
    rowf[2 * wv] = cnt;
    rowf[2 * wv + 1] = eff;
  }
}

// One workgroup per (mask batch, head): nnz (sum), max row (max), empty rows
// (count), effective blocks (sum) over the head's rows.
__global__ void k_head_features(const int32_t *__restrict__ rowf, const HeadMeta *__restrict__ hm,
                                int Hq, int64_t rows_per_bm, unsigned long long *__restrict__ feat) {
  __shared__ unsigned long long red[4][kThreads / 64];
  const int bm = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const HeadMeta m = hm[h];
  const int32_t *rf = rowf + 2 * ((int64_t)bm * rows_per_bm + m.row_off);
  unsigned long long nnz = 0, mx = 0, empty = 0, eff = 0;
  for (int64_t q = threadIdx.x; q < m.nqb; q += kThreads) {
    const unsigned long long c = (unsigned)rf[2 * q];
    nnz += c;
    mx = c > mx ? c : mx;
    empty += c == 0;
    eff += (unsigned)rf[2 * q + 1];
  }
  for (int o = 32; o > 0; o >>= 1) {
    nnz += __shfl_xor(nnz, o);
    const unsigned long long t = __shfl_xor(mx, o);
    mx = t > mx ? t : mx;
    empty += __shfl_xor(empty, o);
    eff += __shfl_xor(eff, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[0][w] = nnz, red[1][w] = mx, red[2][w] = empty, red[3][w] = eff;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long f[4] = {0, 0, 0, 0};
    for (int i = 0; i < kThreads / 64; ++i) {
      f[0] += red[0][i];
      f[1] = red[1][i] > f[1] ? red[1][i] : f[1];
      f[2] += red[2][i];
      f[3] += red[3][i];
    }
    for (int k = 0; k < 4; ++k) feat[(int64_t)blockIdx.x * 4 + k] = f[k];
  }
}

// Query-block interleave costs: one wave per (head, candidate interleave
// s = 2^c) and 16 of its 128-row tiles (over the mask batches); it counts
// the key blocks that some query block of a tile selects (the mask as given,
// from the row bitmaps) and adds the sum to cost[h][c] (integer atomics: the
// sums do not depend on their order). Only
// heads whose 32- or 64-row blocks merge into 128-row tiles, and only
// candidates with s * mq <= nq, are counted; the host picks the cheapest.
// With keys_ok (no causal bound, no paging), heads of 32-key blocks also
// count, per key interleave s' = 2^c' with 2 s' <= nk, the 64-key tiles in
// which the tile selects a block, into kcost[h][c][c'].
constexpr int kCostTiles = 16;  // tiles per wave of k_qil_cost (one atomic per wave and counter)
__global__ void k_qil_cost(const unsigned long long *__restrict__ bits, int64_t bits_per_bm,
                           const HeadMeta *__restrict__ hm, int Hq, int nbm,
                           const int64_t *__restrict__ wave_off, int64_t nwaves,
                           unsigned long long *__restrict__ cost, int keys_ok,
                           unsigned long long *__restrict__ kcost) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  if (wv >= nwaves) return;
  // wave_off[h * kQilCands + c] = first wave of (head, candidate), over all mask batches
  int lo = 0, hi = Hq * kQilCands - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wave_off[mid] <= wv) lo = mid;
    else hi = mid - 1;
  }
  const int h = lo / kQilCands, c = lo % kQilCands;
  const HeadMeta m = hm[h];
  const int lm = 7 - __builtin_ctz(m.bq);  // 128-row tiles
  const int64_t ntiles = ((int64_t)m.nqb + (1 << lm) - 1) >> lm;
  const int64_t words = (m.nkb + 63) >> 6;
  const bool keys = keys_ok && m.bk == 32;
  int cnt = 0;
  int kc[kKilCands] = {0, 0, 0, 0};
  // tiles kCostTiles * (this wave's index within its (head, candidate)) ..,
  // numbered over the mask batches
  const int64_t k0 = (wv - wave_off[lo]) * kCostTiles;
  for (int64_t k = k0; k < k0 + kCostTiles; ++k) {
    const int bm = (int)(k / ntiles);
    const int64_t t = k % ntiles;
    if (bm >= nbm) break;
    const unsigned long long *hb = bits + bm * bits_per_bm + m.bits_off;
    // the tile's row bitmaps (at most 4: 32- or 64-row blocks in 128-row tiles)
    const unsigned long long *rp[4];
    for (int iq = 0; iq < 4; ++iq) {
      const int64_t qb = iq < (1 << lm) ? qblock_of(t, iq, c, lm, m.nqb) : m.nqb;
      rp[iq] = qb < m.nqb ? hb + qb * words : nullptr;
    }
    for (int64_t w = lane; w < words; w += 64) {
      // key blocks 64 w .. 64 w + 63 that some query block of the tile selects
      unsigned long long x = 0;
      for (int iq = 0; iq < 4; ++iq)
        if (rp[iq]) x |= rp[iq][w];
      cnt += __popcll(x);
      if (keys) {
        // 64-key tiles of two 32-key blocks under key interleave s = 2^ck: in
        // a full group of 2s blocks, tile j holds blocks j and j + s (bit j of
        // x | x >> s, j mod 2s < s); past the last full group, consecutive
        // pairs. 2s divides 64, so a group never straddles two words.
        constexpr unsigned long long kPat[kKilCands] = {0x5555555555555555ull, 0x3333333333333333ull,
                                                        0x0F0F0F0F0F0F0F0Full, 0x00FF00FF00FF00FFull};
#pragma unroll
        for (int ck = 0; ck < kKilCands; ++ck) {
          if ((int64_t(2) << ck) > m.nkb) break;
          const int64_t fullend = (m.nkb >> (ck + 1)) << (ck + 1);  // blocks in full groups
          const int64_t lo64 = w << 6;
          const unsigned long long fm = fullend <= lo64 ? 0ull
                                        : (fullend >= lo64 + 64 ? ~0ull : ((1ull << (fullend - lo64)) - 1ull));
          const unsigned long long yf = (x | (x >> (1 << ck))) & kPat[ck] & fm;
          const unsigned long long yt = (x | (x >> 1)) & kPat[0] & ~fm;
          kc[ck] += __popcll(yf) + __popcll(yt);
        }
      }
    }
  }
  cnt = wave_sum(cnt);
  if (lane == 0 && cnt) atomicAdd(&cost[h * kQilCands + c], (unsigned long long)cnt);
  if (!keys) return;
#pragma unroll
  for (int ck = 0; ck < kKilCands; ++ck) {
    const int v = wave_sum(kc[ck]);
    if (lane == 0 && v) atomicAdd(&kcost[(h * kQilCands + c) * kKilCands + ck], (unsigned long long)v);
  }
}

// Count page-table entries that the keys [0, Skv) use and that point outside
// the pool.
__global__ void k_check_pages(const int32_t *__restrict__ table, int B, int pps, int64_t used,
                              int npages, int32_t *__restrict__ counters) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * used) return;
  const int32_t pg = table[(i / used) * pps + i % used];
  if (pg < 0 || pg >= npages) atomicAdd(&counters[CNT_BADPAGE], 1);
}

// -------------------------------------------------------------------------
// Physical mapping (keep / merge / subdivide) with live bits
// -------------------------------------------------------------------------

struct MapArgs {
  const uint8_t *mask, *U;
  const bsa_acsr_head *acsr;  // affine row descriptors in place of mask bytes (ACSR plans)
  const unsigned long long *bits;  // row bitmaps of the features pass (mask plans without union)
  int64_t bits_per_bm;
  const HeadMeta *hm;
  const int32_t *page_table;
  int64_t mask_bstride, unkb, Sq, off, nqt, nkt, nlists;
  int32_t Hq, Hkv, G, bcast, uni, paged, causal, tq, tk, pps, P;
  int32_t *list_len;
  const int32_t *list_off;
  int32_t *ent_kt, *ent_page;
  uint32_t *ent_live;
};

// Live bits of physical tile (qt, kt) for list head h: bit (iq * mk + ik) is
// set iff the logical block covering query sub-block iq and key sub-block ik
// is selected (by the union in union mode, by one of the head's affine runs
// in an ACSR plan) and, when causal, the sub-block's first key is not after
// its last query.
__device__ __forceinline__ uint32_t live_bits(const MapArgs &a, int bm, int h, int g, int64_t qt,
                                              int64_t kt) {
  const HeadMeta m = a.hm[h];
  const int64_t bq = m.bq, bk = m.bk;
  // Block and tile sizes are powers of two: index arithmetic by shifts (a
  // 64-bit division per lane would dominate the kernel).
  const int lbq = __builtin_ctz(m.bq), lbk = __builtin_ctz(m.bk);
  const int ltq = __builtin_ctz(a.tq), ltk = __builtin_ctz(a.tk);
  const int mq = (!a.uni && bq < a.tq) ? 1 << (ltq - lbq) : 1;
  const int mk = bk < a.tk ? 1 << (ltk - lbk) : 1;
  const int64_t aq = bq < a.tq ? bq : a.tq, ak = bk < a.tk ? bk : a.tk;
  const uint8_t *mb = a.acsr ? nullptr : a.mask + bm * a.mask_bstride + m.mask_off;
  const uint8_t *u = a.uni ? a.U + ((int64_t)bm * a.Hkv + g) * a.unkb : nullptr;
  uint32_t live = 0;
  for (int iq = 0; iq < mq; ++iq) {
    const int64_t qb = bq < a.tq ? qblock_of(qt, iq, m.lqil, ltq - lbq, m.nqb) : (qt << ltq) >> lbq;
    if (!u && qb >= m.nqb) continue;
    int64_t first[BSA_ACSR_MAX_RUNS];
    const int nruns = a.acsr ? a.acsr[h].num_runs : 0;
    for (int j = 0; j < nruns; ++j) first[j] = acsr_first(a.acsr[h].runs[j], qb);
    for (int ik = 0; ik < mk; ++ik) {
      const int64_t kb = bk < a.tk ? tile_key_block(m, ltk - lbk, kt, ik) : (kt << ltk) >> lbk;
      if (kb >= m.nkb) continue;
      if (a.acsr) {
        bool sel = false;
        for (int j = 0; j < nruns && !sel; ++j) sel = acsr_in_run(a.acsr[h].runs[j], first[j], kb);
        if (!sel) continue;
      } else if (!(u ? u[kb] : mb[qb * m.nkb + kb])) {
        continue;
      }
      if (!u && a.causal) {
        const int64_t q0 = bq < a.tq ? qb * bq : qt * a.tq;
        const int64_t qlast = min(q0 + aq, a.Sq) - 1;
        if (kt * a.tk + ik * ak > qlast + a.off) continue;
      }
      live |= 1u << (iq * mk + ik);
    }
  }
  return live;
}

// One wave per list. EMIT = false: count live tiles. EMIT = true: write them
// at list_off[l] in ascending key-tile order (ballot + prefix popcount).
template <bool EMIT, bool BITS>
__global__ void k_map(MapArgs a) {
  const int lane = threadIdx.x & 63;
  // one list per wave: the index is wave-uniform, so head metadata and
  // descriptors come through scalar loads
  const int64_t l = (int64_t)__builtin_amdgcn_readfirstlane(
      (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6));
  if (l >= a.nlists) return;
  int lb, h, g;
  int64_t qt = 0;
  if (a.uni) {
    lb = (int)(l / a.Hkv), g = (int)(l % a.Hkv), h = g * a.G;
  } else {
    lb = (int)(l / ((int64_t)a.Hq * a.nqt)), h = (int)((l / a.nqt) % a.Hq), qt = l % a.nqt;
    g = h / a.G;
  }
  const int bm = a.bcast ? 0 : lb;
  const int64_t base = EMIT ? a.list_off[l] : 0;
  int64_t run = 0;
  const HeadMeta m = a.hm[h];
  const int lbq = __builtin_ctz(m.bq), lbk = __builtin_ctz(m.bk);
  const int ltq = __builtin_ctz(a.tq), ltk = __builtin_ctz(a.tk);
  const int mq = (!a.uni && m.bq < a.tq) ? 1 << (ltq - lbq) : 1;
  const int mk = m.bk < a.tk ? 1 << (ltk - lbk) : 1;
  // Tile kt of the list is entry `run + (live tiles of lower lanes)` when
  // live: entries come out in ascending key-tile order.
  auto emit = [&](int kt, uint32_t live) {
    const unsigned long long bal = __ballot(live != 0);
    if (EMIT && live) {
      const int64_t idx = base + run + __popcll(bal & (unsigned long long)lo_mask(lane));
      a.ent_kt[idx] = (int32_t)kt;
      a.ent_live[idx] = live;
      if (a.paged) a.ent_page[idx] = a.page_table[(int64_t)lb * a.pps + (int)(kt * a.tk) / a.P];
    }
    run += __popcll(bal);
  };
  if constexpr (BITS) {
    // Mask plans without union whose heads all have key blocks of at least
    // one tile (bk >= tk) and at most 8 query sub-blocks per tile (the host
    // launches this form only then): the 64 key tiles of a chunk fall in one
    // 64-bit word of each row's bitmap (written by the features pass: bit kb
    // of row qb is set iff the mask selects (qb, kb)), so a chunk costs a few
    // shifts per lane and query sub-block, and no mask byte is read.
    const int nkt32 = (int)a.nkt, sh = lbk - ltk;
    const int64_t words = (m.nkb + 63) >> 6, aq = m.bq < a.tq ? m.bq : a.tq;
    const unsigned long long *hb = a.bits + bm * a.bits_per_bm + m.bits_off;
    const unsigned long long *wr[8];  // the sub-blocks' row bitmaps (null: no such row)
    int klim[8];  // last key tile whose first key is within the causal limit
#pragma unroll
    for (int iq = 0; iq < 8; ++iq) {
      wr[iq] = nullptr, klim[iq] = -1;
      if (iq >= mq) continue;
      const int64_t qb = m.bq < a.tq ? qblock_of(qt, iq, m.lqil, ltq - lbq, m.nqb) : (qt << ltq) >> lbq;
      if (qb >= m.nqb) continue;
      wr[iq] = hb + qb * words;
      const int64_t q0 = m.bq < a.tq ? qb * m.bq : qt * a.tq;
      // a sub-block is dropped when its first key lies after its last query
      const int64_t lim = a.causal ? min(q0 + aq, a.Sq) - 1 + a.off : INT64_MAX;
      klim[iq] = lim < 0 ? -1 : (int)min<int64_t>(lim >> ltk, INT32_MAX);
    }
    if constexpr (!EMIT) {
      // Count only: lane j takes chunk j (key tiles 64 j .. 64 j + 63) of
      // each group of 64 chunks, builds its 64-bit live-tile mask from the
      // rows' bitmap fields (each key block's bit spread over its 2^sh
      // tiles, then cut at the causal limit and the last tile) and counts it.
      int cnt = 0;
      for (int c0 = 0; (int64_t)c0 * 64 < nkt32; c0 += 64) {
        const int k0 = (c0 + lane) * 64;  // this lane's first tile (maybe past the end)
        const int kb0 = k0 >> sh;
        const int64_t wi = min<int64_t>(kb0 >> 6, words - 1);
        unsigned long long any = 0;
#pragma unroll
        for (int iq = 0; iq < 8; ++iq) {
          if (!wr[iq]) continue;
          any |= spread_bits(wr[iq][wi] >> (kb0 & 63), sh) & prefix_mask((int64_t)klim[iq] - k0 + 1);
        }
        cnt += __popcll(any & prefix_mask((int64_t)nkt32 - k0));
      }
      cnt = wave_sum(cnt);
      if (lane == 0) a.list_len[l] = (int32_t)cnt;
      return;
    }
    // Each row's bitmap is read 64 words at a time, one word per lane (one
    // coalesced load per row, all rows' loads before any wait); a chunk
    // takes its word from the lane that holds it.
    for (int64_t wbase = 0; wbase < words; wbase += 64) {
      unsigned long long rw[8];
      const int64_t wl = min(wbase + lane, words - 1);
#pragma unroll
      for (int iq = 0; iq < 8; ++iq) rw[iq] = wr[iq] ? wr[iq][wl] : 0ull;
      // the chunks of 64 key tiles whose key blocks lie in these words
      const int kbeg = (int)((64 * wbase) << sh);
      const int kend = (int)min<int64_t>(nkt32, (64 * (wbase + 64)) << sh);
      for (int k0 = kbeg; k0 < kend; k0 += 64) {
        const int kt = k0 + lane, kb0 = k0 >> sh;   // kb0: first key block of the chunk
        const int bit = (kb0 & 63) + (lane >> sh);  // < 64: the chunk's blocks share a word
        const int wi = (int)((kb0 >> 6) - wbase);   // the lane holding the chunk's word
        uint32_t live = 0;
#pragma unroll
        for (int iq = 0; iq < 8; ++iq) {
          if (!wr[iq]) continue;
          const unsigned long long wd =
              ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(rw[iq] >> 32), wi) << 32) |
              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rw[iq], wi);
          if (((wd >> bit) & 1ull) && kt <= klim[iq]) live |= 1u << iq;
        }
        // (past the last tile a key block may still exist: Skv need not be a
        // multiple of bk)
        emit(kt, kt < nkt32 ? live : 0u);
      }
    }
    return;
  }
  if (a.uni && !a.acsr) {
    // Union lists (one per batch and kv group, so few waves, each waiting on
    // its own loads): the group's union row, kMapBatch key tiles per lane,
    // each byte loaded at a clamped index before any is tested. The same
    // live bits as live_bits below: one query sub-block, and no causal cut
    // (the union spans every query block of the group).
    const uint8_t *urow = a.U + ((int64_t)bm * a.Hkv + g) * a.unkb;
    const int nkb32 = (int)m.nkb, nkt32 = (int)a.nkt;  // below 2^31
    for (int k0 = 0; k0 < nkt32; k0 += 64 * kMapBatch) {
      uint32_t live[kMapBatch];
#pragma unroll
      for (int u = 0; u < kMapBatch; ++u) live[u] = 0;
      for (int ik = 0; ik < mk; ++ik) {
        int kb[kMapBatch];
        uint8_t v[kMapBatch];
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u) {
          const int kt = k0 + 64 * u + lane;
          kb[u] = kt >= nkt32 ? nkb32
                  : (m.bk < a.tk ? (int)tile_key_block(m, ltk - lbk, kt, ik) : (int)(((uint32_t)kt << ltk) >> lbk));
        }
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u) v[u] = urow[(uint32_t)min(kb[u], nkb32 - 1)];
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u)
          if (kb[u] < nkb32 && v[u]) live[u] |= 1u << ik;
      }
#pragma unroll
      for (int u = 0; u < kMapBatch; ++u) emit(k0 + 64 * u + lane, live[u]);
    }
    if (!EMIT && lane == 0) a.list_len[l] = (int32_t)run;
    return;
  }
  if (!a.uni && !a.acsr && mq <= 8) {
    // Mask plans: the list's query blocks, their mask rows and causal
    // limits do not depend on the key tile, so they are found once (the same
    // live bits as live_bits below, for up to 8 query sub-blocks).
    const int64_t aq = m.bq < a.tq ? m.bq : a.tq, ak = m.bk < a.tk ? m.bk : a.tk;
    const uint8_t *mb = a.mask + bm * a.mask_bstride + m.mask_off;
    int64_t rowoff[8], lim[8];
    for (int iq = 0; iq < mq; ++iq) {
      const int64_t qb = m.bq < a.tq ? qblock_of(qt, iq, m.lqil, ltq - lbq, m.nqb) : (qt << ltq) >> lbq;
      rowoff[iq] = qb < m.nqb ? qb * m.nkb : -1;
      const int64_t q0 = m.bq < a.tq ? qb * m.bq : qt * a.tq;
      // a sub-block is dropped when its first key lies after its last query
      lim[iq] = a.causal ? min(q0 + aq, a.Sq) - 1 + a.off : INT64_MAX;
    }
    const int nkb32 = (int)m.nkb, nkt32 = (int)a.nkt;
    // kMapBatch key tiles per lane at a time: for each key sub-block and
    // pair of query sub-blocks, the batch's mask bytes of both rows are
    // loaded before any is tested, so a wave waits once per pair and batch
    // rather than once per row and 64 tiles (the kernel is bound by those
    // waits). Loads take a clamped index (a missing row reads row iq0 again)
    // and are tested afterwards: a load under a lane condition would be
    // waited for at once. Key tiles, key blocks and key positions are below
    // 2^31, so the indices are 32-bit.
    for (int k0 = 0; k0 < nkt32; k0 += 64 * kMapBatch) {
      uint32_t live[kMapBatch];
#pragma unroll
      for (int u = 0; u < kMapBatch; ++u) live[u] = 0;
      for (int ik = 0; ik < mk; ++ik) {
        int kb[kMapBatch];
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u) {
          const int kt = k0 + 64 * u + lane;
          kb[u] = kt >= nkt32 ? nkb32
                  : (m.bk < a.tk ? (int)tile_key_block(m, ltk - lbk, kt, ik) : (int)(((uint32_t)kt << ltk) >> lbk));
        }
#pragma unroll
        for (int iq0 = 0; iq0 < 8; iq0 += 2) {  // (unrolled: rowoff and lim stay in registers)
          if (iq0 >= mq) break;
          const bool r0 = rowoff[iq0] >= 0, r1 = iq0 + 1 < mq && rowoff[iq0 + 1] >= 0;
          if (!r0 && !r1) continue;
          const uint8_t *m0 = mb + (r0 ? rowoff[iq0] : rowoff[iq0 + 1]);
          const uint8_t *m1 = r1 ? mb + rowoff[iq0 + 1] : m0;
          uint8_t v0[kMapBatch], v1[kMapBatch];
#pragma unroll
          for (int u = 0; u < kMapBatch; ++u) {
            const uint32_t kc = (uint32_t)min(kb[u], nkb32 - 1);
            v0[u] = m0[kc];
            v1[u] = m1[kc];
          }
#pragma unroll
          for (int u = 0; u < kMapBatch; ++u) {
            if (kb[u] >= nkb32) continue;
            // first key of the sub-block (exact for every tile that exists)
            const int64_t kfirst = (int64_t)(k0 + 64 * u + lane) * a.tk + ik * ak;
            if (r0 && v0[u] && kfirst <= lim[iq0]) live[u] |= 1u << (iq0 * mk + ik);
            if (r1 && v1[u] && kfirst <= lim[iq0 + 1]) live[u] |= 1u << ((iq0 + 1) * mk + ik);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kMapBatch; ++u) emit(k0 + 64 * u + lane, live[u]);
    }
    if (!EMIT && lane == 0) a.list_len[l] = (int32_t)run;
    return;
  }
  for (int64_t k0 = 0; k0 < a.nkt; k0 += 64) {
    const int64_t kt = k0 + lane;
    const uint32_t live = kt < a.nkt ? live_bits(a, bm, h, g, qt, kt) : 0u;
    const unsigned long long bal = __ballot(live != 0);
    if (EMIT && live) {
      const int64_t idx = base + run + __popcll(bal & (unsigned long long)lo_mask(lane));
      a.ent_kt[idx] = (int32_t)kt;
      a.ent_live[idx] = live;
      // key positions are below 2^31: a 32-bit division
      if (a.paged) a.ent_page[idx] = a.page_table[(int64_t)lb * a.pps + (int)(kt * a.tk) / a.P];
    }
    run += __popcll(bal);
  }
  if (!EMIT && lane == 0) a.list_len[l] = (int32_t)run;
}

// -------------------------------------------------------------------------
// Exclusive prefix scan (int32, three phases)
// -------------------------------------------------------------------------

// Exclusive scan of one value per thread over a 256-thread workgroup.
__device__ int block_excl_scan(int v, int *total) {
  __shared__ int wsum[kThreads / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < kThreads / 64; ++i) {
    before += i < w ? wsum[i] : 0;
    tot += wsum[i];
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__global__ void k_scan_reduce(const int32_t *__restrict__ in, int64_t n, int32_t *__restrict__ bsum) {
  const int64_t base = blockIdx.x * (int64_t)kScanBlock + threadIdx.x * 4;
  int s = 0;
  for (int u = 0; u < 4; ++u)
    if (base + u < n) s += in[base + u];
  int tot;
  block_excl_scan(s, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ void k_scan_top(int32_t *__restrict__ bsum, int64_t nb) {
  int carry = 0;
  for (int64_t base = 0; base < nb; base += kScanBlock) {
    int v[4], s = 0;
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + threadIdx.x * 4 + u;
      v[u] = i < nb ? bsum[i] : 0;
      s += v[u];
    }
    int tot;
    int run = carry + block_excl_scan(s, &tot);
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + threadIdx.x * 4 + u;
      if (i < nb) bsum[i] = run;
      run += v[u];
    }
    carry += tot;
  }
}

// out[i] = sum of in[0..i); out[n] = total. in and out may be the same array.
__global__ void k_scan_apply(const int32_t *in, int64_t n, const int32_t *__restrict__ bsum,
                             int32_t *out) {
  const int64_t base = blockIdx.x * (int64_t)kScanBlock + threadIdx.x * 4;
  int v[4], s = 0;
  for (int u = 0; u < 4; ++u) {
    v[u] = base + u < n ? in[base + u] : 0;
    s += v[u];
  }
  int tot;
  int run = bsum[blockIdx.x] + block_excl_scan(s, &tot);
  for (int u = 0; u < 4; ++u) {
    if (base + u < n) out[base + u] = run;
    run += v[u];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == kThreads - 1) out[n] = run;
}

// Whole scan in one workgroup (small arrays), in batches of kScanBatch
// rounds of 1024 consecutive elements: every thread loads its element of
// each round of the batch (coalesced, all loads in flight at once), the waves
// scan their 64-element pieces, and after one barrier each thread adds the
// totals of the pieces before its own and of the earlier rounds. in and out
// may be the same array (each element is read by the thread that writes it,
// before it writes it). Workgroup g scans the g-th of gridDim.x arrays laid
// out `stride` elements apart; out[n] receives the total.
constexpr int kScanThreads = 1024, kScanBatch = 8;
__global__ __launch_bounds__(kScanThreads) void k_scan_single(const int32_t *in, int64_t n,
                                                              int32_t *out, int64_t stride) {
  constexpr int NW = kScanThreads / 64;
  __shared__ int wsum[kScanBatch][NW];
  in += blockIdx.x * stride;
  out += blockIdx.x * stride;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int carry = 0;  // total of the batches before this one
  for (int64_t b0 = 0; b0 < n; b0 += (int64_t)kScanBatch * kScanThreads) {
    int v[kScanBatch], x[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      // a clamped index, zeroed after the load (a load under a lane
      // condition would be waited for at once)
      const int64_t i = b0 + (int64_t)u * kScanThreads + t;
      v[u] = in[min(i, n - 1)];
      if (i >= n) v[u] = 0;
    }
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      x[u] = v[u];
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x[u], o);
        if (lane >= o) x[u] += y;
      }
      if (lane == 63) wsum[u][w] = x[u];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      int before = 0, tot = 0;
      for (int i = 0; i < NW; ++i) {
        const int s = wsum[u][i];
        before += i < w ? s : 0;
        tot += s;
      }
      const int64_t i = b0 + (int64_t)u * kScanThreads + t;
      if (i < n) out[i] = carry + before + x[u] - v[u];
      carry += tot;
    }
    __syncthreads();  // wsum is rewritten by the next batch
  }
  if (t == 0) out[n] = carry;
}

constexpr int64_t kSingleScanMax = 1 << 16;

bsa_status scan(const int32_t *in, int64_t n, int32_t *out, int32_t *bsum, hipStream_t s) {
  if (n <= kSingleScanMax) {
    hipLaunchKernelGGL(k_scan_single, dim3(1), dim3(kScanThreads), 0, s, in, n, out, (int64_t)0);
    HIP_TRY(hipGetLastError());
    return BSA_OK;
  }
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)nb), dim3(kThreads), 0, s, in, n, bsum);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(kThreads), 0, s, bsum, nb);
  hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nb), dim3(kThreads), 0, s, in, n, bsum, out);
  HIP_TRY(hipGetLastError());
  return BSA_OK;
}

// -------------------------------------------------------------------------
// Rows and work list (task organization)
// -------------------------------------------------------------------------

struct RowArgs {
  const int32_t *list_off, *ent_kt;
  int32_t *row_ent, *cnt_items, *cnt_slots, *cnt_comb;
  int64_t nrows, nqt, Sq, off;
  int32_t Hq, Hkv, G, pack, uni, causal, nlb, tq, tr, tk, split;
};

// Row r = (b, head or group, q-tile). Union rows take the causal prefix of
// their group's table; every row gets its item, partial-slot and combine counts.
__global__ void k_rows(RowArgs a) {
  const int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (r >= a.nrows) return;
  const int nh = a.pack ? a.Hkv : a.Hq;
  const int64_t qt = r % a.nqt;
  const int hh = (int)((r / a.nqt) % nh);
  const int b = (int)(r / (a.nqt * nh));
  const int lb = a.nlb == 1 ? 0 : b;
  const int64_t l = a.uni ? (int64_t)lb * a.Hkv + (a.pack ? hh : hh / a.G)
                          : ((int64_t)lb * a.Hq + hh) * a.nqt + qt;
  const int32_t e0 = a.list_off[l];
  int32_t e1 = a.list_off[l + 1];
  if (a.uni && a.causal) {
    const int64_t lim = min((qt + 1) * a.tr, a.Sq) - 1 + a.off;
    int32_t lo = e0, hi = e1;
    while (lo < hi) {
      const int32_t mid = lo + ((hi - lo) >> 1);
      if ((int64_t)a.ent_kt[mid] * a.tk <= lim) lo = mid + 1;
      else hi = mid;
    }
    e1 = lo;
  }
  a.row_ent[2 * r] = e0;
  a.row_ent[2 * r + 1] = e1;
  const int64_t n = e1 - e0;
  const int64_t k = (a.split > 0 && n > a.split) ? (n + a.split - 1) / a.split : 1;
  a.cnt_items[r] = (int32_t)k;
  a.cnt_slots[r] = k > 1 ? (int32_t)k : 0;
  a.cnt_comb[r] = k > 1 ? 1 : 0;
}

// Emit each row's items (balanced chunks of a split row) and combine record.
__global__ void k_items(const int32_t *__restrict__ row_ent, const int32_t *__restrict__ item_off,
                        const int32_t *__restrict__ slot_off, const int32_t *__restrict__ comb_off,
                        int64_t nrows, int4 *__restrict__ items, int32_t *__restrict__ comb) {
  const int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (r >= nrows) return;
  const int64_t e0 = row_ent[2 * r], n = row_ent[2 * r + 1] - e0;
  const int64_t k = item_off[r + 1] - item_off[r];
  for (int64_t j = 0; j < k; ++j)
    items[item_off[r] + j] = make_int4((int)r, (int)(e0 + j * n / k), (int)(e0 + (j + 1) * n / k),
                                       k > 1 ? (int)(slot_off[r] + j) : -1);
  if (k > 1) {
    const int32_t c = comb_off[r];
    comb[3 * c] = (int32_t)r, comb[3 * c + 1] = slot_off[r], comb[3 * c + 2] = (int32_t)k;
  }
}

__global__ void k_totals(const int32_t *list_off, int64_t nlists, const int32_t *item_off,
                         const int32_t *slot_off, const int32_t *comb_off, int64_t nrows,
                         int32_t *counters) {
  counters[CNT_ENT] = list_off[nlists];
  counters[CNT_ITEMS] = item_off[nrows];
  counters[CNT_SLOTS] = slot_off[nrows];
  counters[CNT_COMB] = comb_off[nrows];
}

// Longest-first order: stable counting sort on key min(length, 1023),
// descending. hist[k * nchunks + c] counts items of chunk c with key index
// k = 1023 - key; its exclusive scan gives each (key, chunk) its first slot.
__global__ void k_lpt_hist(const int4 *__restrict__ items, const int32_t *__restrict__ counters,
                           int64_t nchunks, int32_t *__restrict__ hist) {
  __shared__ int h[kLptKeys];
  for (int i = threadIdx.x; i < kLptKeys; i += kThreads) h[i] = 0;
  __syncthreads();
  const int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  if (i < counters[CNT_ITEMS]) {
    const int4 it = items[i];
    atomicAdd(&h[kLptKeys - 1 - min(it.z - it.y, kLptKeys - 1)], 1);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < kLptKeys; k += kThreads) hist[k * nchunks + blockIdx.x] = h[k];
}

__global__ void k_lpt_place(const int4 *__restrict__ items, const int32_t *__restrict__ counters,
                            int64_t nchunks, const int32_t *__restrict__ start,
                            int4 *__restrict__ out) {
  __shared__ int keys[kThreads];
  const int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  const bool valid = i < counters[CNT_ITEMS];
  int4 it = make_int4(0, 0, 0, 0);
  int key = -1;
  if (valid) {
    it = items[i];
    key = kLptKeys - 1 - min(it.z - it.y, kLptKeys - 1);
  }
  keys[threadIdx.x] = key;
  __syncthreads();
  if (valid) {
    int rank = 0;
    for (int t = 0; t < (int)threadIdx.x; ++t) rank += keys[t] == key;
    out[start[key * nchunks + blockIdx.x] + rank] = it;
  }
}

unsigned grid_for(int64_t threads) { return (unsigned)((threads + kThreads - 1) / kThreads); }

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// -------------------------------------------------------------------------
// Key-major chunk index for the backward pass
// -------------------------------------------------------------------------

struct KvIndexArgs {
  const int32_t *list_off, *ent_kt;
  const uint32_t *ent_live;
  const HeadMeta *hm;
  int64_t Sq, off, nqt, nkt, nbuckets;
  int32_t Hq, Hkv, G, nkp, tq, uni, causal;
  int32_t *cnt;
  const int32_t *boff;
  int32_t *q0, *meta;
  uint32_t *live;
};

// Lower bound of kt0 in the sorted list [lo, hi), then the live words of
// tiles kt0 .. kt0 + NKT - 1 (0 for a tile the list does not hold).
template <int NKT>
__device__ __forceinline__ void tile_live(const KvIndexArgs &a, int lo, int hi, int kt0, uint32_t (&lv)[NKT]) {
  const int end = hi;
  while (lo < hi) {
    const int mid = lo + ((hi - lo) >> 1);
    if (a.ent_kt[mid] < kt0) lo = mid + 1;
    else hi = mid;
  }
  for (int t = 0; t < NKT; ++t) {
    lv[t] = 0u;
    if (lo < end && a.ent_kt[lo] == kt0 + t) lv[t] = a.ent_live[lo++];
  }
}

// One wave per bucket (list batch lb, kv head g, group kp of NKT consecutive
// key tiles = 128 keys). A chunk is 32 consecutive queries of one head that
// may see a key of the group: its row's list holds one of the tiles (in
// union mode the group's table does), its queries exist, it is causally
// feasible for the group's first key, and a live bit of its query
// sub-blocks is set. Chunks are emitted in (head, tile, chunk) order with
// their first query, a packed word (head within the group | chunk index within
// the plan row << 8 | lq << 11 | lk << 16 | mk << 21) and the NKT live words.
// EMIT = false counts them.
template <bool EMIT, int NKT>
__global__ void k_kv_chunks(KvIndexArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t bk = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  if (bk >= a.nbuckets) return;
  const int kp = (int)(bk % a.nkp), g = (int)((bk / a.nkp) % a.Hkv), lb = (int)(bk / ((int64_t)a.nkp * a.Hkv));
  const int kt0 = kp * NKT;
  const int64_t kb0 = (int64_t)kp * 128;
  const int cpr = a.tq / 32;
  const int64_t base = EMIT ? a.boff[bk] : 0;
  int64_t run = 0;
  // Emit the chunks of one query range whose flags are in bal (lane = chunk).
  auto emit = [&](unsigned long long bal, int64_t q0, int hloc, int cidx, const HeadMeta &m,
                  const uint32_t (&lv)[NKT]) {
    if (EMIT && ((bal >> lane) & 1ull)) {
      const int64_t idx = base + run + __popcll(bal & (unsigned long long)lo_mask(lane));
      a.q0[idx] = (int32_t)q0;
      a.meta[idx] = hloc | (cidx << 8) | (m.lq << 11) | (m.lk << 16) | (m.mk << 21);
      for (int t = 0; t < NKT; ++t) a.live[NKT * idx + t] = lv[t];
    }
    run += __popcll(bal);
  };
  auto feasible = [&](int64_t q0) {
    if (q0 >= a.Sq) return false;
    const int64_t last = min(q0 + 31, a.Sq - 1);
    return !(a.causal && kb0 > last + a.off);
  };
  if (a.uni) {
    const int64_t l = (int64_t)lb * a.Hkv + g;
    uint32_t lv[NKT];
    tile_live<NKT>(a, a.list_off[l], a.list_off[l + 1], kt0, lv);
    bool any = false;
    for (int t = 0; t < NKT; ++t) any |= lv[t] != 0u;
    if (any) {
      const int64_t nch = (a.Sq + 31) / 32;
      for (int h = g * a.G; h < (g + 1) * a.G; ++h) {
        const HeadMeta m = a.hm[h];
        for (int64_t c0 = 0; c0 < nch; c0 += 64) {
          const int64_t q0 = 32 * (c0 + lane);
          emit(__ballot(c0 + lane < nch && feasible(q0)), q0, h - g * a.G, 0, m, lv);
        }
      }
    }
  } else {
    for (int h = g * a.G; h < (g + 1) * a.G; ++h) {
      const HeadMeta m = a.hm[h];
      const int niq = m.lq >= 5 ? 1 : (32 >> m.lq);
      for (int64_t qb = 0; qb < a.nqt; qb += 64) {
        const int64_t qt = qb + lane;
        uint32_t lv[NKT];
        bool any = false;
        for (int t = 0; t < NKT; ++t) lv[t] = 0u;
        if (qt < a.nqt) {
          const int64_t l = ((int64_t)lb * a.Hq + h) * a.nqt + qt;
          tile_live<NKT>(a, a.list_off[l], a.list_off[l + 1], kt0, lv);
          for (int t = 0; t < NKT; ++t) any |= lv[t] != 0u;
        }
        unsigned long long rows = __ballot(any);
        while (rows) {
          const int bit = __builtin_ctzll(rows);
          rows &= rows - 1;
          uint32_t rl[NKT];
          for (int t = 0; t < NKT; ++t) rl[t] = __shfl(lv[t], bit);
          // lane = chunk of the row; its first query, through the interleave
          const int64_t q0 = lane < cpr ? tile_query(m, __builtin_ctz(a.tq), qb + bit, 32 * lane) : a.Sq;
          bool ok = lane < cpr && feasible(q0);
          if (ok) {
            const int iq0 = (32 * lane) >> m.lq;
            const uint64_t cb = ((1ull << (m.mk * niq)) - 1ull) << (iq0 * m.mk);
            bool hit = false;
            for (int t = 0; t < NKT; ++t) hit |= ((uint64_t)rl[t] & cb) != 0;
            ok = hit;
          }
          emit(__ballot(ok), q0, h - g * a.G, lane, m, rl);
        }
      }
    }
  }
  if (!EMIT && lane == 0) a.cnt[bk] = (int32_t)run;
}

// Small host data to device memory through kernel arguments: the arguments
// are captured at launch, so the call neither waits for the stream nor keeps
// a host buffer alive until a copy has run.
struct PutArgs {
  void *dst;
  uint32_t words;
  uint32_t data[448];
};
__global__ void k_put(PutArgs a) {
  for (uint32_t i = threadIdx.x; i < a.words; i += blockDim.x) ((uint32_t *)a.dst)[i] = a.data[i];
}

static bsa_status put_async(void *dst, const void *src, size_t bytes, hipStream_t s) {
  constexpr size_t kChunk = sizeof(PutArgs::data);
  for (size_t o = 0; o < bytes; o += kChunk) {
    PutArgs a;
    const size_t n = std::min(kChunk, bytes - o);
    a.dst = (uint8_t *)dst + o;
    a.words = (uint32_t)(n / 4);
    memcpy(a.data, (const uint8_t *)src + o, n);
    hipLaunchKernelGGL(k_put, dim3(1), dim3(kThreads), 0, s, a);
  }
  HIP_TRY(hipGetLastError());
  return BSA_OK;
}

bsa_status plan_features(Plan &p, const uint8_t *mask, const int32_t *page_table) {
  hipStream_t s = p.stream;
  int64_t rows_per_bm = 0, mask_bstride = 0, bits_off = 0;
  std::vector<HeadMeta> &hm = p.hmeta_host;
  hm.assign(p.Hq, HeadMeta{});
  for (int h = 0; h < p.Hq; ++h) {
    const int64_t nq = (p.Sq + p.bq[h] - 1) / p.bq[h], nk = (p.Skv + p.bk[h] - 1) / p.bk[h];
    hm[h] = HeadMeta{mask_bstride, rows_per_bm, bits_off, (int32_t)nq, (int32_t)nk, p.bq[h], p.bk[h], 0, 0, 0, 0};
    rows_per_bm += nq;
    mask_bstride += nq * nk;
    bits_off += nq * ((nk + 63) / 64);
  }
  HIP_TRY(hipMemcpyAsync(p.hmeta, hm.data(), sizeof(HeadMeta) * p.Hq, hipMemcpyHostToDevice, s));
  if (p.uni && p.unkb > 0)
    hipLaunchKernelGGL(k_union, dim3(grid_for((int64_t)p.nbm * p.Hkv * p.unkb)), dim3(kThreads), 0,
                       s, mask, p.hmeta, mask_bstride, p.Hkv, p.G, (int)p.nbm, p.unkb, p.uni_bits);
  if (p.nbm * rows_per_bm > 0)
    hipLaunchKernelGGL(k_row_features, dim3(grid_for(p.nbm * rows_per_bm * 64)), dim3(kThreads), 0,
                       s, mask, p.hmeta, p.Hq, p.Hkv, p.G, (int)p.nbm, rows_per_bm, mask_bstride,
                       p.uni ? p.uni_bits : nullptr, p.unkb, p.causal, p.off, p.Sq, p.row_feat,
                       p.row_bits, p.bits_per_bm);
  hipLaunchKernelGGL(k_head_features, dim3((unsigned)(p.nbm * p.Hq)), dim3(kThreads), 0, s,
                     p.row_feat, p.hmeta, p.Hq, rows_per_bm, p.feat_dev);
  // Query-block interleave costs (non-union plans; the tile shape is not yet
  // known, so 128-row tiles are assumed and the host keeps interleave 1 for
  // any other shape). Wave offsets per (head, candidate) go as kernel
  // arguments through a small device array written by k_put.
  if (!p.uni) {
    std::vector<int64_t> woff(p.Hq * kQilCands + 1, 0);
    int64_t nw = 0;
    for (int h = 0; h < p.Hq; ++h) {
      const int64_t bq = p.bq[h], nq = (p.Sq + bq - 1) / bq;
      for (int c = 0; c < kQilCands; ++c) {
        woff[h * kQilCands + c] = nw;
        const int64_t mq = bq < 128 ? 128 / bq : 1;
        if (bq >= 32 && bq < 128 && (int64_t(1) << c) * mq <= nq)
          nw += (p.nbm * ((nq + mq - 1) / mq) + kCostTiles - 1) / kCostTiles;
      }
    }
    woff[p.Hq * kQilCands] = nw;
    if (nw > 0) {
      unsigned long long *kcost = p.qil_dev + (size_t)p.Hq * kQilCands;
      int64_t *woff_dev = (int64_t *)(kcost + (size_t)p.Hq * kQilCands * kKilCands);
      if (bsa_status st = put_async(woff_dev, woff.data(), sizeof(int64_t) * woff.size(), s)) return st;
      hipLaunchKernelGGL(k_qil_cost, dim3(grid_for(nw * 64)), dim3(kThreads), 0, s, p.row_bits,
                         p.bits_per_bm, p.hmeta, p.Hq, (int)p.nbm, (const int64_t *)woff_dev, nw, p.qil_dev,
                         (!p.causal && !p.paged && p.dtype == BSA_BF16 && p.G == 1) ? 1 : 0, kcost);
    }
  }
  if (p.paged && p.Skv > 0) {
    const int64_t used = (p.Skv + p.P - 1) / p.P;
    hipLaunchKernelGGL(k_check_pages, dim3(grid_for(p.B * used)), dim3(kThreads), 0, s, page_table,
                       p.B, p.pps, used, p.npages, p.counters);
  }
  HIP_TRY(hipGetLastError());
  return BSA_OK;
}

bsa_status plan_features_acsr(Plan &p, const bsa_acsr_head *heads, bsa_acsr_head *dev_heads,
                              const bsa_problem &pr) {
  std::vector<HeadMeta> &hm = p.hmeta_host;
  hm.assign(p.Hq, HeadMeta{});
  int64_t rows = 0, mask_off = 0;
  for (int h = 0; h < p.Hq; ++h) {
    const int64_t nq = (p.Sq + p.bq[h] - 1) / p.bq[h], nk = (p.Skv + p.bk[h] - 1) / p.bk[h];
    hm[h] = HeadMeta{mask_off, rows, 0, (int32_t)nq, (int32_t)nk, p.bq[h], p.bk[h], 0, 0, 0, 0};
    rows += nq;
    mask_off += nq * nk;
  }
  // (the head metadata goes up with its live-bit geometry once the tile
  // shape is known, in plan_build)
  static_assert(sizeof(HeadMeta) % 4 == 0 && sizeof(bsa_acsr_head) % 4 == 0, "word copies");
  if (bsa_status st = put_async(dev_heads, heads, sizeof(bsa_acsr_head) * p.Hq, p.stream)) return st;
  p.acsr = dev_heads;
  p.feat.assign(4 * (size_t)p.Hq, 0);
  acsr_features(pr, heads, p.feat.data());
  p.qil_cost.assign((size_t)kQilCands * p.Hq, 0);
  p.kil_cost.assign((size_t)kQilCands * kKilCands * p.Hq, 0);
  acsr_qil_costs(pr, heads, p.qil_cost.data(), p.kil_cost.data());
  return BSA_OK;
}

size_t plan_scratch_bytes(const Plan &p) {
  const int64_t nchunks = (p.item_cap + kThreads - 1) / kThreads;
  const int64_t big = std::max<int64_t>({p.nlists + 1, 3 * (p.nrows + 1), kLptKeys * nchunks + 1});
  size_t b = 0;
  b += align_up(sizeof(int32_t) * (p.nlists + 1));          // list lengths
  b += align_up(sizeof(int32_t) * 3 * (p.nrows + 1));       // item / slot / combine counts
  b += align_up(sizeof(int32_t) * 3 * (p.nrows + 1));       // their scans
  b += align_up(sizeof(int32_t) * (big / kScanBlock + 2));  // scan block sums
  b += align_up(sizeof(int32_t) * (kLptKeys * nchunks + 1)); // longest-first histogram
  b += align_up(sizeof(int4) * (p.item_cap + 1));           // unsorted items
  return b;
}

bsa_status plan_build(Plan &p, const uint8_t *mask, const int32_t *page_table, void *scratch,
                      size_t scratch_bytes) {
  hipStream_t s = p.stream;
  uint8_t *sp = (uint8_t *)scratch;
  auto take = [&](size_t bytes) {
    uint8_t *r = sp;
    sp += align_up(bytes);
    return r;
  };
  const int64_t nchunks = (p.item_cap + kThreads - 1) / kThreads;
  int32_t *list_len = (int32_t *)take(sizeof(int32_t) * (p.nlists + 1));
  int32_t *cnt = (int32_t *)take(sizeof(int32_t) * 3 * (p.nrows + 1));
  int32_t *off = (int32_t *)take(sizeof(int32_t) * 3 * (p.nrows + 1));
  const int64_t big = std::max<int64_t>({p.nlists + 1, 3 * (p.nrows + 1), kLptKeys * nchunks + 1});
  int32_t *bsum = (int32_t *)take(sizeof(int32_t) * (big / kScanBlock + 2));
  int32_t *hist = (int32_t *)take(sizeof(int32_t) * (kLptKeys * nchunks + 1));
  int4 *raw_items = (int4 *)take(sizeof(int4) * (p.item_cap + 1));
  if ((size_t)(sp - (uint8_t *)scratch) > scratch_bytes)
    return fail(BSA_ERR_HIP, "planner scratch too small");

  // Live-bit decoding and query-block interleave per head, now that the
  // tile shape is known, sent as kernel arguments (no host buffer has to
  // outlive the call).
  for (int h = 0; h < p.Hq; ++h) {
    HeadMeta &m = p.hmeta_host[h];
    const int aq = std::min(m.bq, p.rg.tq), ak = std::min(m.bk, p.rg.tk);
    m.lq = p.uni ? 30 : __builtin_ctz(aq), m.lk = __builtin_ctz(ak), m.mk = p.rg.tk / ak;
    m.lqil = __builtin_ctz(p.qil[h]);
    m.lkil = __builtin_ctz(p.kil[h]);
  }
  if (bsa_status st = put_async(p.hmeta, p.hmeta_host.data(), sizeof(HeadMeta) * p.Hq, s)) return st;

  MapArgs m{};
  m.mask = mask, m.U = p.uni_bits, m.acsr = p.acsr, m.hm = p.hmeta, m.page_table = page_table;
  m.bits = p.row_bits, m.bits_per_bm = p.bits_per_bm;
  int64_t mask_bstride = 0;
  for (int h = 0; h < p.Hq; ++h)
    mask_bstride += ((p.Sq + p.bq[h] - 1) / p.bq[h]) * ((p.Skv + p.bk[h] - 1) / p.bk[h]);
  m.mask_bstride = mask_bstride, m.unkb = p.unkb, m.Sq = p.Sq, m.off = p.off;
  m.nqt = p.nqt, m.nkt = p.nkt, m.nlists = p.nlists;
  m.Hq = p.Hq, m.Hkv = p.Hkv, m.G = p.G, m.bcast = p.nbm == 1 ? 1 : 0, m.uni = p.uni;
  m.paged = p.paged, m.causal = p.causal, m.tq = p.rg.tq, m.tk = p.rg.tk, m.pps = p.pps, m.P = p.P;
  m.list_len = list_len, m.list_off = p.list_off;
  m.ent_kt = p.ent_kt, m.ent_page = p.ent_page, m.ent_live = p.ent_live;

  const unsigned gl = grid_for(p.nlists * 64);
  // The bitmap form of k_map when every head allows it.
  bool bits = p.row_bits != nullptr && !p.uni && !p.acsr;
  for (int h = 0; h < p.Hq && bits; ++h)
    bits = p.bk[h] >= p.rg.tk && (p.bq[h] >= p.rg.tq || p.rg.tq / p.bq[h] <= 8);
  if (p.nlists > 0) {
    if (bits) hipLaunchKernelGGL((k_map<false, true>), dim3(gl), dim3(kThreads), 0, s, m);
    else hipLaunchKernelGGL((k_map<false, false>), dim3(gl), dim3(kThreads), 0, s, m);
  }
  if (bsa_status st = scan(list_len, p.nlists, p.list_off, bsum, s)) return st;
  if (p.nlists > 0) {
    if (bits) hipLaunchKernelGGL((k_map<true, true>), dim3(gl), dim3(kThreads), 0, s, m);
    else hipLaunchKernelGGL((k_map<true, false>), dim3(gl), dim3(kThreads), 0, s, m);
  }

  RowArgs ra{};
  ra.list_off = p.list_off, ra.ent_kt = p.ent_kt, ra.row_ent = p.row_ent;
  ra.cnt_items = cnt, ra.cnt_slots = cnt + (p.nrows + 1), ra.cnt_comb = cnt + 2 * (p.nrows + 1);
  ra.nrows = p.nrows, ra.nqt = p.nqt, ra.Sq = p.Sq, ra.off = p.off;
  ra.Hq = p.Hq, ra.Hkv = p.Hkv, ra.G = p.G, ra.pack = p.rg.pack, ra.uni = p.uni;
  ra.causal = p.causal, ra.nlb = (int)p.nlb, ra.tq = p.rg.tq, ra.tr = p.tr, ra.tk = p.rg.tk;
  ra.split = p.rg.split;
  if (p.nrows > 0) hipLaunchKernelGGL(k_rows, dim3(grid_for(p.nrows)), dim3(kThreads), 0, s, ra);
  int32_t *item_off = off, *slot_off = off + (p.nrows + 1), *comb_off = off + 2 * (p.nrows + 1);
  if (p.nrows <= kSingleScanMax) {
    // The three row counts (items, partial slots, combine records) in one launch.
    hipLaunchKernelGGL(k_scan_single, dim3(3), dim3(kScanThreads), 0, s, ra.cnt_items, p.nrows, item_off,
                       p.nrows + 1);
  } else {
    if (bsa_status st = scan(ra.cnt_items, p.nrows, item_off, bsum, s)) return st;
    if (bsa_status st = scan(ra.cnt_slots, p.nrows, slot_off, bsum, s)) return st;
    if (bsa_status st = scan(ra.cnt_comb, p.nrows, comb_off, bsum, s)) return st;
  }
  int4 *dst = p.rg.sched == 1 ? raw_items : (int4 *)p.items;
  if (p.nrows > 0)
    hipLaunchKernelGGL(k_items, dim3(grid_for(p.nrows)), dim3(kThreads), 0, s, p.row_ent, item_off,
                       slot_off, comb_off, p.nrows, dst, p.comb);
  hipLaunchKernelGGL(k_totals, dim3(1), dim3(1), 0, s, p.list_off, p.nlists, item_off, slot_off,
                     comb_off, p.nrows, p.counters);
  if (p.rg.sched == 1 && nchunks > 0) {
    hipLaunchKernelGGL(k_lpt_hist, dim3((unsigned)nchunks), dim3(kThreads), 0, s, raw_items,
                       p.counters, nchunks, hist);
    if (bsa_status st = scan(hist, kLptKeys * nchunks, hist, bsum, s)) return st;
    hipLaunchKernelGGL(k_lpt_place, dim3((unsigned)nchunks), dim3(kThreads), 0, s, raw_items,
                       p.counters, nchunks, hist, (int4 *)p.items);
  }
  HIP_TRY(hipGetLastError());
  return BSA_OK;
}

// Upper bound on the chunks of the key-major index.
static int64_t kv_chunk_cap(const Plan &p, int nkt_per) {
  const int64_t nkp = (p.nkt + nkt_per - 1) / nkt_per;
  if (p.uni) return std::max<int64_t>((int64_t)p.nlb * p.Hkv * nkp * p.G * ((p.Sq + 31) / 32), 1);
  return std::max<int64_t>(p.ent_cap * (p.rg.tq / 32), 1);
}

size_t plan_kv_index_bytes(const Plan &p, int nkt_per) {
  const int64_t nkp = (p.nkt + nkt_per - 1) / nkt_per;
  const int64_t nb = (int64_t)p.nlb * p.Hkv * nkp;
  const int64_t cap = kv_chunk_cap(p, nkt_per);
  size_t b = 0;
  b += align_up(sizeof(int32_t) * (nb + 1));              // counts
  b += align_up(sizeof(int32_t) * (nb + 1));              // offsets
  b += align_up(sizeof(int32_t) * (nb / kScanBlock + 2)); // scan block sums
  b += align_up(sizeof(int32_t) * cap);                   // first queries
  b += align_up(sizeof(int32_t) * cap);                   // packed words
  b += align_up(sizeof(uint32_t) * nkt_per * cap);        // live words
  return b;
}

bsa_status plan_kv_index(const Plan &p, int nkt_per, void *scratch, KvIndex *out, hipStream_t s) {
  const int64_t nkp = (p.nkt + nkt_per - 1) / nkt_per;
  const int64_t nb = (int64_t)p.nlb * p.Hkv * nkp;
  const int64_t cap = kv_chunk_cap(p, nkt_per);
  uint8_t *sp = (uint8_t *)scratch;
  auto take = [&](size_t bytes) {
    uint8_t *r = sp;
    sp += align_up(bytes);
    return r;
  };
  KvIndexArgs a{};
  a.list_off = p.list_off, a.ent_kt = p.ent_kt, a.ent_live = p.ent_live, a.hm = p.hmeta;
  a.Sq = p.Sq, a.off = p.off, a.nqt = p.nqt, a.nkt = p.nkt, a.nbuckets = nb;
  a.Hq = p.Hq, a.Hkv = p.Hkv, a.G = p.G, a.nkp = (int32_t)nkp, a.tq = p.rg.tq;
  a.uni = p.uni, a.causal = p.causal;
  a.cnt = (int32_t *)take(sizeof(int32_t) * (nb + 1));
  int32_t *off = (int32_t *)take(sizeof(int32_t) * (nb + 1));
  int32_t *bsum = (int32_t *)take(sizeof(int32_t) * (nb / kScanBlock + 2));
  a.boff = off;
  a.q0 = (int32_t *)take(sizeof(int32_t) * cap);
  a.meta = (int32_t *)take(sizeof(int32_t) * cap);
  a.live = (uint32_t *)take(sizeof(uint32_t) * nkt_per * cap);
  out->off = off, out->q0 = a.q0, out->meta = a.meta, out->live = a.live, out->nkp = nkp;
  if (nb == 0) return BSA_OK;
  const unsigned grid = grid_for(nb * 64);
  if (nkt_per == 2) hipLaunchKernelGGL((k_kv_chunks<false, 2>), dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_kv_chunks<false, 1>), dim3(grid), dim3(kThreads), 0, s, a);
  if (bsa_status st = scan(a.cnt, nb, off, bsum, s)) return st;
  if (nkt_per == 2) hipLaunchKernelGGL((k_kv_chunks<true, 2>), dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_kv_chunks<true, 1>), dim3(grid), dim3(kThreads), 0, s, a);
  HIP_TRY(hipGetLastError());
  return BSA_OK;
}

}  // namespace bsa
