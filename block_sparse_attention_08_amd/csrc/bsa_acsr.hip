// Affine-compressed sparse rows: argument checks and mask features counted
// on the host.
//
// SPLAT (abstract) observes that the masks of common sparse attention
// patterns have regular geometric properties and stores them in an
// affine-compressed sparse-row format, so that a row's columns follow from
// the row index instead of being listed. Here a head's logical mask is the
// union of up to four runs; run j selects, in query block r, the key blocks
//   floor(row_num_j * r / row_den_j) + offset_j + stride_j * i,  0 <= i < count_j,
// that fall in [0, nkb). The planner needs, per head, the selected blocks,
// the largest row, the empty rows and the blocks the causal bound leaves
// reachable. Each row's count is the size of a union of arithmetic
// progressions cut to a range: one run is a closed form, runs of stride one
// are merged intervals, and anything else goes by inclusion and exclusion
// over the runs, each intersection of progressions being one progression
// (Chinese remainder theorem) or empty. No row is enumerated block by block.
#include "bsa_internal.h"

#include <algorithm>

namespace bsa {
namespace {

typedef __int128 i128;

constexpr int64_t kMaxNum = int64_t(1) << 20, kMaxOff = int64_t(1) << 40;
constexpr int64_t kMaxStride = int64_t(1) << 31, kMaxCount = int64_t(1) << 40;
constexpr int64_t kMaxSpan = int64_t(1) << 50;

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// {first + stride * i : 0 <= i < count}, count >= 1.
struct Prog {
  int64_t first, stride, last;
};

// Elements of progression p in [lo, hi].
int64_t prog_count(const Prog &p, int64_t lo, int64_t hi) {
  const int64_t a = std::max(lo, p.first), b = std::min(hi, p.last);
  if (a > b) return 0;
  if (p.stride == 1) return b - a + 1;
  const int64_t i0 = cdiv64(a - p.first, p.stride), i1 = (b - p.first) / p.stride;
  return i1 >= i0 ? i1 - i0 + 1 : 0;
}

i128 mod128(i128 a, i128 m) {
  const i128 r = a % m;
  return r < 0 ? r + m : r;
}

// Inverse of a modulo m (gcd(a, m) = 1, m >= 1), by the extended Euclidean
// algorithm.
i128 inv_mod(i128 a, i128 m) {
  if (m == 1) return 0;
  i128 r0 = mod128(a, m), r1 = m, s0 = 1, s1 = 0;
  while (r1 != 0) {
    const i128 q = r0 / r1;
    i128 t = r0 - q * r1;
    r0 = r1, r1 = t;
    t = s0 - q * s1;
    s0 = s1, s1 = t;
  }
  return mod128(s0, m);
}

i128 gcd128(i128 a, i128 b) {
  while (b != 0) {
    const i128 t = a % b;
    a = b, b = t;
  }
  return a < 0 ? -a : a;
}

// |union of ps[0..n) cut to [lo, hi]|.
int64_t union_count(const Prog *ps, int n, int64_t lo, int64_t hi) {
  if (n == 0 || lo > hi) return 0;
  if (n == 1) return prog_count(ps[0], lo, hi);
  bool unit = true;
  for (int i = 0; i < n; ++i) unit &= ps[i].stride == 1;
  if (unit) {
    // merged intervals
    std::pair<int64_t, int64_t> iv[BSA_ACSR_MAX_RUNS];
    int m = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t a = std::max(lo, ps[i].first), b = std::min(hi, ps[i].last);
      if (a <= b) iv[m++] = {a, b};
    }
    std::sort(iv, iv + m);
    int64_t tot = 0, ca = 0, cb = -1;
    bool open = false;
    for (int i = 0; i < m; ++i) {
      if (open && iv[i].first <= cb + 1) {
        cb = std::max(cb, iv[i].second);
      } else {
        if (open) tot += cb - ca + 1;
        ca = iv[i].first, cb = iv[i].second, open = true;
      }
    }
    if (open) tot += cb - ca + 1;
    return tot;
  }
  // inclusion and exclusion over the nonempty subsets
  int64_t tot = 0;
  for (unsigned s = 1; s < (1u << n); ++s) {
    i128 t = 0, L = 1;
    int64_t a = lo, b = hi;
    bool empty = false;
    for (int i = 0; i < n && !empty; ++i) {
      if (!((s >> i) & 1u)) continue;
      a = std::max(a, ps[i].first), b = std::min(b, ps[i].last);
      // combine x = t (mod L) with x = first_i (mod stride_i)
      const i128 m = ps[i].stride, g = gcd128(L, m), diff = (i128)ps[i].first - t;
      if (mod128(diff, g) != 0) {
        empty = true;
        break;
      }
      const i128 mg = m / g;
      const i128 k = mod128((diff / g) % mg * inv_mod(L / g, mg), mg);
      t = t + L * k;
      L = L / g * m;
      t = mod128(t, L);
    }
    if (empty || a > b) continue;
    const i128 x0 = (i128)a + mod128(t - a, L);
    const int64_t c = x0 > b ? 0 : (int64_t)(((i128)b - x0) / L) + 1;
    tot += (__builtin_popcount(s) & 1) ? c : -c;
  }
  return tot;
}

}  // namespace

bsa_status acsr_check(const bsa_problem &pr, const bsa_acsr_head *heads) {
  if (pr.mask_batch_broadcast != 1)
    return fail(BSA_ERR_INVALID_ARG, "ACSR plans need mask_batch_broadcast = 1 (one pattern for every batch)");
  if (pr.gqa_union) return fail(BSA_ERR_UNSUPPORTED, "ACSR plans do not support gqa_union");
  if (pr.paged) return fail(BSA_ERR_UNSUPPORTED, "ACSR plans do not support paged K/V");
  if (!heads) return fail(BSA_ERR_INVALID_ARG, "heads is NULL");
  for (int h = 0; h < pr.num_q_heads; ++h) {
    const bsa_acsr_head &d = heads[h];
    const std::string where = " (head " + std::to_string(h) + ")";
    if (d.num_runs < 0 || d.num_runs > BSA_ACSR_MAX_RUNS || d.reserved != 0)
      return fail(BSA_ERR_INVALID_ARG, "num_runs must be in [0, 4] and reserved 0" + where);
    for (int j = 0; j < d.num_runs; ++j) {
      const bsa_acsr_run &u = d.runs[j];
      if (u.row_den < 1 || u.row_den > kMaxNum || u.row_num < -kMaxNum || u.row_num > kMaxNum)
        return fail(BSA_ERR_INVALID_ARG, "row_num must be in [-2^20, 2^20] and row_den in [1, 2^20]" + where);
      if (u.offset < -kMaxOff || u.offset > kMaxOff)
        return fail(BSA_ERR_INVALID_ARG, "offset must be in [-2^40, 2^40]" + where);
      if (u.stride < 1 || u.stride > kMaxStride || u.count < 0 || u.count > kMaxCount ||
          (u.count > 0 && u.stride > kMaxSpan / u.count))
        return fail(BSA_ERR_INVALID_ARG,
                    "stride must be in [1, 2^31], count in [0, 2^40], stride * count <= 2^50" + where);
    }
  }
  return BSA_OK;
}

void acsr_features(const bsa_problem &pr, const bsa_acsr_head *heads, int64_t *out) {
  for (int h = 0; h < pr.num_q_heads; ++h) {
    const int64_t bq = pr.block_q[h], bk = pr.block_k[h];
    const int64_t nqb = (pr.seqlen_q + bq - 1) / bq, nkb = (pr.seqlen_kv + bk - 1) / bk;
    const bsa_acsr_head &d = heads[h];
    int64_t nnz = 0, mx = 0, empty = 0, eff = 0;
    for (int64_t r = 0; r < nqb; ++r) {
      Prog ps[BSA_ACSR_MAX_RUNS];
      int n = 0;
      for (int j = 0; j < d.num_runs; ++j) {
        const bsa_acsr_run &u = d.runs[j];
        if (u.count == 0) continue;
        const int64_t f = acsr_first(u, r);
        // a single block is a progression of stride one
        const int64_t st = u.count == 1 ? 1 : u.stride;
        ps[n++] = Prog{f, st, f + u.stride * (u.count - 1)};
      }
      const int64_t c = union_count(ps, n, 0, nkb - 1);
      int64_t e = c;
      if (pr.causal) {
        // key blocks whose first key the row's last query can reach
        const int64_t qlast = std::min(pr.seqlen_q, (r + 1) * bq) - 1;
        const int64_t kbmax = qlast + pr.causal_kv_offset < 0 ? -1 : (qlast + pr.causal_kv_offset) / bk;
        e = kbmax >= nkb - 1 ? c : union_count(ps, n, 0, kbmax);
      }
      nnz += c;
      mx = std::max(mx, c);
      empty += c == 0;
      eff += e;
    }
    out[4 * h] = nnz, out[4 * h + 1] = mx, out[4 * h + 2] = empty, out[4 * h + 3] = eff;
  }
}

}  // namespace bsa

namespace bsa {

// Query-block interleave costs of an ACSR plan, counted on the host as the
// mask planner's k_qil_cost counts them on the device: for each head with
// 32- or 64-row blocks and each candidate s = 2^c with s * mq <= nq (mq =
// 128 / bq), the key blocks that some query block of each 128-row tile
// selects, summed over the tiles. A tile's rows are expanded from the runs
// into one bit set of the head's key blocks.
void acsr_qil_costs(const bsa_problem &pr, const bsa_acsr_head *heads, int64_t *out, int64_t *kout) {
  const bool keys_ok = !pr.causal && !pr.paged && pr.dtype == BSA_BF16 && pr.num_q_heads == pr.num_kv_heads;
  for (int h = 0; h < pr.num_q_heads; ++h) {
    const int64_t bq = pr.block_q[h], bk = pr.block_k[h];
    const int64_t nq = (pr.seqlen_q + bq - 1) / bq, nk = (pr.seqlen_kv + bk - 1) / bk;
    for (int c = 0; c < kQilCands; ++c) out[h * kQilCands + c] = 0;
    for (int c = 0; c < kQilCands * kKilCands; ++c) kout[h * kQilCands * kKilCands + c] = 0;
    if (bq < 32 || bq >= 128) continue;
    const int64_t mq = 128 / bq;
    const int lm = __builtin_ctz((unsigned)mq);
    std::vector<uint64_t> bits((size_t)((nk + 63) / 64));
    const bsa_acsr_head &d = heads[h];
    for (int c = 0; c < kQilCands && (int64_t(1) << c) * mq <= nq; ++c) {
      int64_t cost = 0;
      for (int64_t t = 0; t < (nq + mq - 1) / mq; ++t) {
        std::fill(bits.begin(), bits.end(), 0ull);
        for (int64_t iq = 0; iq < mq; ++iq) {
          const int64_t qb = qblock_of(t, iq, c, lm, nq);
          if (qb >= nq) continue;
          for (int j = 0; j < d.num_runs; ++j) {
            const bsa_acsr_run &u = d.runs[j];
            const int64_t f = acsr_first(u, qb);
            if (u.stride == 1) {
              // the interval [f, f + count) clipped to [0, nk), a word at a time
              const int64_t lo = std::max<int64_t>(f, 0), hi = std::min<int64_t>(f + u.count, nk);
              for (int64_t kb = lo; kb < hi;) {
                const int64_t w = kb >> 6, end = std::min(hi, (w + 1) << 6);
                const int n = (int)(end - kb);
                bits[(size_t)w] |= (n == 64 ? ~0ull : ((1ull << n) - 1ull)) << (kb & 63);
                kb = end;
              }
              continue;
            }
            // blocks f + stride * i in [0, nk), 0 <= i < count
            int64_t i0 = f >= 0 ? 0 : (-f + u.stride - 1) / u.stride;
            for (int64_t i = i0; i < u.count; ++i) {
              const int64_t kb = f + u.stride * i;
              if (kb >= nk) break;
              bits[(size_t)(kb >> 6)] |= 1ull << (kb & 63);
            }
          }
        }
        for (uint64_t w : bits) cost += __builtin_popcountll(w);
        // 64-key tiles (two 32-key blocks) with a selected block, per key
        // interleave s' = 2^ck with 2 s' <= nk
        if (keys_ok && bk == 32)
          for (int ck = 0; ck < kKilCands && (int64_t(2) << ck) <= nk; ++ck) {
            int64_t n = 0;
            for (int64_t kt = 0; 2 * kt < nk; ++kt) {
              bool any = false;
              for (int ik = 0; ik < 2 && !any; ++ik) {
                const int64_t kb = qblock_of(kt, ik, ck, 1, nk);
                any = kb < nk && ((bits[(size_t)(kb >> 6)] >> (kb & 63)) & 1ull);
              }
              n += any;
            }
            kout[(h * kQilCands + c) * kKilCands + ck] += n;
          }
      }
      out[h * kQilCands + c] = cost;
    }
  }
}

}  // namespace bsa
