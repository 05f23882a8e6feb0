// Backward of block-sparse attention over a forward plan, for gfx950 (CDNA4).
//
// For a scalar loss with upstream gradient dO, softmax attention restricted to
// each query row's allowed keys has, by the chain rule through the softmax
// (whose Jacobian is diag(P) - P P^T),
//   dV_j = sum_i P_ij dO_i
//   dP_ij = dO_i . V_j,   Delta_i = sum_j P_ij dP_ij = dO_i . O_i
//   dS_ij = P_ij (dP_ij - Delta_i)
//   dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i,
// with P recomputed from Q, K and the forward's log-sum-exp,
// P_ij = exp(scale Q_i . K_j - LSE_i), over exactly the keys the forward
// allowed (Tessera, abstract: compute only the selected blocks; the training
// side of the same sparse attention). FlashAttention's recomputation scheme,
// which the related-work page describes as tiling plus fusion, is the model:
// no score matrix is stored.
//
// Two kernels and no atomics: every output element is accumulated by one
// workgroup in a fixed order, so the results are reproducible bit for bit.
//   k_bwd_dq    one workgroup per row of the forward plan (a query tile, or a
//               packed GQA group tile), one wave per 32 queries, walking the
//               row's key-tile list like the forward. S^T = K Q^T and
//               dP^T = V dO^T put one query in each lane (per-lane LSE and
//               Delta); dQ^T += K^T dS^T reads K^T with LDS transpose reads.
//               It also writes Delta (from O and dO) for the second kernel.
//   k_bwd_dkdv  one workgroup per (batch, kv head, key tile), one wave per 32
//               keys, K and V rows held in registers. It finds the query
//               tiles that visit its key tile by searching each plan row's
//               sorted key-tile list (or, in GQA-union mode, the group's
//               table once), then streams their queries through LDS in
//               32-row chunks, the next chunk's loads in flight while the
//               current one is computed: S = Q K^T and dP = dO V^T put one
//               key in each lane; dV^T += dO^T P and dK^T += Q^T dS take P
//               and dS straight from the accumulators as MFMA operands.
#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MFMA row permutation: when A-operand lane m supplies row perm_rows(m), the
// 32x32 accumulator value j of lane half hh belongs to row
// 16*(j/8) + 8*hh + (j%8), so each group of 8 accumulators is 8 consecutive
// rows, the B-operand layout of the next MFMA over that index.
__device__ __forceinline__ int perm_rows(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float halfwave_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)pr[0]) + __builtin_bit_cast(float, (uint32_t)pr[1]);
}

// A operand X^T of a 32x32x16 MFMA, for a row-major bf16 tile X in LDS whose
// rows are the contraction index: lane (n, hh) receives X[r0 + 8hh + i][c0 + n]
// for i = 0..7, by two transpose reads (each 16-lane group reads a 4 x 16
// block and every lane gets one column of it).
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t *x, int stride, int r0, int c0, int lane) {
  const int vj = lane & 15, vsub = (lane >> 4) & 1, hh = lane >> 5;
  const int ra = r0 + 8 * hh + (vj >> 2);
  const int col = c0 + 16 * vsub + 4 * (vj & 3);
  const uint16_t *pa = x + ra * stride + col;
  const uint16_t *pb = pa + 4 * stride;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pa);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pb);
  const s16x4 both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

// ---------------------------------------------------------------------------
// dQ (and Delta) per plan row
// ---------------------------------------------------------------------------
template <int D, int TK, int TQ>
__global__ __launch_bounds__(2 * TQ) void k_bwd_dq(BwdArgs a) {
  constexpr int T = 2 * TQ;                     // 64 lanes per 32 query rows
  constexpr int RS = D + 8;                     // LDS row stride (elements), padded
  constexpr int TILE = TK * RS;
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int LPT = (TK * CPR + T - 1) / T;   // 16-byte loads per thread per tile
  constexpr int NKB = TK / 32, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * TILE];  // K, V; two buffers

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int r = blockIdx.x;
  const int nqt = (int)a.nqt;
  const int nh = a.pack ? a.Hkv : a.Hq;
  const int qt = r % nqt, hrow = (r / nqt) % nh, b = r / (nqt * nh);
  const int head = a.pack ? hrow * a.G + (32 * wave) / a.tr : hrow;
  const int g = (a.pack ? hrow * a.G : hrow) / a.G;
  const int qbase = a.pack ? 0 : 32 * wave;
  const int64_t q0 = a.pack ? (int64_t)qt * a.tr + (32 * wave) % a.tr : (int64_t)qt * a.tq + 32 * wave;
  const int64_t qpos = q0 + n;
  const bool qvalid = qpos < a.Sq;
  const HeadMeta hm = a.hm[head];

  // Q and dO rows as B operands (lane: query n, dims 16c + 8hh .. +8); Delta.
  const uint16_t *Qp = (const uint16_t *)a.q + b * a.q_sb + head * a.q_sh + (qvalid ? qpos : 0) * a.q_ss;
  const uint16_t *Dp = (const uint16_t *)a.dout + b * a.do_sb + head * a.do_sh + (qvalid ? qpos : 0) * a.do_ss;
  const uint16_t *Op = (const uint16_t *)a.o + b * a.o_sb + head * a.o_sh + (qvalid ? qpos : 0) * a.o_ss;
  bf16x8 qb[D / 16], dob[D / 16];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const uint4 xq = qvalid ? *(const uint4 *)(Qp + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0);
    const uint4 xd = qvalid ? *(const uint4 *)(Dp + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0);
    const uint4 xo = qvalid ? *(const uint4 *)(Op + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0);
    qb[c] = __builtin_bit_cast(bf16x8, xq);
    dob[c] = __builtin_bit_cast(bf16x8, xd);
    const bf16x8 ov = __builtin_bit_cast(bf16x8, xo);
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart = __builtin_fmaf((float)ov[i], (float)dob[c][i], dpart);
  }
  const float delta = halfwave_sum(dpart);
  const int64_t rowix = ((int64_t)b * a.Hq + head) * a.Sq + qpos;
  if (qvalid && hh == 0) a.delta[rowix] = delta;
  const float L = qvalid ? a.lse[rowix] : -INFINITY;
  // exp2(s * scale_log2 - lse2) is P; +inf makes P = 0 for rows without keys
  // and for padding rows past the sequence end.
  const float lse2 = L == -INFINITY ? INFINITY : L * kLog2e;

  const int e0 = a.row_ent[2 * r], e1 = a.row_ent[2 * r + 1];
  const uint16_t *Kb = (const uint16_t *)a.k + b * a.k_sb + g * a.k_sh;
  const uint16_t *Vb = (const uint16_t *)a.v + b * a.v_sb + g * a.v_sh;
  uint4 kr[LPT], vr[LPT];
  auto load = [&](int e) {
    const int64_t k0 = (int64_t)a.ent_kt[e] * TK;
    const int64_t left = a.Skv - k0;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int c = tid + T * u;
      const int row = c / CPR, col = (c % CPR) * 8;
      const bool ok = c < TK * CPR && row < left;
      kr[u] = ok ? *(const uint4 *)(Kb + (k0 + row) * a.k_ss + col) : make_uint4(0, 0, 0, 0);
      vr[u] = ok ? *(const uint4 *)(Vb + (k0 + row) * a.v_ss + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
    uint16_t *ks = lds + buf * 2 * TILE, *vs = ks + TILE;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int c = tid + T * u;
      if (c < TK * CPR) {
        const int row = c / CPR, col = (c % CPR) * 8;
        *(uint4 *)(ks + row * RS + col) = kr[u];
        *(uint4 *)(vs + row * RS + col) = vr[u];
      }
    }
  };

  // Live-bit geometry of this wave's rows (as in the forward).
  const int iq_lo = qbase >> hm.lq;
  const int niq = hm.lq >= 5 ? 1 : (32 >> hm.lq);
  const uint64_t wbits = ((1ull << (hm.mk * niq)) - 1ull) << (iq_lo * hm.mk);
  const int qsub = ((qbase + n) >> hm.lq) * hm.mk;
  const int skv32 = (int)a.Skv;
  const int qlim0 = (int)max<int64_t>(-64, min<int64_t>(q0 + a.off, a.Skv));

  f32x16 dq[NDB];
#pragma unroll
  for (int u = 0; u < NDB; ++u) dq[u] = f32x16{};

  if (e0 < e1) {
    load(e0);
    store(0);
    __syncthreads();
  }
  for (int e = e0; e < e1; ++e) {
    const int buf = (e - e0) & 1;
    if (e + 1 < e1) load(e + 1);
    const uint16_t *ks = lds + buf * 2 * TILE, *vs = ks + TILE;
    const int kb0 = a.ent_kt[e] * TK;
    const uint32_t live = a.ent_live[e];
    const bool need = (kb0 + TK > skv32) || (a.causal && kb0 + TK - 1 > qlim0) ||
                      ((uint64_t)live & wbits) != wbits;
    // Allowed keys of this lane's query as bit masks over the tile.
    uint64_t km[(TK + 63) / 64];
#pragma unroll
    for (int w64 = 0; w64 < (TK + 63) / 64; ++w64) km[w64] = ~0ull;
    if (need) {
      const uint32_t lbits = live >> qsub;
      int lim = skv32 - kb0;
      if (a.causal) lim = min(lim, qlim0 + n + 1 - kb0);
      const int klim = max(0, min(lim, TK));
      const int ak = 1 << hm.lk;
      const uint64_t sub = ak >= 64 ? ~0ull : ((1ull << ak) - 1ull);
#pragma unroll
      for (int w64 = 0; w64 < (TK + 63) / 64; ++w64) {
        uint64_t m = 0;
        for (int ik = 0; ik < hm.mk; ++ik)
          if ((lbits >> ik) & 1u) {
            const int k0b = ik * ak - 64 * w64;
            if (k0b >= 64 || k0b + ak <= 0) continue;
            m |= k0b >= 0 ? sub << k0b : sub >> -k0b;
          }
        const int lo = klim - 64 * w64;
        m &= lo >= 64 ? ~0ull : (lo <= 0 ? 0ull : ((1ull << lo) - 1ull));
        km[w64] = m >> (8 * hh);  // accumulator keys are offset by 8 on the upper half-wave
      }
    }
#pragma unroll
    for (int t = 0; t < NKB; ++t) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const uint16_t *kr0 = ks + (32 * t + perm_rows(n)) * RS + 8 * hh;
      const uint16_t *vr0 = vs + (32 * t + perm_rows(n)) * RS + 8 * hh;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(kr0 + 16 * c), qb[c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(vr0 + 16 * c), dob[c], dp, 0, 0, 0);
      }
      uint32_t dsw[8];
#pragma unroll
      for (int jj = 0; jj < 16; jj += 2) {
        float ds2[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int kl = 32 * t + 16 * ((jj + x) >> 3) + ((jj + x) & 7);  // without the 8*hh term
          const bool ok = (km[kl / 64] >> (kl % 64)) & 1ull;
          const float p = ok ? fexp2(__builtin_fmaf(s[jj + x], a.scale_log2, -lse2)) : 0.f;
          ds2[x] = p * (dp[jj + x] - delta);
        }
        dsw[jj / 2] = pack_bf16x2(ds2[0], ds2[1]);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 bop = as_bf16x8(dsw[4 * c2], dsw[4 * c2 + 1], dsw[4 * c2 + 2], dsw[4 * c2 + 3]);
#pragma unroll
        for (int u = 0; u < NDB; ++u)
          dq[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(ks, RS, 32 * t + 16 * c2, 32 * u, lane),
                                                          bop, dq[u], 0, 0, 0);
      }
    }
    if (e + 1 < e1) store(buf ^ 1);
    __syncthreads();
  }

  if (qvalid) {
    uint16_t *dp = (uint16_t *)a.dq + b * a.dq_sb + head * a.dq_sh + qpos * a.dq_ss;
#pragma unroll
    for (int u = 0; u < NDB; ++u)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * u + 8 * q4 + 4 * hh;
        *(uint2 *)(dp + d0) = make_uint2(pack_bf16x2(dq[u][4 * q4] * a.scale, dq[u][4 * q4 + 1] * a.scale),
                                         pack_bf16x2(dq[u][4 * q4 + 2] * a.scale, dq[u][4 * q4 + 3] * a.scale));
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV per (batch, kv head, key tile)
// ---------------------------------------------------------------------------
template <int D, int TK>
__global__ __launch_bounds__(2 * TK) void k_bwd_dkdv(BwdArgs a) {
  constexpr int T = 2 * TK;                     // 64 lanes per 32 keys
  constexpr int RS = D + 8;
  constexpr int CH = 32 * RS;                   // one 32-row chunk of Q or dO
  constexpr int CPR = D / 8;
  constexpr int LPT = (32 * CPR + T - 1) / T;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * CH];  // Q, dO; two buffers
  __shared__ float s_lse[2][32], s_del[2][32];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int nkt = (int)a.nkt, nqt = (int)a.nqt;
  const int item = blockIdx.x;
  const int kt = item % nkt, g = (item / nkt) % a.Hkv, b = item / (nkt * a.Hkv);
  const int kb0 = kt * TK;
  const int klocal = 32 * wave + n;            // this lane's key within the tile
  const int key = kb0 + klocal;
  const int skv32 = (int)a.Skv, sq32 = (int)a.Sq;  // sequence lengths are below 2^31
  const bool kvalid = key < skv32;

  // K and V rows of this lane's key as B operands (dims 16c + 8hh .. +8).
  bf16x8 kb[D / 16], vb[D / 16];
  {
    const uint16_t *kp = (const uint16_t *)a.k + b * a.k_sb + g * a.k_sh + (int64_t)(kvalid ? key : 0) * a.k_ss;
    const uint16_t *vp = (const uint16_t *)a.v + b * a.v_sb + g * a.v_sh + (int64_t)(kvalid ? key : 0) * a.v_ss;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      kb[c] = __builtin_bit_cast(bf16x8, kvalid ? *(const uint4 *)(kp + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0));
      vb[c] = __builtin_bit_cast(bf16x8, kvalid ? *(const uint4 *)(vp + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0));
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int u = 0; u < NDB; ++u) dk[u] = f32x16{}, dv[u] = f32x16{};

  // ---- enumeration of the query chunks that visit this key tile ----
  // A chunk is 32 consecutive queries of one head. Non-union: the rows
  // (b, h, qt) of the group's heads whose sorted key-tile list holds kt
  // (binary search, 64 rows per ballot), then the row's chunks. Union: the
  // group's table holds kt or not; if it does, every causally feasible chunk
  // of every head of the group visits it.
  const int cpr = a.tq / 32;                    // chunks per plan row (non-union)
  const int nch = (sq32 + 31) / 32;             // chunks per head (union)
  const int lb = a.nlb == 1 ? 0 : b;
  int h = g * a.G - 1, qtb = 0, qt = 0, ci = 0, cend = 0;
  uint64_t bal = 0;
  uint32_t lvl = 0, rl = 0;
  HeadMeta hm{};
  uint32_t ulive = 0;
  if (a.uni) {
    const int l = lb * a.Hkv + g;
    int lo = a.list_off[l], hi = a.list_off[l + 1];
    while (lo < hi) {
      const int mid = lo + ((hi - lo) >> 1);
      if (a.ent_kt[mid] < kt) lo = mid + 1;
      else hi = mid;
    }
    ulive = (lo < a.list_off[l + 1] && a.ent_kt[lo] == kt) ? a.ent_live[lo] : 0u;
  }
  auto search = [&]() {
    const int q = qtb + lane;
    uint32_t lv = 0;
    if (q < nqt) {
      const int64_t row = ((int64_t)b * a.Hq + h) * a.nqt + q;
      int lo = a.row_ent[2 * row], hi = a.row_ent[2 * row + 1];
      const int end = hi;
      while (lo < hi) {
        const int mid = lo + ((hi - lo) >> 1);
        if (a.ent_kt[mid] < kt) lo = mid + 1;
        else hi = mid;
      }
      if (lo < end && a.ent_kt[lo] == kt) lv = a.ent_live[lo];
    }
    lvl = lv;
    bal = __ballot(lv != 0u);
  };
  // Next chunk: its head, first query, offset within its plan row, live bits.
  struct Chunk {
    int h, q0, qoff;
    uint32_t live;
    int lq, lk, mk;
  };
  auto next = [&](Chunk &o) -> bool {
    for (;;) {
      if (ci < cend) {
        const int cc = ci++;
        const int cq0 = a.uni ? 32 * cc : qt * a.tq + 32 * cc;
        if (cq0 >= sq32) {
          ci = cend;
          continue;
        }
        const int last = min(cq0 + 31, sq32 - 1);
        if (a.causal && (int64_t)kb0 > (int64_t)last + a.off) continue;
        const int qoff = a.uni ? 0 : 32 * cc;
        const uint32_t live = a.uni ? ulive : rl;
        if (!a.uni) {
          const int iq0 = qoff >> hm.lq, niq = hm.lq >= 5 ? 1 : (32 >> hm.lq);
          const uint64_t cb = ((1ull << (hm.mk * niq)) - 1ull) << (iq0 * hm.mk);
          if (((uint64_t)live & cb) == 0) continue;
        }
        o = Chunk{h, cq0, qoff, live, hm.lq, hm.lk, hm.mk};
        return true;
      }
      if (!a.uni && bal) {
        const int bit = __builtin_ctzll(bal);
        bal &= bal - 1;
        qt = qtb + bit;
        rl = __builtin_amdgcn_readlane(lvl, bit);
        ci = 0, cend = cpr;
        continue;
      }
      if (!a.uni && h >= g * a.G && qtb + 64 < nqt) {
        qtb += 64;
        search();
        continue;
      }
      if (++h >= (g + 1) * a.G) return false;
      hm = a.hm[h];
      if (a.uni) {
        if (ulive == 0) return false;
        // first chunk whose last query can reach the tile's first key
        const int64_t need = (int64_t)kb0 - a.off - 31;
        ci = (!a.causal || need <= 0) ? 0 : (int)min<int64_t>((need + 31) / 32, nch);
        cend = nch;
      } else {
        qtb = 0;
        search();
      }
    }
  };

  // ---- chunk staging: Q and dO rows, LSE (log2, +inf for no keys) and Delta ----
  uint4 qr[LPT], dr[LPT];
  float lse_r = 0.f, del_r = 0.f;
  auto load = [&](const Chunk &c) {
    const uint16_t *Qp = (const uint16_t *)a.q + b * a.q_sb + c.h * a.q_sh;
    const uint16_t *Dp = (const uint16_t *)a.dout + b * a.do_sb + c.h * a.do_sh;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int x = tid + T * u;
      const int row = x / CPR, col = (x % CPR) * 8;
      const bool ok = x < 32 * CPR && c.q0 + row < sq32;
      qr[u] = ok ? *(const uint4 *)(Qp + (int64_t)(c.q0 + row) * a.q_ss + col) : make_uint4(0, 0, 0, 0);
      dr[u] = ok ? *(const uint4 *)(Dp + (int64_t)(c.q0 + row) * a.do_ss + col) : make_uint4(0, 0, 0, 0);
    }
    if (tid < 32) {
      const bool ok = c.q0 + tid < sq32;
      const int64_t ix = ((int64_t)b * a.Hq + c.h) * a.Sq + c.q0 + tid;
      const float L = ok ? a.lse[ix] : -INFINITY;
      lse_r = L == -INFINITY ? INFINITY : L * kLog2e;
      del_r = ok ? a.delta[ix] : 0.f;
    }
  };
  auto store = [&](int buf) {
    uint16_t *qs = lds + buf * 2 * CH, *ds = qs + CH;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int x = tid + T * u;
      if (x < 32 * CPR) {
        const int row = x / CPR, col = (x % CPR) * 8;
        *(uint4 *)(qs + row * RS + col) = qr[u];
        *(uint4 *)(ds + row * RS + col) = dr[u];
      }
    }
    if (tid < 32) s_lse[buf][tid] = lse_r, s_del[buf][tid] = del_r;
  };

  Chunk cur{}, nxt{};
  bool have = next(cur);
  if (have) {
    load(cur);
    store(0);
    __syncthreads();
  }
  int buf = 0;
  while (have) {
    const bool more = next(nxt);
    if (more) load(nxt);
    const uint16_t *qs = lds + buf * 2 * CH, *dos = qs + CH;

    // S = Q K^T and dP = dO V^T: lane = key n, accumulator j = query row
    // 16*(j/8) + 8*hh + (j%8) of the chunk.
    f32x16 s = f32x16{}, dp = f32x16{};
    const uint16_t *qrow = qs + perm_rows(n) * RS + 8 * hh;
    const uint16_t *drow = dos + perm_rows(n) * RS + 8 * hh;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(qrow + 16 * c), kb[c], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(drow + 16 * c), vb[c], dp, 0, 0, 0);
    }
    // Is every (query, key) pair of this wave's 32 x 32 block allowed?
    const int ik0 = (32 * wave) >> cur.lk, nik = cur.lk >= 5 ? 1 : (32 >> cur.lk);
    const int iq0 = cur.qoff >> cur.lq, niq = cur.lq >= 5 ? 1 : (32 >> cur.lq);
    uint64_t wb = 0;
    for (int iq = 0; iq < niq; ++iq) wb |= ((1ull << nik) - 1ull) << ((iq0 + iq) * cur.mk + ik0);
    const bool need = ((uint64_t)cur.live & wb) != wb || kb0 + 32 * wave + 31 >= skv32 ||
                      cur.q0 + 31 >= sq32 || (a.causal && (int64_t)kb0 + 32 * wave + 31 > (int64_t)cur.q0 + a.off);
    uint32_t pw[8], dw[8];
#pragma unroll
    for (int jj = 0; jj < 16; jj += 2) {
      float pp[2], dd[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int qrw = 16 * ((jj + x) >> 3) + 8 * hh + ((jj + x) & 7);
        bool ok = true;
        if (need) {
          const int bit = ((cur.qoff + qrw) >> cur.lq) * cur.mk + (klocal >> cur.lk);
          ok = ((cur.live >> bit) & 1u) && kvalid && cur.q0 + qrw < sq32 &&
               (!a.causal || (int64_t)key <= (int64_t)cur.q0 + qrw + a.off);
        }
        const float p = ok ? fexp2(__builtin_fmaf(s[jj + x], a.scale_log2, -s_lse[buf][qrw])) : 0.f;
        pp[x] = p;
        dd[x] = p * (dp[jj + x] - s_del[buf][qrw]);
      }
      pw[jj / 2] = pack_bf16x2(pp[0], pp[1]);
      dw[jj / 2] = pack_bf16x2(dd[0], dd[1]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS (rows d, columns keys).
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const bf16x8 pb = as_bf16x8(pw[4 * c2], pw[4 * c2 + 1], pw[4 * c2 + 2], pw[4 * c2 + 3]);
      const bf16x8 db = as_bf16x8(dw[4 * c2], dw[4 * c2 + 1], dw[4 * c2 + 2], dw[4 * c2 + 3]);
#pragma unroll
      for (int u = 0; u < NDB; ++u) {
        dv[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(dos, RS, 16 * c2, 32 * u, lane), pb, dv[u], 0, 0, 0);
        dk[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(qs, RS, 16 * c2, 32 * u, lane), db, dk[u], 0, 0, 0);
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    cur = nxt;
    have = more;
    buf ^= 1;
  }

  if (kvalid) {
    uint16_t *kp = (uint16_t *)a.dk + b * a.dk_sb + g * a.dk_sh + (int64_t)key * a.dk_ss;
    uint16_t *vp = (uint16_t *)a.dv + b * a.dv_sb + g * a.dv_sh + (int64_t)key * a.dv_ss;
#pragma unroll
    for (int u = 0; u < NDB; ++u)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * u + 8 * q4 + 4 * hh;
        *(uint2 *)(kp + d0) = make_uint2(pack_bf16x2(dk[u][4 * q4] * a.scale, dk[u][4 * q4 + 1] * a.scale),
                                         pack_bf16x2(dk[u][4 * q4 + 2] * a.scale, dk[u][4 * q4 + 3] * a.scale));
        *(uint2 *)(vp + d0) = make_uint2(pack_bf16x2(dv[u][4 * q4], dv[u][4 * q4 + 1]),
                                         pack_bf16x2(dv[u][4 * q4 + 2], dv[u][4 * q4 + 3]));
      }
  }
}

template <int D, int TK>
void launch_dq(const BwdArgs &a, int tq, unsigned grid, hipStream_t s) {
  if (tq == 256) hipLaunchKernelGGL((k_bwd_dq<D, TK, 256>), dim3(grid), dim3(512), 0, s, a);
  else hipLaunchKernelGGL((k_bwd_dq<D, TK, 128>), dim3(grid), dim3(256), 0, s, a);
}

template <int D>
void launch_d(const BwdArgs &a, unsigned dq_grid, unsigned kv_grid, hipStream_t s) {
  if (dq_grid) {
    if (a.tk == 128) launch_dq<D, 128>(a, a.tq, dq_grid, s);
    else launch_dq<D, 64>(a, a.tq, dq_grid, s);
  }
  if (kv_grid) {
    if (a.tk == 128) hipLaunchKernelGGL((k_bwd_dkdv<D, 128>), dim3(kv_grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dkdv<D, 64>), dim3(kv_grid), dim3(128), 0, s, a);
  }
}

}  // namespace

bsa_status backward_launch(const Plan &p, const BwdArgs &a, hipStream_t s) {
  const int64_t kv_items = (int64_t)p.B * p.Hkv * p.nkt;
  if (p.nrows > 0x7fffffff || kv_items > 0x7fffffff)
    return fail(BSA_ERR_UNSUPPORTED, "too many tiles for one launch");
  const unsigned dq_grid = (unsigned)p.nrows, kv_grid = (unsigned)kv_items;
  if (p.D == 128) launch_d<128>(a, dq_grid, kv_grid, s);
  else launch_d<64>(a, dq_grid, kv_grid, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BSA_ERR_HIP, std::string("backward launch: ") + hipGetErrorString(e));
  return BSA_OK;
}

}  // namespace bsa
