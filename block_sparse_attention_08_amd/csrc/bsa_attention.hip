// Fused block-sparse attention forward for gfx950 (CDNA4).
//
// Computes, for every work item of a plan (one physical query tile and a range
// of its key-tile list), exact softmax attention restricted to the selected
// tiles (Tessera, abstract: compute only the blocks the logical mask selects)
// with an online softmax, the tiling-and-fusion scheme of FlashAttention that
// the related-work page describes (attention as matrix products interleaved
// with a softmax).
//
// Layout of the work on the chip:
//   - A workgroup is 4 waves; each wave owns 32 query rows, so a physical
//     query tile is 128 rows (or, for a packed GQA group, 128/G positions of
//     each of its G heads: the heads share every K/V tile).
//   - Scores are computed transposed, S^T = K Q^T, with the 32x32 MFMA: each
//     lane then holds one query and 16 keys per 32-key block, so the row max
//     and row sum are in-lane reductions plus one exchange between the two
//     half-waves. The key rows feeding the MFMA are permuted (bits 2 and 3 of
//     the row index swapped) so that each lane's 8 consecutive accumulator
//     values are 8 consecutive keys, which is exactly the B-operand layout of
//     the following P V^T MFMA: P never leaves registers.
//   - O is accumulated transposed, O^T = V^T P^T, so each lane owns one query
//     and the online-softmax rescale is per lane.
//   - K and V tiles are double buffered in LDS: the loads of the next tiles
//     are in flight while the current one is computed. The bf16 kernel
//     loads them straight from HBM into XOR-swizzled row-major LDS (buffer
//     loads with an LDS destination) and reads the V^T operands with LDS
//     transpose reads; the fp32 kernel stages its tiles through registers.
//     Rows beyond the sequence read as zero and are masked.
//   - Workgroups are persistent (the bf16 kernel: one queue of items per XCD,
//     taken with atomic tickets, in row order, longest-first, or row order
//     dealt to the XCDs in blocks; the fp32 kernel: items i, i + grid, ...),
//     so consecutive items (neighbouring query tiles that share key tiles)
//     run on the same XCD and reuse its L2.
#include "bsa_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kTileQ = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#define HIP_TRY(expr)                                                          \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess)                                                      \
      return fail(BSA_ERR_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key row (within a 32-key block) that MFMA A-operand lane m supplies, so that
// output accumulator j of lane half hh holds key 16*(j/8) + 8*hh + (j%8).
__device__ __forceinline__ int perm_bf16(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
// fp32 variant: accumulator j of half hh holds key 2*j + hh.
__device__ __forceinline__ int perm_f32(int m) { return 8 * (m >> 3) + 2 * (m & 3) + ((m >> 2) & 1); }

// Key offset (within a 32-key block) of accumulator j for lane half hh.
template <bool BF>
__device__ __forceinline__ int acc_key(int j, int hh) {
  if constexpr (BF) return 16 * (j >> 3) + 8 * hh + (j & 7);
  else return 2 * j + hh;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Geometry of the wave's 32 query rows for row r of the plan.
struct RowGeo {
  int b, head, g;
  int64_t q0;  // first query position of this wave
  int qbase;   // offset of the wave's first row within the physical tile (live bits)
};

__device__ __forceinline__ RowGeo row_geo(const AttnArgs &a, int r, int wave) {
  RowGeo o;
  const int nh = a.pack ? a.Hkv : a.Hq;
  const int64_t qt = r % a.nqt;
  const int hrow = (int)((r / a.nqt) % nh);
  o.b = (int)(r / (a.nqt * nh));
  if (a.pack) {
    o.head = hrow * a.G + (32 * wave) / a.tr;
    o.q0 = qt * a.tr + (32 * wave) % a.tr;
    o.qbase = 0;
  } else {
    o.head = hrow;
    o.q0 = tile_query(a.hm[hrow], __builtin_ctz(a.tq), qt, 32 * wave);  // (query-block interleave)
    o.qbase = 32 * wave;
  }
  o.g = o.head / a.G;
  return o;
}

// Batch, head and query position of row R (0 .. Tq-1) of plan row r. Packed
// tiles (pack 1) hold the group's heads one after another, tr positions each;
// interleaved tiles (pack 2) hold position-major rows, heads interleaved
// (row R: head R mod G, position R / G), so the rows of a few positions all
// fall in the first wave.
struct RowPos {
  int b, head;
  int64_t q;
};
__device__ __forceinline__ RowPos tile_row(const AttnArgs &a, int r, int R) {
  const int nh = a.pack ? a.Hkv : a.Hq;
  const int64_t qt = r % a.nqt;
  const int hrow = (int)((r / a.nqt) % nh);
  RowPos o;
  o.b = (int)(r / (a.nqt * nh));
  if (a.pack == 2) {
    o.head = hrow * a.G + R % a.G, o.q = qt * a.tr + R / a.G;
  } else if (a.pack) {
    o.head = hrow * a.G + R / a.tr, o.q = qt * a.tr + R % a.tr;
  } else {
    o.head = hrow, o.q = tile_query(a.hm[hrow], __builtin_ctz(a.tq), qt, R);
  }
  return o;
}

template <int D, int TK, bool BF>
struct Cfg {
  using E = typename std::conditional<BF, uint16_t, float>::type;
  static constexpr int EPV = 16 / sizeof(E);            // elements per 16-byte vector
  static constexpr int KS = D + EPV;                    // K row stride (elements), padded
  static constexpr int VS = BF ? TK + 8 : D + EPV;      // V^T row stride (bf16) or V row stride
  static constexpr int KBUF = TK * KS;
  static constexpr int VBUF = BF ? D * VS : TK * VS;
  static constexpr int BUF = KBUF + VBUF;
  static constexpr int NKB = TK / 32;                   // 32-key score blocks
  static constexpr int NDB = D / 32;                    // 32-wide output blocks
  static constexpr int KCH = TK * D / EPV;              // 16-byte chunks per K tile
  static constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  // bf16 V: blocks of 4 keys x 8 dims, transposed into LDS.
  static constexpr int VBLK = BF ? (TK / 4) * (D / 8) : KCH;
  static constexpr int VPT = (VBLK + kThreads - 1) / kThreads;
};

template <int D, int TK, bool BF>
__global__ __launch_bounds__(kThreads) void k_attn(AttnArgs a) {
  using C = Cfg<D, TK, BF>;
  using E = typename C::E;
  __shared__ __attribute__((aligned(16))) E lds[2 * C::BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int nitems = a.counters[CNT_ITEMS];
  const int grid = gridDim.x;
  int lid = blockIdx.x;
  if ((grid & 7) == 0) lid = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);

  const E *__restrict__ Q = (const E *)a.q;
  const E *__restrict__ K = (const E *)a.k;
  const E *__restrict__ V = (const E *)a.v;

  for (int it = lid; it < nitems; it += grid) {
    const int4 item = ((const int4 *)a.items)[it];
    const int r = item.x, e0 = item.y, e1 = item.z, slot = item.w;
    const RowGeo geo = row_geo(a, r, wave);
    // All waves of the workgroup share b and kv group g (packed heads are one group).
    const RowGeo geo0 = row_geo(a, r, 0);
    const HeadMeta hm = a.hm[geo.head];
    const int64_t qpos = geo.q0 + n;
    const bool qvalid = qpos < a.Sq;

    // Q fragments (MFMA B operand of S^T = K Q^T), loaded once per item.
    bf16x8 qb[BF ? D / 16 : 1];
    float qf[BF ? 1 : D / 2];
    {
      const E *qp = Q + geo.b * a.q_sb + geo.head * a.q_sh + (qvalid ? qpos : 0) * a.q_ss;
      if constexpr (BF) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          uint4 x = qvalid ? *(const uint4 *)(qp + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0);
          qb[c] = __builtin_bit_cast(bf16x8, x);
        }
      } else {
#pragma unroll
        for (int c = 0; c < D / 2; ++c) qf[c] = qvalid ? qp[2 * c + hh] : 0.f;
      }
    }

    f32x16 o[C::NDB];
#pragma unroll
    for (int u = 0; u < C::NDB; ++u) o[u] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // ---- K/V tile staging ----
    uint4 kreg[C::KPT];
    uint4 vreg[BF ? 4 * C::VPT : C::VPT];
    // First row of key tile e in a K or V tensor (dense, or a page of the pool).
    auto kv_base = [&](const E *base, int64_t sb, int64_t sh, int64_t ss, int e) -> const E * {
      const int64_t k0 = (int64_t)a.ent_kt[e] * TK;
      if (a.paged) return base + (int64_t)a.ent_page[e] * sb + (k0 % a.P) * ss + geo0.g * sh;
      return base + geo0.b * sb + geo0.g * sh + k0 * ss;
    };
    auto load_tile = [&](int e) {
      const int64_t left = a.Skv - (int64_t)a.ent_kt[e] * TK;  // rows of the tile that exist
      const E *kb = kv_base(K, a.k_sb, a.k_sh, a.k_ss, e);
      const E *vb = kv_base(V, a.v_sb, a.v_sh, a.v_ss, e);
#pragma unroll
      for (int u = 0; u < C::KPT; ++u) {
        const int c = tid + kThreads * u;
        const int row = c / (D / C::EPV), col = (c % (D / C::EPV)) * C::EPV;
        kreg[u] = (c < C::KCH && row < left) ? *(const uint4 *)(kb + row * a.k_ss + col) : make_uint4(0, 0, 0, 0);
      }
      if constexpr (BF) {
#pragma unroll
        for (int u = 0; u < C::VPT; ++u) {
          const int bi = tid + kThreads * u;
          const int kg = bi % (TK / 4), dg = bi / (TK / 4);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = 4 * kg + rr;
            vreg[4 * u + rr] = (bi < C::VBLK && row < left) ? *(const uint4 *)(vb + row * a.v_ss + 8 * dg)
                                                            : make_uint4(0, 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < C::VPT; ++u) {
          const int c = tid + kThreads * u;
          const int row = c / (D / C::EPV), col = (c % (D / C::EPV)) * C::EPV;
          vreg[u] = (c < C::KCH && row < left) ? *(const uint4 *)(vb + row * a.v_ss + col) : make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto store_tile = [&](int buf) {
      E *ks = lds + buf * C::BUF;
      E *vs = ks + C::KBUF;
#pragma unroll
      for (int u = 0; u < C::KPT; ++u) {
        const int c = tid + kThreads * u;
        if (c < C::KCH) {
          const int row = c / (D / C::EPV), col = (c % (D / C::EPV)) * C::EPV;
          *(uint4 *)(ks + row * C::KS + col) = kreg[u];
        }
      }
      if constexpr (BF) {
#pragma unroll
        for (int u = 0; u < C::VPT; ++u) {
          const int bi = tid + kThreads * u;
          if (bi < C::VBLK) {
            const int kg = bi % (TK / 4), dg = bi / (TK / 4);
            const uint32_t *w0 = (const uint32_t *)&vreg[4 * u + 0];
            const uint32_t *w1 = (const uint32_t *)&vreg[4 * u + 1];
            const uint32_t *w2 = (const uint32_t *)&vreg[4 * u + 2];
            const uint32_t *w3 = (const uint32_t *)&vreg[4 * u + 3];
#pragma unroll
            for (int d2 = 0; d2 < 4; ++d2) {
              // even dim 8*dg + 2*d2: low halves; odd dim: high halves.
              uint2 ev, od;
              ev.x = __builtin_amdgcn_perm(w1[d2], w0[d2], 0x05040100u);
              ev.y = __builtin_amdgcn_perm(w3[d2], w2[d2], 0x05040100u);
              od.x = __builtin_amdgcn_perm(w1[d2], w0[d2], 0x07060302u);
              od.y = __builtin_amdgcn_perm(w3[d2], w2[d2], 0x07060302u);
              *(uint2 *)(vs + (8 * dg + 2 * d2) * C::VS + 4 * kg) = ev;
              *(uint2 *)(vs + (8 * dg + 2 * d2 + 1) * C::VS + 4 * kg) = od;
            }
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < C::VPT; ++u) {
          const int c = tid + kThreads * u;
          if (c < C::KCH) {
            const int row = c / (D / C::EPV), col = (c % (D / C::EPV)) * C::EPV;
            *(uint4 *)(vs + row * C::VS + col) = vreg[u];
          }
        }
      }
    };

    // Live bits of this wave's rows: sub-blocks iq_lo .. iq_lo + niq - 1.
    const int iq_lo = geo.qbase >> hm.lq;
    const int niq = hm.lq >= 5 ? 1 : (32 >> hm.lq);
    const uint64_t wbits = ((1ull << (hm.mk * niq)) - 1ull) << (iq_lo * hm.mk);
    const uint32_t wbits32 = (uint32_t)wbits;  // the wave's live bits (at most 32 per tile)

    if (e0 < e1) {
      load_tile(e0);
      store_tile(0);
      __syncthreads();
    }
    for (int e = e0; e < e1; ++e) {
      const int buf = (e - e0) & 1;
      if (e + 1 < e1) load_tile(e + 1);
      const E *ks = lds + buf * C::BUF;
      const E *vs = ks + C::KBUF;

      // ---- S^T = K Q^T ----
      f32x16 s[C::NKB];
#pragma unroll
      for (int t = 0; t < C::NKB; ++t) {
        s[t] = f32x16{};
        if constexpr (BF) {
          const E *kr = ks + (32 * t + perm_bf16(n)) * C::KS + 8 * hh;
#pragma unroll
          for (int c = 0; c < D / 16; ++c) {
            bf16x8 af = __builtin_bit_cast(bf16x8, *(const uint4 *)(kr + 16 * c));
            s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qb[c], s[t], 0, 0, 0);
          }
        } else {
          const E *kr = ks + (32 * t + perm_f32(n)) * C::KS + hh;
#pragma unroll
          for (int c = 0; c < D / 2; ++c)
            s[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * c], qf[c], s[t], 0, 0, 0);
        }
      }

      // ---- mask (only tiles that need it) ----
      const int64_t kbase = (int64_t)a.ent_kt[e] * TK;
      const uint32_t live = a.ent_live[e];
      const bool need = (kbase + TK > a.Skv) || (a.causal && kbase + TK - 1 > geo.q0 + a.off) ||
                        ((uint64_t)live & wbits) != wbits;
      if (need) {
        const int qsub = ((geo.qbase + n) >> hm.lq) * hm.mk;
#pragma unroll
        for (int t = 0; t < C::NKB; ++t)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kl = 32 * t + acc_key<BF>(j, hh);
            const int64_t kpos = kbase + kl;
            const bool ok = ((live >> (qsub + (kl >> hm.lk))) & 1u) && kpos < a.Skv &&
                            (!a.causal || kpos <= qpos + a.off);
            if (!ok) s[t][j] = -INFINITY;
          }
      }

      // ---- online softmax (log2 domain) ----
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < C::NKB; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[t][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fexp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < C::NKB; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = fexp2(__builtin_fmaf(s[t][j], a.scale_log2, -m_use));
          s[t][j] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int u = 0; u < C::NDB; ++u) o[u] *= alpha;

      // ---- O^T += V^T P^T ----
      if constexpr (BF) {
        bf16x8 pb[C::NKB][2];
#pragma unroll
        for (int t = 0; t < C::NKB; ++t)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            uint4 w;
            w.x = pack_bf16x2(s[t][8 * c2 + 0], s[t][8 * c2 + 1]);
            w.y = pack_bf16x2(s[t][8 * c2 + 2], s[t][8 * c2 + 3]);
            w.z = pack_bf16x2(s[t][8 * c2 + 4], s[t][8 * c2 + 5]);
            w.w = pack_bf16x2(s[t][8 * c2 + 6], s[t][8 * c2 + 7]);
            pb[t][c2] = __builtin_bit_cast(bf16x8, w);
          }
#pragma unroll
        for (int u = 0; u < C::NDB; ++u) {
          const E *vr = vs + (32 * u + n) * C::VS + 8 * hh;
#pragma unroll
          for (int t = 0; t < C::NKB; ++t)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
              bf16x8 af = __builtin_bit_cast(bf16x8, *(const uint4 *)(vr + 32 * t + 16 * c2));
              o[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[t][c2], o[u], 0, 0, 0);
            }
        }
      } else {
#pragma unroll
        for (int u = 0; u < C::NDB; ++u)
#pragma unroll
          for (int t = 0; t < C::NKB; ++t)
#pragma unroll
            for (int c = 0; c < 16; ++c) {
              const float av = vs[(32 * t + 2 * c + hh) * C::VS + 32 * u + n];
              o[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, s[t][c], o[u], 0, 0, 0);
            }
      }

      if (e + 1 < e1) store_tile(buf ^ 1);
      __syncthreads();
    }

    // ---- finalize ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    if (slot < 0) {
      if (qvalid) {
        E *op = (E *)a.o + geo.b * a.o_sb + geo.head * a.o_sh + qpos * a.o_ss;
#pragma unroll
        for (int u = 0; u < C::NDB; ++u)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * u + 8 * q4 + 4 * hh;
            const float x0 = o[u][4 * q4] * inv, x1 = o[u][4 * q4 + 1] * inv;
            const float x2 = o[u][4 * q4 + 2] * inv, x3 = o[u][4 * q4 + 3] * inv;
            if constexpr (BF) {
              *(uint2 *)(op + d0) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
            } else {
              *(float4 *)(op + d0) = make_float4(x0, x1, x2, x3);
            }
          }
        if (hh == 0) a.lse[((int64_t)geo.b * a.Hq + geo.head) * a.Sq + qpos] = lse;
      }
    } else if (qvalid && slot < a.part_slots) {  // the combine reads partials of existing rows only
      const int64_t prow = (int64_t)slot * kTileQ + 32 * wave + n;
      float *pp = a.part_o + prow * D;
#pragma unroll
      for (int u = 0; u < C::NDB; ++u)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * u + 8 * q4 + 4 * hh;
          *(float4 *)(pp + d0) = make_float4(o[u][4 * q4] * inv, o[u][4 * q4 + 1] * inv,
                                             o[u][4 * q4 + 2] * inv, o[u][4 * q4 + 3] * inv);
        }
      if (hh == 0) a.part_lse[prow] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel: K/V tiles stream from HBM straight into LDS with buffer loads
// (no register staging; rows past the end of the sequence read as zero from
// the buffer range check), in an XOR-swizzled row-major layout that keeps the
// MFMA operand reads free of bank conflicts. The V^T operand of P V^T is read
// with the LDS transpose read (ds_read_b64_tr_b16): two reads give a lane 8
// consecutive keys of one head-dim column. The online softmax rescales O only
// when a row maximum has grown by more than 2^8 since the last rescale; the
// final O / l is the same quantity either way.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// A workgroup owns a TQ-row query tile (128 or 256) split into 32-row
// slices, one per wave (four or eight waves).
template <int D, int TK, int TQ>
struct CfgB {
  static constexpr int WAVES = TQ / 32;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWB = D * 2;                     // bytes per K/V row in LDS
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int TILEB = TK * ROWB;                // bytes of one K (or V) tile
  static constexpr int LOADS = TILEB / (THREADS * 16);   // 16-byte loads per thread per tile
  static constexpr int RPL = THREADS / CPR;              // tile rows covered by one load
  static constexpr int NKB = TK / 32;
  static constexpr int NDB = D / 32;
  // K rows: 16-byte chunk c of row r sits at chunk c ^ swz_k(r); V rows: c ^ swz_v(r).
  static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
  // A thread's slot in load u sits RPL rows below its slot in load 0 with the
  // same swizzle, so one per-thread offset serves every load of a tile.
  static_assert((D == 128 && RPL % 16 == 0) || (D == 64 && RPL % 4 == 0), "swizzle period");
};

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
// One 16-byte-per-lane buffer load into LDS at M0 (lane l writes M0 + 16 l),
// written as assembly: the compiler then does not treat every later LDS read
// as possibly aliasing it (it would wait for all such loads at the first LDS
// read, emptying a deep ring). The kernels that keep their tiles in one LDS
// array (deep rings, D = 64, e4m3 tiles) issue all their tile loads this way
// and order them and the reads of their tiles themselves (waits, then a
// barrier); M0 has no other user in those kernels.
__device__ __forceinline__ void dma16(v4u32 rsrc, int voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "m0");
}
// The same with a uniform byte offset added to the lane's (soffset).
__device__ __forceinline__ void dma16_so(v4u32 rsrc, int voff, uint32_t lds_addr, int soff) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %3 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr), "s"(soff)
      : "m0");
}

// s_waitcnt with only the vector-memory counter constrained (<= n, n < 64).
#define BSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

constexpr float kRescaleThreshold = 8.0f;  // log2 units: P values stay below 2^8

// max over lanes l and l ^ 32 (the two half-waves hold the two key halves).
__device__ __forceinline__ float halfwave_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)pr[0]), __builtin_bit_cast(float, (uint32_t)pr[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)pr[0]) + __builtin_bit_cast(float, (uint32_t)pr[1]);
}

// Plan arrays are read-only while a kernel runs; reading them through the
// constant address space makes uniform loads scalar.
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef __attribute__((address_space(4))) const uint32_t cuint32;
typedef __attribute__((address_space(4))) const float cfloat;

// Values that are the same on every lane (they derive from the work item and
// the entry index only), moved to scalar registers so buffer descriptors and
// LDS bases built from them stay scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename T>
__device__ __forceinline__ const T *uniform(const T *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T *)(((uint64_t)hi << 32) | lo);
}

// OCP FP8 E4M3 to bf16 for 8 bytes (every e4m3 value is exact in bf16).
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 w) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false), a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  const f2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false), b1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  return make_uint4(pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a1[0], a1[1]), pack_bf16x2(b0[0], b0[1]),
                    pack_bf16x2(b1[0], b1[1]));
}

// KV8: K and V are OCP FP8 E4M3 bytes with one fp32 scale per kv head. At
// D = 128 the e4m3 tiles stream into LDS like bf16 ones and are widened to
// bf16 as the MFMA operands are read (K rows by 8-byte reads, V^T by 8-bit
// transpose reads). At D = 64 they are loaded into registers where the bf16
// path issues its loads and written, widened, to the bf16 layout at the end of
// the tile (K tile j+2 and V tile j+1 go to buffers no wave reads during tile
// j). Either way the MFMAs are the bf16 path's on exact values; the K scale
// is folded into the softmax scale and the V scale into the final 1/l.
//
// NS = stages of the K and V rings. NS = 2: two K tiles and two V tiles; K
// runs one tile ahead of V: while the softmax of tile j runs, the S^T MFMAs
// of tile j+1 are already issued, and the loads of K tile j+2 and V tile j+1
// are in flight. NS = 4 (e4m3 tiles of a few live rows, such as decode
// steps, whose time goes to waiting on loads rather than to arithmetic): K
// tile j+4 and V tile j+3 are issued at tile j, so three tiles stream while
// one is used, with partial waits on the vector-memory counter.
template <int D, int TK, int TQ, bool PAGED, bool KV8 = false, int NS = 2, bool KIL = false>
__global__ __launch_bounds__(64 * (TQ / 32), (TK == 128 && TQ == 128) ? 1 : 2) void k_attn_bf16(AttnArgs a) {
  using C = CfgB<D, TK, TQ>;
  // e4m3 tiles at D = 128 stream into LDS as they are (KD)
  constexpr bool KD = KV8 && D == 128;
  static_assert(NS == 2 || (NS == 4 && KD), "stages");
  // one ring slot: a bf16 tile, or for deep e4m3 rings the e4m3 tile itself
  constexpr int SLOT = (NS > 2 && KD) ? TK * D : C::TILEB;
  // D = 128, two stages: one LDS variable per buffer, chosen by the tile
  // index's parity, which the tile loop (unrolled by two) knows at compile
  // time. Every access then names one variable, so the compiler can tell the
  // reads of a tile from the loads that are filling the other buffer and
  // does not wait for those loads before the reads. Otherwise one array,
  // indexed at run time (at D = 64, and for e4m3 tiles, the unrolled loop
  // needs more registers than the occupancy allows), whose loads are issued
  // from assembly for the same reason.
  constexpr bool RING = NS > 2 || D != 128 || KV8;
  // Waves skip the tiles in which none of their query sub-blocks is live.
  constexpr bool SKIP = !KV8 && !PAGED;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_ring[RING ? 2 * NS * SLOT : 64];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[RING ? 64 : SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[RING ? 64 : SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v0[RING ? 64 : SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v1[RING ? 64 : SLOT];
  // Buffer of K / V tile i; par is std::integral_constant<int, i & 1>.
  auto kbuf = [&](int i, auto par) -> uint8_t * {
    if constexpr (RING) return lds_ring + (i & (NS - 1)) * SLOT;
    else return decltype(par)::value ? lds_k1 : lds_k0;
  };
  auto vbuf = [&](int i, auto par) -> uint8_t * {
    if constexpr (RING) return lds_ring + (NS + (i & (NS - 1))) * SLOT;
    else return decltype(par)::value ? lds_v1 : lds_v0;
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // = this wave's 32-row slice
  const int n = lane & 31, hh = lane >> 5;
  const int nitems = a.counters[CNT_ITEMS];
  // Work distribution: workgroups are dispatched round-robin over the 8 XCDs,
  // so workgroup b runs on XCD b % 8 (when the grid is a multiple of 8). Each
  // XCD owns a queue of items:
  //   sched 0: a contiguous stretch of the work list in row order
  //            (neighbouring query tiles share K/V in that XCD's L2);
  //   sched 1: every 8th item in longest-first order (the XCDs get equal
  //            shares of long and short items);
  //   sched 2: row order dealt in blocks of kDeal items to the XCDs in turn
  //            (neighbouring tiles still share an XCD, and all XCDs work in
  //            one region of the list at a time, so the K/V they stream
  //            together fits the last-level cache; balanced when the rows'
  //            lengths change along the list).
  // Its workgroups take items from it with an atomic ticket, so an XCD's
  // workgroups finish together however the item lengths vary.
  const int nq = (gridDim.x & 7) == 0 ? kQueuesPerSet : 1;
  const int xq = blockIdx.x % nq;
  const bool strided = a.sched == 1, dealt = a.sched == 2;
  constexpr int kDeal = 64;
  const int nfull = nitems / kDeal, rem = nitems % kDeal;
  const int qbeg = strided ? xq : (dealt ? 0 : (int)((int64_t)xq * nitems / nq));
  const int qcnt = strided ? (nitems - xq + nq - 1) / nq
                   : dealt ? (nfull > xq ? (nfull - xq + nq - 1) / nq : 0) * kDeal +
                                 ((rem > 0 && nfull % nq == xq) ? rem : 0)
                           : (int)((int64_t)(xq + 1) * nitems / nq) - qbeg;
  int *const qctr = a.queue + xq;
  __shared__ int s_ticket;
  const uint16_t *__restrict__ Q = (const uint16_t *)a.q;

  // Per-lane LDS offsets that do not depend on the tile.
  const int krow0 = perm_bf16(n);  // K operand row within a 32-key block
  const int vj = lane & 15, vdsub = (lane >> 4) & 1;
  const int vrow0 = 8 * hh + (vj >> 2);  // V^T operand rows 16 c2 + vrow0 (+4)
  const int vbyte = 8 * (vj & 1);
  const int nqt = (int)a.nqt;
  // Per-thread byte offsets of its 16-byte slot in load 0 of a K / V tile.
  const int trow = tid / C::CPR, tpos = tid % C::CPR;
  const int koff0 = trow * (int)a.k_ss * 2 + ((tpos ^ C::swz_k(trow)) << 4);
  const int voff0 = trow * (int)a.v_ss * 2 + ((tpos ^ C::swz_v(trow)) << 4);
  const int kstep = C::RPL * (int)a.k_ss * 2, vstep = C::RPL * (int)a.v_ss * 2;
  const int skv32 = (int)a.Skv;  // sequence lengths are below 2^31
  const int ptiles = PAGED ? a.P / TK : 1;  // key tiles per page
  const bool ptiles_pow2 = (ptiles & (ptiles - 1)) == 0;

  if (tid == 0) s_ticket = atomicAdd(qctr, 1);
  __syncthreads();
  for (int tk = __builtin_amdgcn_readfirstlane(s_ticket); tk < qcnt;) {
    // The next ticket is taken now; its value is needed only after this item.
    int next_ticket = 0;
    if (tid == 0) next_ticket = atomicAdd(qctr, 1);
    const int it = strided ? qbeg + tk * nq : dealt ? ((tk / kDeal) * nq + xq) * kDeal + tk % kDeal : qbeg + tk;
    const int4 item = ((const int4 *)a.items)[it];
    const int r = item.x, e0 = item.y, nent = item.z - item.y, slot = item.w;

    // Entry metadata through the constant address space, so the loads are
    // scalar (SGPRs, no wait behind the tile loads). A rolling window holds
    // entries j, j+1, j+2; entry j+3 is loaded one iteration ahead.
    struct Meta {
      int kt, pg;
      uint32_t lv;
    };
    auto load_meta = [&](int j) {
      Meta m{0, 0, 0};
      if (nent <= 0) return m;  // an item without entries reads no metadata
      const int ee = e0 + min(j, nent - 1);
      if constexpr ((PAGED || D == 64) && !KV8) {
        // paged and D = 64 bf16 kernels: the entry arrays' addresses are read
        // from the kernel-argument segment per call (scalar loads one tile
        // ahead) rather than kept in scalar registers (whose spills were
        // restored in the tile loop: chunked prefill -3.7%, affine -1 to
        // -2%; e4m3 decode +1%, so it keeps the plain reads)
        const __attribute__((address_space(4))) AttnArgs *kp =
            (const __attribute__((address_space(4))) AttnArgs *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(kp));
        m.kt = ((const cint32 *)kp->ent_kt)[ee];
        m.pg = PAGED ? ((const cint32 *)kp->ent_page)[ee] : 0;
        m.lv = ((const cuint32 *)kp->ent_live)[ee];
      } else {
        m.kt = ((const cint32 *)a.ent_kt)[ee];
        m.pg = PAGED ? ((const cint32 *)a.ent_page)[ee] : 0;
        m.lv = ((const cuint32 *)a.ent_live)[ee];
      }
      return m;
    };
    Meta m0 = load_meta(0), m1 = load_meta(1), m2 = load_meta(2);
    Meta m3{0, 0, 0}, m4{0, 0, 0};  // deep rings: entries j+3, j+4
    if constexpr (NS == 4) m3 = load_meta(3), m4 = load_meta(4);

    // Row geometry (32-bit: rows, heads and tiles are all below 2^31).
    const int nh = a.pack ? a.Hkv : a.Hq;
    const int qt = r % nqt, hrow = (r / nqt) % nh, b = r / (nqt * nh);
    const int g = (a.pack ? hrow * a.G : hrow) / a.G;
    const bool ilv = a.pack == 2;  // heads interleaved row by row
    // wave-uniform head (an interleaved tile's heads are one union group and
    // share their key blocks, so the group's first head gives the live-bit
    // geometry) and the lane's own head
    const int head_w = a.pack ? hrow * a.G + (ilv ? 0 : (32 * wave) / a.tr) : hrow;
    const int head = ilv ? head_w + (32 * wave + n) % a.G : head_w;
    const int qbase = a.pack ? 0 : 32 * wave;
    const HeadMeta hm = a.hm[head_w];
    // First key of key tile kt, and the keys skipped between its two 32-key
    // blocks (key column c sits at x + c, plus y for c >= 32; contiguous
    // tiles: (kt * TK, 0)). KIL: the plan has key-interleaved heads (then
    // 128 x 64 tiles over contiguous K/V); other plans run without the
    // arithmetic.
    auto ktile = [&](int kt) -> int2 {
      if constexpr (KIL) return key_tile_span(hm, kt);
      return make_int2(kt * TK, 0);
    };
    // (a tile that merges query blocks may take them interleaved: its
    // 32-row slices then lie in different places of the sequence)
    const int64_t q0 = ilv ? (int64_t)qt * a.tr + (32 * wave) / a.G
                           : (a.pack ? (int64_t)qt * a.tr + (32 * wave) % a.tr
                                     : tile_query(hm, __builtin_ctz(a.tq), qt, 32 * wave));
    const int qd = ilv ? n / a.G : n;  // the lane's query is q0 + qd
    const int64_t qpos = q0 + qd;
    const bool qvalid = qpos < a.Sq;
    // A wave none of whose rows exist skips the arithmetic (it still loads
    // its share of every tile and meets every barrier).
    const bool wlive = __any(qvalid);
    // Largest key position the wave's first query may see under the causal
    // bound (query q0 + qd sees keys up to q0 + qd + off), clamped to
    // [-64, Skv]: beyond either end the tests below give the same answers.
    const int qlim0 = (int)max<int64_t>(-64, min<int64_t>(q0 + a.off, a.Skv));
    bf16x8 qb[D / 16];
    {
      const uint16_t *qp = Q + b * a.q_sb + head * a.q_sh + (qvalid ? qpos : 0) * a.q_ss;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        uint4 x = qvalid ? *(const uint4 *)(qp + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0);
        qb[c] = __builtin_bit_cast(bf16x8, x);
      }
    }
    // Deep rings: Q has landed before any tile load is issued, so the
    // compiler has no load of its own outstanding in the tile loop (it would
    // otherwise wait for every load, tile loads included, before using Q).
    if constexpr (NS == 4) BSA_WAIT_VM(0);
    const uint16_t *kbase_ptr = (const uint16_t *)a.k + (PAGED ? 0 : b * a.k_sb) + g * a.k_sh;
    const uint16_t *vbase_ptr = (const uint16_t *)a.v + (PAGED ? 0 : b * a.v_sb) + g * a.v_sh;
    // Softmax scale * log2(e) (times the K scale for e4m3 K); only the e4m3
    // path reads the scales (once per item, by a scalar load: a vector load
    // inside the tile loop would make the compiler wait for the tile loads),
    // the bf16 path reads the argument as it is.
    const int g_u = uniform(g);
    float sl2_kv8 = 0.f;
    if constexpr (KV8) sl2_kv8 = a.scale_log2 * ((const cfloat *)a.k_scale)[g_u];
#define BSA_SL2 (KV8 ? sl2_kv8 : a.scale_log2)

    // KV8 tile staging: 16 e4m3 bytes per load, row x / (D/16), columns
    // 16 * (x % (D/16)) .., written as two 16-byte bf16 chunks.
    // D = 128: e4m3 tiles stream straight into LDS like bf16 ones (KD) and are
    // widened when the MFMA operands are read; D = 64: register staging.
    constexpr int L8 = (KV8 && !KD) ? (TK * D / 16 + C::THREADS - 1) / C::THREADS : 0;
    uint4 k8r[L8 > 0 ? L8 : 1], v8r[L8 > 0 ? L8 : 1];
    // e4m3 tensors: one byte per element, so strides count bytes.
    const uint8_t *k8base = (const uint8_t *)a.k + (PAGED ? 0 : b * a.k_sb) + g * a.k_sh;
    const uint8_t *v8base = (const uint8_t *)a.v + (PAGED ? 0 : b * a.v_sb) + g * a.v_sh;
    auto load8 = [&](const void *base_, int64_t sb, int64_t ss, const Meta &m, uint4 (&r)[L8 > 0 ? L8 : 1]) {
      const uint8_t *base = (const uint8_t *)base_;
      const int2 kt2 = ktile(m.kt);
      const int k0 = kt2.x;
      const int left = skv32 - k0;  // the tile's rows at positions below this exist
      const int prow = ptiles_pow2 ? (m.kt & (ptiles - 1)) * TK : (m.kt % max(ptiles, 1)) * TK;
      const uint8_t *tb = PAGED ? base + (int64_t)m.pg * sb + (int64_t)prow * ss : base + (int64_t)k0 * ss;
#pragma unroll
      for (int u = 0; u < L8; ++u) {
        const int x = tid + C::THREADS * u;
        const int row = x / (D / 16), c8 = x % (D / 16);
        const int pos = row + (row >= 32 ? kt2.y : 0);
        r[u] = (x < TK * D / 16 && pos < left) ? *(const uint4 *)(tb + (int64_t)pos * ss + 16 * c8)
                                               : make_uint4(0, 0, 0, 0);
      }
    };
    auto store8 = [&](const uint4 (&r)[L8 > 0 ? L8 : 1], uint8_t *dst, bool is_v) {
#pragma unroll
      for (int u = 0; u < L8; ++u) {
        const int x = tid + C::THREADS * u;
        if (x < TK * D / 16) {
          const int row = x / (D / 16), c8 = x % (D / 16);
          const int sw = is_v ? C::swz_v(row) : C::swz_k(row);
          *(uint4 *)(dst + row * C::ROWB + (((2 * c8) ^ sw) << 4)) = e4m3x8_to_bf16(make_uint2(r[u].x, r[u].y));
          *(uint4 *)(dst + row * C::ROWB + (((2 * c8 + 1) ^ sw) << 4)) = e4m3x8_to_bf16(make_uint2(r[u].z, r[u].w));
        }
      }
    };
    (void)k8r, (void)v8r;

    // Buffer loads of one K or V tile of local entry j into dst (every thread).
    // Rows past the sequence end lie beyond the descriptor's range and read 0.
    auto issue = [&](const uint16_t *base, int64_t sb, int64_t ss, const Meta &m, uint8_t *dst_tile,
                     int off0, int step) {
      const int2 kt2 = ktile(m.kt);
      const int k0 = kt2.x;
      // rows of the tile's span that exist (its second block lies kt2.y rows
      // further on in a key-interleaved tile; the rows between are not read)
      const int left = min(skv32 - k0, TK + kt2.y);
      // Extra byte offset of the loads that fill the tile's second 32-key block.
      const int soff = kt2.y * (int)ss * 2;
      // Row of the tile within its page (pages hold whole key tiles).
      const int prow = ptiles_pow2 ? (m.kt & (ptiles - 1)) * TK : (m.kt % max(ptiles, 1)) * TK;
      const uint16_t *tb = PAGED ? base + (int64_t)m.pg * sb + (int64_t)prow * ss
                                 : base + (int64_t)k0 * ss;
      const int bytes = (left - 1) * (int)ss * 2 + D * 2;
      // One LDS array (deep rings, D = 64): the loads are issued from
      // assembly, so the reads of tile j do not wait for the loads filling
      // the other buffers; the tile loop waits for them itself.
      if constexpr (RING) {
        const uint64_t tbv = (uint64_t)tb;
        const v4u32 rs = {(uint32_t)tbv, (uint32_t)(tbv >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) {
          uint8_t *dst = dst_tile + (u * C::THREADS + wave * 64) * 16;
          if (KIL && u * C::RPL >= 32) dma16_so(rs, off0 + u * step, (uint32_t)(uintptr_t)(lds_void *)dst, soff);
          else dma16(rs, off0 + u * step, (uint32_t)(uintptr_t)(lds_void *)dst);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)tb, 0, bytes, 0x00020000);
        // The wave's byte offset, opaque to the compiler: the LDS addresses
        // of the loads are then formed per call from one scalar, instead of
        // one kept live per load and buffer (which spills scalar registers).
        int wofs = wave * 64 * 16;
        asm volatile("" : "+s"(wofs));
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) {
          uint8_t *dst = dst_tile + u * C::THREADS * 16 + wofs;  // lane-linear 1 KiB per wave
          const int vo = off0 + u * step + (u * C::RPL >= 32 ? soff : 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, vo, 0, 0, 0);
        }
      }
    };
    auto issue_k = [&](int j, auto par, const Meta &m) { issue(kbase_ptr, a.k_sb, a.k_ss, m, kbuf(j, par), koff0, kstep); };
    auto issue_v = [&](int j, auto par, const Meta &m) { issue(vbase_ptr, a.v_sb, a.v_ss, m, vbuf(j, par), voff0, vstep); };
    // e4m3 tiles (KD): rows of D bytes, 16-byte chunk c of row r at slot
    // c ^ swz8(r). K rows are read 8 bytes at a time by 32 lanes on 32 rows
    // (swz8_k spreads rows of one parity over the 8 slots); V is read by
    // 8-bit transpose reads, 8 rows x 2 chunks per 16-lane pair (swz8_v gives
    // rows r, r+2, r+4, r+6 disjoint chunk pairs).
    constexpr int CPR8 = D / 16, RPL8 = C::THREADS / CPR8;
    constexpr int LOADS8 = (TK * D) / (C::THREADS * 16);
    auto swz8_k = [](int r) { return (r >> 1) & 7; };
    auto swz8_v = [](int r) { return 2 * ((r >> 1) & 3); };
    const int trow8 = tid / CPR8, tpos8 = tid % CPR8;
    const int k8off0 = trow8 * (int)a.k_ss + ((tpos8 ^ swz8_k(trow8)) << 4);
    const int v8off0 = trow8 * (int)a.v_ss + ((tpos8 ^ swz8_v(trow8)) << 4);
    auto issue8 = [&](const uint8_t *base, int64_t sb, int64_t ss, const Meta &m, uint8_t *dst_tile, int off0) {
      const int2 kt2 = ktile(m.kt);
      const int k0 = kt2.x;
      const int left = min(skv32 - k0, TK + kt2.y);
      const int soff = kt2.y * (int)ss;  // loads of the second 32-key block
      const int prow = ptiles_pow2 ? (m.kt & (ptiles - 1)) * TK : (m.kt % max(ptiles, 1)) * TK;
      const uint8_t *tb = PAGED ? base + (int64_t)m.pg * sb + (int64_t)prow * ss : base + (int64_t)k0 * ss;
      const int bytes = (left - 1) * (int)ss + D;
      if constexpr (RING) {  // assembly-issued, as for bf16 tiles in one array
        const uint64_t tbv = (uint64_t)tb;
        const v4u32 rs = {(uint32_t)tbv, (uint32_t)(tbv >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
#pragma unroll
        for (int u = 0; u < LOADS8; ++u) {
          uint8_t *dst = dst_tile + (u * C::THREADS + wave * 64) * 16;
          if (KIL && u * RPL8 >= 32) dma16_so(rs, off0 + u * RPL8 * (int)ss, (uint32_t)(uintptr_t)(lds_void *)dst, soff);
          else dma16(rs, off0 + u * RPL8 * (int)ss, (uint32_t)(uintptr_t)(lds_void *)dst);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)tb, 0, bytes, 0x00020000);
#pragma unroll
        for (int u = 0; u < LOADS8; ++u) {
          uint8_t *dst = dst_tile + (u * C::THREADS + wave * 64) * 16;
          const int vo = off0 + u * RPL8 * (int)ss + (u * RPL8 >= 32 ? soff : 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, vo, 0, 0, 0);
        }
      }
    };
    auto issue_k8 = [&](int j, auto par, const Meta &m) { issue8(k8base, a.k_sb, a.k_ss, m, kbuf(j, par), k8off0); };
    auto issue_v8 = [&](int j, auto par, const Meta &m) { issue8(v8base, a.v_sb, a.v_ss, m, vbuf(j, par), v8off0); };
    (void)issue_k8, (void)issue_v8;
    // Lane offsets of the K fragments of the first 32-key block. The swizzle
    // (swz_k: row & 15 at D = 128) has a period of 16 rows, so the second block's fragments
    // lie 32 rows further on, and a fragment's address is a per-lane offset
    // plus a constant (buffer base, block) that the LDS read carries as its
    // immediate offset: no address arithmetic per tile.
    int kofs[D / 16];
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) kofs[cc] = krow0 * C::ROWB + (((2 * cc + hh) ^ C::swz_k(krow0)) << 4);
    (void)kofs;
    auto kfrag = [&](const uint8_t *ks, int i) {
      const int row = 32 * (i / (D / 16)) + krow0;
      if constexpr (KD) {
        const int c8 = i % (D / 16);  // 16 e4m3 bytes per k-step, 8 per half-wave
        const uint2 w = *(const uint2 *)(ks + row * D + ((c8 ^ swz8_k(row)) << 4) + 8 * hh);
        return __builtin_bit_cast(bf16x8, e4m3x8_to_bf16(w));
      } else if constexpr (D == 128) {
        return *(const bf16x8 *)(ks + (i / (D / 16)) * 32 * C::ROWB + kofs[i % (D / 16)]);
      } else {
        const int c = 2 * (i % (D / 16)) + hh;
        return *(const bf16x8 *)(ks + row * C::ROWB + ((c ^ C::swz_k(row)) << 4));
      }
    };

    f32x16 o[C::NDB];
#pragma unroll
    for (int u = 0; u < C::NDB; ++u) o[u] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.f;
    const int iq_lo = qbase >> hm.lq;
    const int niq = hm.lq >= 5 ? 1 : (32 >> hm.lq);
    const uint64_t wbits = ((1ull << (hm.mk * niq)) - 1ull) << (iq_lo * hm.mk);
    const uint32_t wbits32 = (uint32_t)wbits;  // the wave's live bits (at most 32 per tile)
    const int qsub = ((qbase + n) >> hm.lq) * hm.mk;

    constexpr int STEPS = C::NKB * D / 16;     // K fragments per tile
    constexpr int EPS = C::NKB * 16 / STEPS;   // scores exponentiated per step (2 or 4)
    // K fragment of S^T step i. The exponentials take tile j's 32-key score
    // blocks in order, block 0 first. In the kernels that keep their tiles in
    // one ring (not unrolled by two), the S^T MFMAs of tile j+1 beside them
    // build its last block first and then blocks 0, 1, ...: block t < NKB-1
    // is written in the steps right after the exponentials have taken block t,
    // into the same registers, and only the last block is copied per tile.
    // (Only the bf16 kernels over contiguous K/V: in the paged and e4m3 ring
    // kernels the compiler then kept more copies, not fewer.)
    constexpr bool ALIAS = RING && !PAGED && !KV8;
    constexpr auto next_frag = [](int i) {
      if constexpr (ALIAS) return ((i / (D / 16) + C::NKB - 1) % C::NKB) * (D / 16) + i % (D / 16);
      else return i;
    };

    // One tile iteration: softmax of tile j (scores in s_cur), S^T of tile
    // j+1 into s_next, O += V^T P^T of tile j.
    // par is the parity of j (std::integral_constant); flip that of j + 1.
    auto tile = [&](int j, auto par, auto &&s_cur, auto &&s_next) {
      const std::integral_constant<int, 1 - decltype(par)::value> flip;
      // K tile j+1 and V tile j have landed (this wave) ...
      if constexpr (NS == 2) {
        __builtin_amdgcn_s_waitcnt(0);
      } else {
        // ... while the loads issued after them (K tiles j+2 .. j+NS-1 and V
        // tiles j+1 .. j+NS-2 that exist) may still be in flight; loads
        // complete in issue order, so waiting until at most that many remain
        // is enough.
        constexpr int L = KD ? LOADS8 : C::LOADS;
        const int nk = max(0, min(j + NS - 1, nent - 1) - j - 1);
        const int nv = max(0, min(j + NS - 1, nent) - j - 1);
        switch (nk + nv) {
          case 4: BSA_WAIT_VM(4 * L); break;
          case 3: BSA_WAIT_VM(3 * L); break;
          case 2: BSA_WAIT_VM(2 * L); break;
          case 1: BSA_WAIT_VM(L); break;
          default: BSA_WAIT_VM(0); break;
        }
      }
      __syncthreads();  // ... for every wave; K tile j and V tile j-1 are free
      const Meta mn = load_meta(j + NS + 1);
      if constexpr (NS == 4) {
        if constexpr (KD) {
          if (j + 4 < nent) issue_k8(j + 4, par, m4);
          if (j + 3 < nent) issue_v8(j + 3, flip, m3);
        } else {
          if (j + 4 < nent) issue_k(j + 4, par, m4);
          if (j + 3 < nent) issue_v(j + 3, flip, m3);
        }
      } else if constexpr (KD) {
        if (j + 2 < nent) issue_k8(j + 2, par, m2);
        if (j + 1 < nent) issue_v8(j + 1, flip, m1);
      } else if constexpr (KV8) {
        if (j + 2 < nent) load8(k8base, a.k_sb, a.k_ss, m2, k8r);
        if (j + 1 < nent) load8(v8base, a.v_sb, a.v_ss, m1, v8r);
      } else {
        if (j + 2 < nent) issue_k(j + 2, par, m2);
        if (j + 1 < nent) issue_v(j + 1, flip, m1);
      }

      // A wave computes a tile only where one of its query sub-blocks is live
      // in it (a merged tile often selects a key tile for some of its query
      // blocks only); the S^T of tile j+1 is computed only if that tile is
      // live for the wave, and its scores are used only then.
      // (Only kernels whose tiles can merge query blocks: union and paged
      // plans give every wave every entry, and e4m3 tiles would spill
      // registers for the second path.)
      if constexpr (SKIP) {
        if (wlive && (m0.lv & wbits32) == 0u && j + 1 < nent && (m1.lv & wbits32) != 0u) {
          const uint8_t *ks = kbuf(j + 1, flip);
          bf16x8 kf[STEPS];
#pragma unroll
          for (int i = 0; i < 3 && i < STEPS; ++i) kf[i] = kfrag(ks, next_frag(i));
#pragma unroll
          for (int i = 0; i < STEPS; ++i) {
            if (i + 3 < STEPS) kf[i + 3] = kfrag(ks, next_frag(i + 3));
            const int t = next_frag(i) / (D / 16), cc = i % (D / 16);
            s_next[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qb[cc], cc == 0 ? f32x16{} : s_next[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      const bool lj = [&] {
        if constexpr (SKIP) return wlive && (m0.lv & wbits32) != 0u;
        else return wlive;
      }();
      if (lj) {
      // ---- mask tile j (sequence end, causal diagonal, dead sub-blocks) ----
      // 32-bit scalar tests: positions and the causal offset are below 2^31.
      const int2 kt2 = ktile(m0.kt);
      const int kb0 = kt2.x;
      const uint32_t live = m0.lv;
      const bool need = (kb0 + kt2.y + TK > skv32) || (a.causal && kb0 + TK - 1 > qlim0) ||
                        ((uint64_t)live & wbits) != wbits;
      if (need) {
        // Allowed keys of this lane's query as bit masks over the tile (64
        // keys per mask): live key sub-blocks, then the prefix of keys that
        // exist and satisfy the causal bound. (In a key-interleaved tile, never
        // causal, the first block is whole whenever the second lies kt2.y
        // further on, so the prefix counts from the second block's shift.)
        const uint32_t lbits = live >> qsub;
        int lim = skv32 - kb0 - kt2.y;
        if (a.causal) lim = min(lim, qlim0 + qd + 1 - kb0);
        const int klim = max(0, min(lim, TK));
        const int ak = 1 << hm.lk;  // keys per live bit
        const uint64_t sub = ak >= 64 ? ~0ull : ((1ull << ak) - 1ull);
        uint64_t km[(TK + 63) / 64];
#pragma unroll
        for (int w64 = 0; w64 < (TK + 63) / 64; ++w64) {
          uint64_t m = 0;
          for (int ik = 0; ik < hm.mk; ++ik)
            if ((lbits >> ik) & 1u) {
              const int k0b = ik * ak - 64 * w64;  // first key of the sub-block in this mask
              if (k0b >= 64 || k0b + ak <= 0) continue;
              m |= k0b >= 0 ? sub << k0b : sub >> -k0b;
            }
          const int lo = klim - 64 * w64;
          m &= lo >= 64 ? ~0ull : (lo <= 0 ? 0ull : ((1ull << lo) - 1ull));
          km[w64] = m >> (8 * hh);  // accumulator keys are offset by 8 on the upper half-wave
        }
#pragma unroll
        for (int t = 0; t < C::NKB; ++t)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int kl = 32 * t + 16 * (jj >> 3) + (jj & 7);  // key offset without the 8*hh term
            if (!((km[kl / 64] >> (kl % 64)) & 1ull)) s_cur[t][jj] = -INFINITY;
          }
      }

      // ---- online softmax of tile j, log2 domain, lazy rescale ----
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < C::NKB; ++t)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s_cur[t][jj]);
      mx = halfwave_max(mx);
      const float cand = mx * BSA_SL2;
      if (__any(cand > m_ref + kRescaleThreshold)) {
        const float m_new = fmaxf(m_ref, cand);
        const float alpha = m_new == -INFINITY ? 1.f : fexp2(m_ref - m_new);
        l_run *= alpha;
#pragma unroll
        for (int u = 0; u < C::NDB; ++u) o[u] *= alpha;
        m_ref = m_new;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;

      // One straight-line block, in a fixed order: each S^T MFMA of tile j+1
      // (independent work) is followed by the exponentials of a slice of tile
      // j, with its K-operand read issued three steps ahead; then the P V^T
      // MFMAs follow their transpose reads. sched_barrier(0) keeps the
      // compiler from regrouping the steps. On the last tile the S^T of a
      // stale buffer is computed and dropped.
      // The wave takes issue priority over the other waves of its SIMD while
      // it interleaves the S^T MFMAs with the exponentials (measured: 2-4%
      // faster than equal priorities, or than raising it for P·V as well).
      __builtin_amdgcn_s_setprio(1);
      uint32_t pw[C::NKB * 8];  // P as packed bf16 pairs
      float psum = 0.f;
      auto exps = [&](int i) {
#pragma unroll
        for (int k2 = 0; k2 < EPS; k2 += 2) {
          const int x = i * EPS + k2;
          const float p0 = fexp2(__builtin_fmaf(s_cur[x / 16][x % 16], BSA_SL2, -m_use));
          const float p1 = fexp2(__builtin_fmaf(s_cur[x / 16][x % 16 + 1], BSA_SL2, -m_use));
          psum = x == 0 ? p0 : psum + p0;  // (no add of the initial zero)
          psum += p1;
          pw[x / 2] = pack_bf16x2(p0, p1);
        }
      };
      {
        const uint8_t *ks = kbuf(j + 1, flip);
        bf16x8 kf[STEPS];
#pragma unroll
        for (int i = 0; i < 3 && i < STEPS; ++i) kf[i] = kfrag(ks, next_frag(i));
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          if (i + 3 < STEPS) kf[i + 3] = kfrag(ks, next_frag(i + 3));
          const int t = next_frag(i) / (D / 16), cc = i % (D / 16);
          s_next[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qb[cc], cc == 0 ? f32x16{} : s_next[t], 0, 0, 0);
          exps(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      l_run += psum;

      // ---- O^T += V^T P^T, V^T fragments by transpose reads of V tile j ----
      {
        const uint8_t *vs = vbuf(j, par);
        constexpr int PV = (TK / 16) * C::NDB;
        auto vfrag = [&](int i) {
          const int c2 = i / C::NDB, u = i % C::NDB;
          if constexpr (KD) {
            // one 8-bit transpose read: each 16-lane group reads 8 key rows x
            // 16 columns and lane j receives column j of them, i.e. 8
            // consecutive keys of head-dim column 32u + n
            const int i16 = lane & 15, grp = (lane >> 4) & 1;
            const int row = 16 * c2 + 8 * hh + (i16 >> 1);
            const int col = 32 * u + 16 * grp + 8 * (i16 & 1);
            typedef int v2i __attribute__((ext_vector_type(2)));
            const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i *)(vs + row * D + (((col >> 4) ^ swz8_v(row)) << 4) + (col & 15)));
            return __builtin_bit_cast(bf16x8, e4m3x8_to_bf16(make_uint2((uint32_t)r[0], (uint32_t)r[1])));
          }
          const int ra = 16 * c2 + vrow0, rb = ra + 4;
          const int chunk = (32 * u + 16 * vdsub + 4 * (vj & 3)) >> 3;
          const uint8_t *pa = vs + ra * C::ROWB + ((chunk ^ C::swz_v(ra)) << 4) + vbyte;
          const uint8_t *pbp = vs + rb * C::ROWB + ((chunk ^ C::swz_v(rb)) << 4) + vbyte;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pa);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pbp);
          const s16x4 both[2] = {lo, hi};
          return __builtin_bit_cast(bf16x8, both);
        };
        bf16x8 vf[PV];
        vf[0] = vfrag(0);
        vf[1] = vfrag(1);
#pragma unroll
        for (int i = 0; i < PV; ++i) {
          if (i + 2 < PV) vf[i + 2] = vfrag(i + 2);
          const int c2 = i / C::NDB, u = i % C::NDB;
          const uint4 w = make_uint4(pw[4 * c2], pw[4 * c2 + 1], pw[4 * c2 + 2], pw[4 * c2 + 3]);
          o[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], __builtin_bit_cast(bf16x8, w), o[u], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      }  // lj
      if constexpr (KV8 && !KD) {
        if (j + 2 < nent) store8(k8r, kbuf(j + 2, par), false);
        if (j + 1 < nent) store8(v8r, vbuf(j + 1, flip), true);
      }
      if constexpr (NS == 4) m0 = m1, m1 = m2, m2 = m3, m3 = m4, m4 = mn;
      else m0 = m1, m1 = m2, m2 = mn;
    };

    // Prologue: K tiles 0 and 1, V tile 0; S^T of tile 0. Then tiles two at a
    // time, the two score buffers swapping roles (no register copies).
    f32x16 sa[C::NKB], sb[C::NKB];
    if (nent > 0) {
      if constexpr (NS == 4) {
        // K tile 0, then (K tile i, V tile i-1) for i = 1, 2, 3: the order in
        // which the tile loop counts them; S^T of tile 0 waits for K tile 0
        // alone.
        auto ik = [&](int i, const Meta &m) {
          if (i < nent) {
            if constexpr (KD) issue_k8(i, Even{}, m);
            else issue_k(i, Even{}, m);
          }
        };
        auto iv = [&](int i, const Meta &m) {
          if (i < nent) {
            if constexpr (KD) issue_v8(i, Even{}, m);
            else issue_v(i, Even{}, m);
          }
        };
        ik(0, m0);
        ik(1, m1), iv(0, m0);
        ik(2, m2), iv(1, m1);
        ik(3, m3), iv(2, m2);
        constexpr int L = KD ? LOADS8 : C::LOADS;
        switch (min(3, nent - 1) + min(3, nent)) {
          case 6: BSA_WAIT_VM(6 * L); break;
          case 5: BSA_WAIT_VM(5 * L); break;
          case 4: BSA_WAIT_VM(4 * L); break;
          case 3: BSA_WAIT_VM(3 * L); break;
          case 2: BSA_WAIT_VM(2 * L); break;
          case 1: BSA_WAIT_VM(L); break;
          default: BSA_WAIT_VM(0); break;
        }
      } else if constexpr (KD) {
        issue_k8(0, Even{}, m0);
        issue_v8(0, Even{}, m0);
        if (nent > 1) issue_k8(1, Odd{}, m1);
      } else if constexpr (KV8) {
        load8(k8base, a.k_sb, a.k_ss, m0, k8r);
        load8(v8base, a.v_sb, a.v_ss, m0, v8r);
        store8(k8r, kbuf(0, Even{}), false);
        store8(v8r, vbuf(0, Even{}), true);
        if (nent > 1) {
          load8(k8base, a.k_sb, a.k_ss, m1, k8r);
          store8(k8r, kbuf(1, Odd{}), false);
        }
      } else {
        issue_k(0, Even{}, m0);
        issue_v(0, Even{}, m0);
        if (nent > 1) issue_k(1, Odd{}, m1);
      }
      if constexpr (NS == 2) __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const uint8_t *ks = kbuf(0, Even{});
      const bool l0 = [&] {
        if constexpr (SKIP) return wlive && (m0.lv & wbits32) != 0u;
        else return wlive;
      }();
      if (l0) {
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          const int t = i / (D / 16), cc = i % (D / 16);
          sa[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(ks, i), qb[cc], cc == 0 ? f32x16{} : sa[t], 0, 0, 0);
        }
      }
    }
    if constexpr (!RING) {
      for (int j = 0; j < nent; j += 2) {
        tile(j, Even{}, sa, sb);
        if (j + 1 < nent) tile(j + 1, Odd{}, sb, sa);
      }
    } else {
      if constexpr (ALIAS) {
        // Tile j+1's blocks 0 .. NKB-2 go straight into sa (see next_frag);
        // its last block goes to sb and is copied.
        struct SView {
          f32x16 *p[C::NKB];
          __device__ f32x16 &operator[](int t) const { return *p[t]; }
        };
        SView cur{}, nxt{};
#pragma unroll
        for (int t = 0; t < C::NKB; ++t) cur.p[t] = &sa[t], nxt.p[t] = t + 1 < C::NKB ? &sa[t] : &sb[t];
        for (int j = 0; j < nent; ++j) {
          tile(j, Even{}, cur, nxt);  // the buffers follow j itself
          sa[C::NKB - 1] = sb[C::NKB - 1];
        }
      } else {
        for (int j = 0; j < nent; ++j) {
          tile(j, Even{}, sa, sb);  // the buffers follow j itself
#pragma unroll
          for (int t = 0; t < C::NKB; ++t) sa[t] = sb[t];
        }
      }
    }
    __syncthreads();  // the next item's first loads reuse the buffers

    // ---- finalize ----
    // bf16 tiles at D = 128, contiguous K/V: the output arguments are read
    // again here, from the kernel-argument segment (which holds `a` at
    // offset 0) through a pointer the compiler cannot see through, instead
    // of being kept in scalar registers through the tile loop (whose scalar
    // spills then vanish; video-DiT -1.8%). Elsewhere it measured slower
    // (paged K/V: +0.7%) or costs vector registers (D = 64 no longer fits
    // three waves per SIMD), so `a` is read as before.
    constexpr bool RELOAD = D == 128 && !KV8 && !PAGED;
    // The scratch's slot count, read here from the kernel-argument segment
    // (not kept in a scalar register through the tile loop).
    auto slot_limit = [&]() -> int {
      const __attribute__((address_space(4))) AttnArgs *kp =
          (const __attribute__((address_space(4))) AttnArgs *)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(kp));
      return kp->part_slots;
    };
    auto store_out = [&](const AttnArgs &oa) {
      const float l_tot = halfwave_sum(l_run);
      const float inv = l_tot > 0.f ? (KV8 ? ((const cfloat *)a.v_scale)[g_u] : 1.f) / l_tot : 0.f;
      const float lse = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
      if (slot < 0) {
        if (qvalid) {
          uint16_t *op = (uint16_t *)oa.o + b * oa.o_sb + head * oa.o_sh + qpos * oa.o_ss;
#pragma unroll
          for (int u = 0; u < C::NDB; ++u)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int d0 = 32 * u + 8 * q4 + 4 * hh;
              *(uint2 *)(op + d0) = make_uint2(pack_bf16x2(o[u][4 * q4] * inv, o[u][4 * q4 + 1] * inv),
                                               pack_bf16x2(o[u][4 * q4 + 2] * inv, o[u][4 * q4 + 3] * inv));
            }
          if (hh == 0) oa.lse[((int64_t)b * oa.Hq + head) * oa.Sq + qpos] = lse;
        }
      } else if (qvalid && slot < slot_limit()) {  // the combine reads partials of existing rows only
        const int64_t prow = (int64_t)slot * TQ + 32 * wave + n;
        float *pp = oa.part_o + prow * D;
#pragma unroll
        for (int u = 0; u < C::NDB; ++u)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * u + 8 * q4 + 4 * hh;
            *(float4 *)(pp + d0) = make_float4(o[u][4 * q4] * inv, o[u][4 * q4 + 1] * inv,
                                               o[u][4 * q4 + 2] * inv, o[u][4 * q4 + 3] * inv);
          }
        if (hh == 0) oa.part_lse[prow] = lse;
      }
    };
    if constexpr (RELOAD) {
      const __attribute__((address_space(4))) AttnArgs *kp =
          (const __attribute__((address_space(4))) AttnArgs *)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(kp));
      store_out(*(const AttnArgs *)kp);
    } else {
      store_out(a);
    }
    // Every thread read the current ticket before the barriers of this item.
    if (tid == 0) s_ticket = next_ticket;
    __syncthreads();
    tk = __builtin_amdgcn_readfirstlane(s_ticket);
  }
}

// Split-KV combine: O = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - M),
// LSE = M + ln sum_s w_s, M = max_s lse_s. A record covers one TQ-row tile.
#undef BSA_SL2

template <int D, bool BF, int TQ>
__global__ __launch_bounds__(kThreads) void k_combine(AttnArgs a, const int32_t *__restrict__ comb) {
  using E = typename std::conditional<BF, uint16_t, float>::type;
  // One wave per query row: a workgroup takes four rows of one record per
  // step (so short and long records alike spread over the whole grid). The
  // lanes hold D / 64 adjacent columns, so each slot's partial row is one
  // contiguous read of the wave; the slot weights exp(lse_s - M) are the
  // same on every lane.
  constexpr int CPL = D / 64, RPW = kThreads / 64, QUADS = TQ / RPW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ncomb = a.counters[CNT_COMB];
  for (int64_t unit = blockIdx.x; unit < (int64_t)ncomb * QUADS; unit += gridDim.x) {
    const int c = (int)(unit / QUADS);
    const int r = comb[3 * c], s0 = comb[3 * c + 1], k = comb[3 * c + 2];
    if (s0 + k > a.part_slots) continue;  // (never: the scratch holds every slot of the plan)
    {
      const int row = (int)(unit % QUADS) * RPW + wave;
      const RowPos geo = tile_row(a, r, row);
      const int64_t qpos = geo.q;
      if (qpos >= a.Sq) continue;
      E *op = (E *)a.o + geo.b * a.o_sb + geo.head * a.o_sh + qpos * a.o_ss;
      float *lp = a.lse + ((int64_t)geo.b * a.Hq + geo.head) * a.Sq + qpos;
      float M = -INFINITY, ws = 0.f;
      float acc[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) acc[j] = 0.f;
      // The partial row of slot s at this lane's columns.
      auto part = [&](int s, float *x) {
        const float *src = a.part_o + ((int64_t)(s0 + s) * TQ + row) * D + CPL * lane;
        if constexpr (CPL == 2) {
          const float2 v = *(const float2 *)src;
          x[0] = v.x, x[1] = v.y;
        } else {
          x[0] = src[0];
        }
      };
      if (k <= 64) {
        // One round of loads: lane s holds slot s's LSE, and the partial
        // rows of the first kAhead slots are read beside it (they do not
        // depend on the maximum); each slot's weight exp(lse_s - M) is then
        // taken from the lane that holds it.
        constexpr int kAhead = 8;
        const float l = lane < k ? a.part_lse[(int64_t)(s0 + lane) * TQ + row] : -INFINITY;
        float x[kAhead][CPL];
#pragma unroll
        for (int s = 0; s < kAhead; ++s)
          if (s < k) part(s, x[s]);
        M = l;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        if (M != -INFINITY) {
          const float wl = lane < k ? expf(l - M) : 0.f;
          ws = wl;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) ws += __shfl_xor(ws, o);
#pragma unroll
          for (int s = 0; s < kAhead; ++s)
            if (s < k) {
              const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
#pragma unroll
              for (int j = 0; j < CPL; ++j) acc[j] += w * x[s][j];
            }
          for (int s = kAhead; s < k; ++s) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
            float y[CPL];
            part(s, y);
#pragma unroll
            for (int j = 0; j < CPL; ++j) acc[j] += w * y[j];
          }
        }
      } else {
        for (int s = lane; s < k; s += 64) M = fmaxf(M, a.part_lse[(int64_t)(s0 + s) * TQ + row]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        if (M != -INFINITY) {
          for (int s = lane; s < k; s += 64) ws += expf(a.part_lse[(int64_t)(s0 + s) * TQ + row] - M);
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) ws += __shfl_xor(ws, o);
#pragma unroll 4
          for (int s = 0; s < k; ++s) {
            const float w = expf(a.part_lse[(int64_t)(s0 + s) * TQ + row] - M);
            float y[CPL];
            part(s, y);
#pragma unroll
            for (int j = 0; j < CPL; ++j) acc[j] += w * y[j];
          }
        }
      }
      if (M == -INFINITY) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) op[CPL * lane + j] = (E)0;
        if (lane == 0) *lp = -INFINITY;
        continue;
      }
      const float inv = 1.f / ws;
      if constexpr (BF && CPL == 2) {
        *(uint32_t *)(op + 2 * lane) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          if constexpr (BF) {
            const uint32_t pk = pack_bf16x2(acc[j] * inv, 0.f);
            op[CPL * lane + j] = (E)(pk & 0xffffu);
          } else {
            op[CPL * lane + j] = acc[j] * inv;
          }
        }
      }
      if (lane == 0) *lp = M + logf(ws);
    }
  }
}

// Zeroes one call's work-queue counters (a kernel, not a memset, so the
// forward stays capturable in a graph).
__global__ void k_zero_queues(int *q) {
  if (threadIdx.x < kQueuesPerSet) q[threadIdx.x] = 0;
}

template <int D, int TK, bool BF, int TQ, bool PAGED = false, bool KV8 = false, int NS = 2, bool KIL = false>
bsa_status launch_one(const Plan &p, const AttnArgs &a, hipStream_t s) {
  if constexpr (BF && !KV8 && NS == 2 && !KIL)
    if (a.kv8) return launch_one<D, TK, BF, TQ, PAGED, true>(p, a, s);
  if constexpr (BF && !PAGED && NS == 2 && !KIL)
    if (a.paged) return launch_one<D, TK, BF, TQ, true, KV8>(p, a, s);
  // Plans with key-interleaved heads (128 x 64 tiles, contiguous K/V).
  if constexpr (BF && !PAGED && NS == 2 && !KIL && TK == 64 && TQ == 128)
    if (p.key_interleaved) return launch_one<D, TK, BF, TQ, PAGED, KV8, NS, true>(p, a, s);
  // Interleaved tiles (a few live rows each: decode steps) of e4m3 K/V stream
  // four deep (eight 8 KiB slots, two workgroups per CU). A bf16 ring that
  // deep needs 128 KiB of LDS, one workgroup per CU, and measured slower.
  if constexpr (BF && NS == 2 && D == 128 && TK == 64 && TQ == 128 && KV8 && !KIL)
    if (a.pack == 2) return launch_one<D, TK, BF, TQ, PAGED, KV8, 4>(p, a, s);
  // Persistent grid: CUs x resident workgroups, per device (devices may
  // differ in CU count).
  constexpr int kMaxDev = 64;
  static std::atomic<int> grids[kMaxDev];
  const int threads = BF ? 64 * (TQ / 32) : kThreads;
  auto kern = BF ? (void (*)(AttnArgs))k_attn_bf16<D, TK, TQ, PAGED, KV8, NS, KIL> : (void (*)(AttnArgs))k_attn<D, 64, false>;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  int g = (dev >= 0 && dev < kMaxDev) ? grids[dev].load(std::memory_order_relaxed) : 0;
  if (g == 0) {
    int cus = 0, occ = 0;
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0));
    g = cus * (occ > 0 ? occ : 1);
    if (dev >= 0 && dev < kMaxDev) grids[dev].store(g, std::memory_order_relaxed);
  }
  if (p.item_cap < g) g = (int)std::max<int64_t>(p.item_cap, 1);
  if constexpr (BF) hipLaunchKernelGGL(k_zero_queues, dim3(1), dim3(64), 0, s, a.queue);
  hipLaunchKernelGGL(kern, dim3(g), dim3(threads), 0, s, a);
  if (p.rg.split > 0 && p.comb_cap > 0) {
    const int cg = (int)std::min<int64_t>(p.comb_cap * (TQ / (kThreads / 64)), 8192);
    hipLaunchKernelGGL((k_combine<D, BF, TQ>), dim3(cg), dim3(kThreads), 0, s, a, p.comb);
  }
  HIP_TRY(hipGetLastError());
  return BSA_OK;
}

}  // namespace

bsa_status attention_launch(const Plan &p, const AttnArgs &a, hipStream_t s) {
  const bool bf = p.dtype == BSA_BF16;
  // fp32 tiles use 64 keys (the planner guarantees it): 128 would not fit LDS twice.
  const int tq = p.rg.tq, tk = p.rg.tk;
  if (bf && tq == 128) {
    if (p.D == 128 && tk == 64) return launch_one<128, 64, true, 128>(p, a, s);
    if (p.D == 64 && tk == 64) return launch_one<64, 64, true, 128>(p, a, s);
    if (p.D == 128 && tk == 128) return launch_one<128, 128, true, 128>(p, a, s);
    if (p.D == 64 && tk == 128) return launch_one<64, 128, true, 128>(p, a, s);
  }
  if (bf && tq == 256) {
    if (p.D == 128 && tk == 64) return launch_one<128, 64, true, 256>(p, a, s);
    if (p.D == 64 && tk == 64) return launch_one<64, 64, true, 256>(p, a, s);
  }
  if (!bf && tq == 128 && p.D == 128 && tk == 64) return launch_one<128, 64, false, 128>(p, a, s);
  if (!bf && tq == 128 && p.D == 64 && tk == 64) return launch_one<64, 64, false, 128>(p, a, s);
  return fail(BSA_ERR_UNSUPPORTED, "no kernel for this head_dim / tile_k");
}

}  // namespace bsa
