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
//   k_bwd_dkdv  one workgroup per (batch, kv head, 128 keys), one wave per 32
//               keys, K and V rows held in registers. The query chunks that
//               visit its keys come from a key-major index built per call
//               from the plan's sorted lists (planner: k_kv_chunks); they
//               stream through LDS three chunks ahead of the arithmetic.
//               S = Q K^T and dP = dO V^T put one key in each lane;
//               dV^T += dO^T P and dK^T += Q^T dS take P and dS straight from
//               the accumulators as MFMA operands.
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

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef __attribute__((address_space(4))) const uint32_t cuint32;

// XOR swizzle of the 16-byte chunks of an LDS row of D bf16: chunk c of row r
// sits at slot c ^ swz(r). Two read patterns must both spread over the 64
// banks: a 16-byte row read has 16 lanes on 16 rows of one aligned group of
// 16 (so swz must differ across those rows), and a transpose read has 32
// lanes on 4 consecutive rows by 4 consecutive chunks of an aligned group of
// 4 (so bits 2-3 of swz must differ across those rows). D = 128 (16 chunks,
// 256-byte rows): swz = (r & 3) << 2 | (r >> 2) & 3. D = 64 (8 chunks,
// two rows per 256 bytes): the same on the row pair index s = r >> 1,
// swz = (s & 1) << 2 | (s >> 1) & 3.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// 16-byte row read: dims 8*c .. 8*c + 7 of row r.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const uint8_t *t, int r, int c) {
  return *(const bf16x8 *)(t + r * (2 * D) + ((c ^ swz<D>(r)) << 4));
}

// Transpose read of a swizzled tile: lane (n, hh) gets X[r0 + 8hh + i][c0 + n], i = 0..7.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag_s(const uint8_t *t, int r0, int c0, int lane) {
  const int vj = lane & 15, vsub = (lane >> 4) & 1, hh = lane >> 5;
  const int ra = r0 + 8 * hh + (vj >> 2), rb = ra + 4;
  const int col = c0 + 16 * vsub + 4 * (vj & 3);
  const int ch = col >> 3, byte = (col & 7) * 2;
  const uint8_t *pa = t + ra * (2 * D) + ((ch ^ swz<D>(ra)) << 4) + byte;
  const uint8_t *pb = t + rb * (2 * D) + ((ch ^ swz<D>(rb)) << 4) + byte;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pa);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pb);
  const s16x4 both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

// s_waitcnt with only the vector-memory counter constrained (<= n).
#define BSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
// Buffer resource of `bytes` bytes at base (raw buffer, no swizzle).
__device__ __forceinline__ v4u32 raw_rsrc(const void *base, int bytes) {
  const uint64_t v = (uint64_t)base;
  return v4u32{(uint32_t)v, (uint32_t)(v >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
}
// Buffer loads straight into LDS at M0 (lane l writes M0 + 16 l, or M0 + 4 l
// for the dword form), written as assembly: the compiler then does not treat
// the later LDS reads of the other ring buffers as possibly aliasing them
// (it would wait for every load in flight, three chunks ahead included,
// before the first such read). The chunk pipeline orders the loads and the
// reads of their buffers itself (partial vmcnt waits, then a barrier). The
// address operand is read at issue; no register receives data. M0 has no
// other user in this kernel.
__device__ __forceinline__ void dma_b128(v4u32 rsrc, int voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "m0");
}
// The same with a uniform byte offset added to the lane's (soffset).
__device__ __forceinline__ void dma_b128_so(v4u32 rsrc, int voff, uint32_t lds_addr, int soff) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %3 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr), "s"(soff)
      : "m0");
}
__device__ __forceinline__ void dma_b32(v4u32 rsrc, int voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "m0");
}
__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)p);
}

// ---------------------------------------------------------------------------
// dQ (and Delta) per plan row
// ---------------------------------------------------------------------------
// K and V tiles stream from HBM straight into LDS (buffer loads to LDS, rows
// past the sequence end read as zero), two buffers, the next tile's loads in
// flight while the current one is computed. K is read as rows (the S^T
// operand) and transposed (the K^T operand of dQ^T); V as rows.
// Work item of workgroup b in a grid of n: workgroups are dispatched
// round-robin over the 8 XCDs (workgroup b on XCD b % 8), so blocks of
// kXcdRun consecutive items go to one XCD, the 8 XCDs taking 8 neighbouring
// blocks at a time: the tiles that neighbouring items share (the query
// tiles of a window, the key groups they see) stay in one XCD's L2. The
// items past the last whole group of 8 * kXcdRun keep their own order.
constexpr int kXcdRun = 64;
__device__ __forceinline__ int xcd_item(int b, int n) {
  const int full = n / (8 * kXcdRun) * (8 * kXcdRun);
  if (b >= full) return b;
  const int x = b & 7, i = b >> 3;
  return ((i / kXcdRun) * 8 + x) * kXcdRun + i % kXcdRun;
}

template <int D, int TK, int TQ, bool KIL = false>
__global__ __launch_bounds__(2 * TQ, TQ == 128 ? 2 : 1) void k_bwd_dq(BwdArgs a) {
  constexpr int T = 2 * TQ;                     // 64 lanes per 32 query rows
  constexpr int WAVES = TQ / 32;
  constexpr int ROWB = 2 * D;
  constexpr int TILEB = TK * ROWB;              // one K (or V) tile
  constexpr int CPR = D / 8;
  constexpr int RPL = T / CPR;                  // tile rows covered by one load
  constexpr int LOADS = TILEB / (T * 16);       // loads per thread per tile
  constexpr int NKB = TK / 32, NDB = D / 32;
  static_assert(RPL % 16 == 0 && LOADS >= 1, "load geometry");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * TILEB];  // K, V; two buffers

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int r = xcd_item(blockIdx.x, gridDim.x);
  const int nqt = (int)a.nqt;
  const int nh = a.pack ? a.Hkv : a.Hq;
  const int qt = r % nqt, hrow = (r / nqt) % nh, b = r / (nqt * nh);
  const int head = a.pack ? hrow * a.G + (32 * wave) / a.tr : hrow;
  const int g = (a.pack ? hrow * a.G : hrow) / a.G;
  const int qbase = a.pack ? 0 : 32 * wave;
  const HeadMeta hm = a.hm[head];
  // (through the query-block interleave of a merged tile)
  const int64_t q0 = a.pack ? (int64_t)qt * a.tr + (32 * wave) % a.tr : tile_query(hm, __builtin_ctz(a.tq), qt, 32 * wave);
  const int64_t qpos = q0 + n;
  const bool qvalid = qpos < a.Sq;
  (void)WAVES;

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
  // and for padding rows past the sequence end. Kept for the dK/dV kernel,
  // which then spends no multiply per score on it.
  const float lse2 = L == -INFINITY ? INFINITY : L * kLog2e;
  if (qvalid && hh == 0) a.lse2[rowix] = lse2;

  const int e0 = a.row_ent[2 * r], nent = a.row_ent[2 * r + 1] - e0;
  const uint16_t *Kb = (const uint16_t *)a.k + b * a.k_sb + g * a.k_sh;
  const uint16_t *Vb = (const uint16_t *)a.v + b * a.v_sb + g * a.v_sh;
  const int skv32 = (int)a.Skv;  // sequence lengths are below 2^31
  const int trow = tid / CPR, tpos = tid % CPR;
  const int koff0 = trow * (int)a.k_ss * 2 + ((tpos ^ swz<D>(trow)) << 4);
  const int voff0 = trow * (int)a.v_ss * 2 + ((tpos ^ swz<D>(trow)) << 4);
  // Loads of tile j (entry e0 + j) into buffer j & 1: K at 2 * buf * TILEB, V after it.
  // First key of a key tile and the keys between its two 32-key blocks
  // (KIL: the plan has key-interleaved heads, with 128 x 64 tiles).
  auto ktile = [&](int kt) -> int2 {
    if constexpr (KIL) return key_tile_span(hm, kt);
    return make_int2(kt * TK, 0);
  };
  auto issue = [&](int j) {
    const int2 kt2 = ktile(((const cint32 *)a.ent_kt)[e0 + j]);
    const int k0 = kt2.x;
    const int left = min(skv32 - k0, TK + kt2.y);
    uint8_t *dst = lds + 2 * (j & 1) * TILEB;
    const v4u32 rk = raw_rsrc(Kb + (int64_t)k0 * a.k_ss, (left - 1) * (int)a.k_ss * 2 + D * 2);
    const v4u32 rv = raw_rsrc(Vb + (int64_t)k0 * a.v_ss, (left - 1) * (int)a.v_ss * 2 + D * 2);
    // (assembly-issued: the reads of tile j do not wait for tile j+1's
    // loads; the loop waits for them at its top)
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      uint8_t *d = dst + (u * T + wave * 64) * 16;
      if (KIL && u * RPL >= 32) {  // rows of the tile's second 32-key block
        dma_b128_so(rk, koff0 + u * RPL * (int)a.k_ss * 2, lds_addr_of(d), kt2.y * (int)a.k_ss * 2);
        dma_b128_so(rv, voff0 + u * RPL * (int)a.v_ss * 2, lds_addr_of(d + TILEB), kt2.y * (int)a.v_ss * 2);
      } else {
        dma_b128(rk, koff0 + u * RPL * (int)a.k_ss * 2, lds_addr_of(d));
        dma_b128(rv, voff0 + u * RPL * (int)a.v_ss * 2, lds_addr_of(d + TILEB));
      }
    }
  };

  // Live-bit geometry of this wave's rows (as in the forward).
  const int iq_lo = qbase >> hm.lq;
  const int niq = hm.lq >= 5 ? 1 : (32 >> hm.lq);
  const uint64_t wbits = ((1ull << (hm.mk * niq)) - 1ull) << (iq_lo * hm.mk);
  const int qsub = ((qbase + n) >> hm.lq) * hm.mk;
  const int qlim0 = (int)max<int64_t>(-64, min<int64_t>(q0 + a.off, a.Skv));

  f32x16 dq[NDB];
#pragma unroll
  for (int u = 0; u < NDB; ++u) dq[u] = f32x16{};

  if (nent > 0) issue(0);
  for (int j = 0; j < nent; ++j) {
    __builtin_amdgcn_s_waitcnt(0);  // tile j has landed (this wave's part)
    __syncthreads();                // ... every wave's; tile j-1's buffer is free
    if (j + 1 < nent) issue(j + 1);
    const uint8_t *__restrict__ ks = lds + 2 * (j & 1) * TILEB;
    const uint8_t *__restrict__ vs = ks + TILEB;
    const int2 kt2 = ktile(((const cint32 *)a.ent_kt)[e0 + j]);
    const int kb0 = kt2.x;
    const uint32_t live = ((const cuint32 *)a.ent_live)[e0 + j];
    const bool need = (kb0 + kt2.y + TK > skv32) || (a.causal && kb0 + TK - 1 > qlim0) ||
                      ((uint64_t)live & wbits) != wbits;
    // Allowed keys of this lane's query as bit masks over the tile.
    uint64_t km[(TK + 63) / 64];
#pragma unroll
    for (int w64 = 0; w64 < (TK + 63) / 64; ++w64) km[w64] = ~0ull;
    if (need) {
      const uint32_t lbits = live >> qsub;
      // (a key-interleaved tile, never causal, has its first block whole
      // whenever the second lies kt2.y further on)
      int lim = skv32 - kb0 - kt2.y;
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
      const int kr = 32 * t + perm_rows(n);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(ks, kr, 2 * c + hh), qb[c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(vs, kr, 2 * c + hh), dob[c], dp, 0, 0, 0);
      }
      // dS of the block; tiles that need no mask (no sequence end, causal
      // diagonal or dead sub-block; rows without keys have lse2 = +inf and
      // so P = 0) skip the per-score key test.
      uint32_t dsw[8];
      auto ds_block = [&](auto masked) {
#pragma unroll
        for (int jj = 0; jj < 16; jj += 2) {
          float ds2[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const float arg = __builtin_fmaf(s[jj + x], a.scale_log2, -lse2);
            float p;
            if constexpr (decltype(masked)::value) {
              const int kl = 32 * t + 16 * ((jj + x) >> 3) + ((jj + x) & 7);  // without the 8*hh term
              const bool ok = (km[kl / 64] >> (kl % 64)) & 1ull;
              p = ok ? fexp2(arg) : 0.f;
            } else {
              p = fexp2(arg);
            }
            ds2[x] = p * (dp[jj + x] - delta);
          }
          dsw[jj / 2] = pack_bf16x2(ds2[0], ds2[1]);
        }
      };
      if (need) ds_block(std::true_type{});
      else ds_block(std::false_type{});
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 bop = as_bf16x8(dsw[4 * c2], dsw[4 * c2 + 1], dsw[4 * c2 + 2], dsw[4 * c2 + 3]);
#pragma unroll
        for (int u = 0; u < NDB; ++u)
          dq[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag_s<D>(ks, 32 * t + 16 * c2, 32 * u, lane),
                                                          bop, dq[u], 0, 0, 0);
      }
    }
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
// dK, dV per (batch, kv head, 128 keys)
// ---------------------------------------------------------------------------
// A workgroup owns 128 consecutive keys: NKT = 128 / TKP key tiles of the
// plan (TKP = 64 or 128), four waves of 32 keys. The query chunks (32 rows)
// that may see them come from the key-major chunk index built for the call;
// they stream through a ring of four LDS buffers with direct-to-LDS buffer
// loads issued three chunks ahead.
template <int D, int TKP>
__global__ __launch_bounds__(256) void k_bwd_dkdv(BwdArgs a) {
  constexpr int T = 256, KW = 128, NKT = KW / TKP, NBUF = 4;
  constexpr int ROWB = 2 * D;                   // bytes per row in LDS
  constexpr int CHB = 32 * ROWB;                // one 32-row chunk of Q or dO
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int RPL = T / CPR;                  // rows covered by one load
  constexpr int LOADS = 32 / RPL;               // loads per thread per chunk and tensor
  constexpr int BUFB = 2 * CHB + 1024;          // Q, dO, LSE (256 B), Delta (256 B), spare
  constexpr int LPC = 2 * LOADS + 1;            // vector-memory ops per thread per chunk
  constexpr int NDB = D / 32;
  static_assert((D == 128 && RPL % 16 == 0) || (D == 64 && RPL % 16 == 0), "swizzle period");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * BUFB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int nkt = (int)a.nkt, nqt = (int)a.nqt;
  const int nkp = (nkt + NKT - 1) / NKT;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int kp = item % nkp, g = (item / nkp) % a.Hkv, b = item / (nkp * a.Hkv);
  const int kt0 = kp * NKT;
  const int wkt = (32 * wave) / TKP;            // this wave's tile within the group
  const int kloc = (32 * wave) % TKP + n;       // this lane's key within its tile
  // This lane's key: the tile's first key plus its column, and past the
  // first 32 keys the gap of a key-interleaved head's 64-key tile (one query
  // head per kv head then, so the kv head's own metadata gives it).
  int key = (kt0 + wkt) * TKP + kloc;
  if constexpr (TKP == 64) {
    const int2 kt2 = key_tile_span(a.hm[g * a.G], kt0 + wkt);
    key = kt2.x + kloc + (kloc >= 32 ? kt2.y : 0);
  }
  const int skv32 = (int)a.Skv, sq32 = (int)a.Sq;  // sequence lengths are below 2^31
  const bool kvalid = key < skv32;
  const int lb = a.nlb == 1 ? 0 : b;

  // K and V rows of this lane's key as B operands (dims 16c + 8hh .. +8).
  bf16x8 kb[D / 16], vb[D / 16];
  {
    const uint16_t *kp_ = (const uint16_t *)a.k + b * a.k_sb + g * a.k_sh + (int64_t)(kvalid ? key : 0) * a.k_ss;
    const uint16_t *vp_ = (const uint16_t *)a.v + b * a.v_sb + g * a.v_sh + (int64_t)(kvalid ? key : 0) * a.v_ss;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      kb[c] = __builtin_bit_cast(bf16x8, kvalid ? *(const uint4 *)(kp_ + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0));
      vb[c] = __builtin_bit_cast(bf16x8, kvalid ? *(const uint4 *)(vp_ + 16 * c + 8 * hh) : make_uint4(0, 0, 0, 0));
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int u = 0; u < NDB; ++u) dk[u] = f32x16{}, dv[u] = f32x16{};

  // The query chunks that may see these keys: entries [e0, e1) of the
  // key-major chunk index (first query, packed head / geometry word, live
  // words), read with scalar loads.
  const int bucket = (lb * a.Hkv + g) * nkp + kp;
  const int e0 = ((const cint32 *)a.t_off)[bucket], e1 = ((const cint32 *)a.t_off)[bucket + 1];

  // ---- chunk loads straight into LDS ----
  // Thread tid fills 16-byte slot tid of each 4 KiB block of a chunk: row
  // tid / CPR, slot tid % CPR, which holds the row's chunk slot ^ swz(row).
  const int trow = tid / CPR, tpos = tid % CPR;
  const int qoff0 = trow * (int)a.q_ss * 2 + ((tpos ^ swz<D>(trow)) << 4);
  const int doff0 = trow * (int)a.do_ss * 2 + ((tpos ^ swz<D>(trow)) << 4);
  // Loads of the chunk with first query q0 and packed word meta into buffer buf.
  // The kv group's first head: Q and dO rows, and its LSE / Delta entries.
  const uint16_t *qgrp = (const uint16_t *)a.q + b * a.q_sb + (int64_t)(g * a.G) * a.q_sh;
  const uint16_t *dgrp = (const uint16_t *)a.dout + b * a.do_sb + (int64_t)(g * a.G) * a.do_sh;
  const int64_t rgrp = ((int64_t)b * a.Hq + g * a.G) * a.Sq;
  // LDS destinations as 32-bit addresses from the array's base, taken once
  // (a generic pointer turned back into an LDS address costs a null test
  // per load).
  const uint32_t lds0 = lds_addr_of(lds);
  auto issue_qm = [&](int q0, int meta, int buf) {
    const int hl = meta & 255;                  // head within the group
    const uint32_t dst = lds0 + buf * BUFB;
    const int rows = min(sq32 - q0, 32);        // rows of the chunk that exist (>= 1)
    // Element offsets within the group: 32-bit products when the host found
    // that every such offset fits (one wave issues every instruction here).
    int64_t qo, dof, ro;
    if (a.grp32) {
      qo = (uint32_t)(hl * a.q_sh32 + q0 * a.q_ss32);
      dof = (uint32_t)(hl * a.do_sh32 + q0 * a.do_ss32);
      ro = (uint32_t)(hl * sq32 + q0);
    } else {
      qo = hl * a.q_sh + (int64_t)q0 * a.q_ss;
      dof = hl * a.do_sh + (int64_t)q0 * a.do_ss;
      ro = hl * a.Sq + q0;
    }
    const uint16_t *qb_ = qgrp + qo;
    const uint16_t *db_ = dgrp + dof;
    const v4u32 rq = raw_rsrc(qb_, (rows - 1) * (int)a.q_ss * 2 + D * 2);
    const v4u32 rd = raw_rsrc(db_, (rows - 1) * (int)a.do_ss * 2 + D * 2);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const uint32_t dq_ = dst + (u * T + wave * 64) * 16;
      dma_b128(rq, qoff0 + u * RPL * (int)a.q_ss * 2, dq_);
      dma_b128(rd, doff0 + u * RPL * (int)a.do_ss * 2, dq_ + CHB);
    }
    // LSE in log2 units (wave 0) and Delta (wave 1) of the chunk's rows, one
    // dword per lane; waves 2 and 3 repeat the LSE load into a spare area so
    // that every wave has the same number of loads in flight per chunk.
    const int64_t rix = rgrp + ro;
    const float *src = wave == 1 ? a.delta + rix : a.lse2 + rix;
    const uint32_t dl = dst + 2 * CHB + (wave == 1 ? 256 : (wave == 0 ? 0 : 512 + 256 * (wave - 2)));
    dma_b32(raw_rsrc(src, rows * 4), lane * 4, dl);
  };
  auto issue = [&](int e, int buf) {
    issue_qm(((const cint32 *)a.t_q0)[e], ((const cint32 *)a.t_meta)[e], buf);
  };

  auto buf_of = [&](int e) { return lds + ((e - e0) & (NBUF - 1)) * BUFB; };
  const int pr = perm_rows(n);
  // A-operand fragment i of the S, dP MFMAs of the chunk in buffer t: even i
  // = Q rows, odd i = dO rows, dims 16 * (i / 2) + 8 * hh.
  auto sdp_frag = [&](const uint8_t *t, int i) { return row_frag<D>(t + (i & 1) * CHB, pr, 2 * (i >> 1) + hh); };
  // A-operand fragment i of the dV, dK MFMAs: i = 2 * (NDB * c2 + u) + (0: dO^T, 1: Q^T).
  auto dkv_frag = [&](const uint8_t *t, int i) {
    const int c2 = (i >> 1) / NDB, u = (i >> 1) % NDB;
    return tr_frag_s<D>(t + ((i & 1) ? 0 : CHB), 16 * c2, 32 * u, lane);
  };
  constexpr int SD = 2 * (D / 16);   // S and dP MFMAs per chunk
  constexpr int KV = 4 * NDB;        // dV and dK MFMAs per chunk
  // LDS operand reads run this many MFMA steps ahead of their use. At D = 128
  // (one wave per SIMD: nothing else covers the read latency) six steps
  // measured 1.4% faster than three and two (video-DiT, long video); at
  // D = 64 (two waves per SIMD) the deeper prefetch was neutral to 1% slower.
  constexpr int kAheadSD = D == 128 ? 6 : 3, kAheadKV = D == 128 ? 6 : 2;

  // ---- pipeline ----
  // Iteration e: chunk e+1 has landed and chunk e is still in LDS; chunks
  // e+2 and e+3 are loading. One straight-line block in a fixed order: each
  // S or dP MFMA of chunk e+1 is followed by a slice of chunk e's
  // exponentials (its S and dP came from the previous iteration), with LDS
  // operands read three steps ahead; then chunk e's dV and dK MFMAs with
  // their transpose reads two steps ahead. sched_barrier(0) keeps the
  // compiler from regrouping the steps.
  for (int j = 0; j < NBUF - 1 && e0 + j < e1; ++j) issue(e0 + j, j);
  f32x16 sa = f32x16{}, da = f32x16{};
  if (e0 < e1) {
    if (e0 + 2 < e1) BSA_WAIT_VM(2 * LPC);
    else if (e0 + 1 < e1) BSA_WAIT_VM(LPC);
    else BSA_WAIT_VM(0);
    __syncthreads();
    const uint8_t *t = buf_of(e0);
#pragma unroll
    for (int i = 0; i < SD; ++i) {
      const bf16x8 f = sdp_frag(t, i);
      if (i & 1) da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, vb[i >> 1], da, 0, 0, 0);
      else sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, kb[i >> 1], sa, 0, 0, 0);
    }
  }
  for (int e = e0; e < e1; ++e) {
    // chunk e's metadata (scalar loads, completed before the LDS work)
    const int q0 = ((const cint32 *)a.t_q0)[e];
    const int meta = ((const cint32 *)a.t_meta)[e];
    uint32_t live = ((const cuint32 *)a.t_live)[NKT * e];
    if (NKT == 2 && wkt == 1) live = ((const cuint32 *)a.t_live)[NKT * e + 1];
    const int e3 = min(e + 3, e1 - 1);  // chunk e+3 (clamped: unused past the end)
    const int q03 = ((const cint32 *)a.t_q0)[e3], meta3 = ((const cint32 *)a.t_meta)[e3];
    if (e + 2 < e1) BSA_WAIT_VM(LPC);
    else BSA_WAIT_VM(0);
    __syncthreads();  // chunk e+1 is in LDS; chunk e-1's buffer is free
    if (e + 3 < e1) issue_qm(q03, meta3, (e - e0 + 3) & (NBUF - 1));
    const uint8_t *tc = buf_of(e), *tn = buf_of(e + 1);  // tn is stale on the last chunk

    // Allowed query rows of this lane's key in chunk e, as a 32-bit mask:
    // live query sub-blocks (at least 16 rows each, so rows 0-15 and 16-31
    // each lie in one), rows that exist, and the causal bound.
    const int qoff = 32 * ((meta >> 8) & 7), lq = (meta >> 11) & 31, lk = (meta >> 16) & 31, mk = (meta >> 21) & 63;
    const int ik = kloc >> lk;
    const uint32_t lo16 = (live >> ((qoff >> lq) * mk + ik)) & 1u;
    const uint32_t hi16 = (live >> (((qoff + 16) >> lq) * mk + ik)) & 1u;
    uint32_t rows = (lo16 ? 0x0000ffffu : 0u) | (hi16 ? 0xffff0000u : 0u);
    const int nrow = sq32 - q0;
    if (nrow < 32) rows &= (1u << nrow) - 1u;
    if (a.causal) {
      const int64_t first = (int64_t)key - q0 - a.off;  // first query row that may see the key
      rows = first <= 0 ? rows : (first >= 32 ? 0u : rows & ~((1u << first) - 1u));
    }
    if (!kvalid) rows = 0u;
    const uint32_t myrows = rows >> (8 * hh);  // bit 16*(j/8) + (j%8) <-> accumulator j
    const float *lse_s = (const float *)(tc + 2 * CHB), *del_s = lse_s + 64;
    float lrow[16], drow[16];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const float4 l0 = *(const float4 *)(lse_s + 16 * h2 + 8 * hh), l1 = *(const float4 *)(lse_s + 16 * h2 + 8 * hh + 4);
      const float4 d0 = *(const float4 *)(del_s + 16 * h2 + 8 * hh), d1 = *(const float4 *)(del_s + 16 * h2 + 8 * hh + 4);
      lrow[8 * h2 + 0] = l0.x, lrow[8 * h2 + 1] = l0.y, lrow[8 * h2 + 2] = l0.z, lrow[8 * h2 + 3] = l0.w;
      lrow[8 * h2 + 4] = l1.x, lrow[8 * h2 + 5] = l1.y, lrow[8 * h2 + 6] = l1.z, lrow[8 * h2 + 7] = l1.w;
      drow[8 * h2 + 0] = d0.x, drow[8 * h2 + 1] = d0.y, drow[8 * h2 + 2] = d0.z, drow[8 * h2 + 3] = d0.w;
      drow[8 * h2 + 4] = d1.x, drow[8 * h2 + 5] = d1.y, drow[8 * h2 + 6] = d1.z, drow[8 * h2 + 7] = d1.w;
    }

    f32x16 sb, db2;
    uint32_t pw[8], dw[8];
    float pe = 0.f, de = 0.f;
    // One wave issues everything on its SIMD here, so instructions count: a
    // chunk whose every row is allowed for every key of the wave (the usual
    // case away from the causal diagonal and the sequence end) takes its
    // exponentials without the per-score row test.
    auto sdp_pass = [&](auto masked) {
      bf16x8 fr[SD];
#pragma unroll
      for (int i = 0; i < kAheadSD; ++i) fr[i] = sdp_frag(tn, i);
#pragma unroll
      for (int i = 0; i < SD; ++i) {
        if (i + kAheadSD < SD) fr[i + kAheadSD] = sdp_frag(tn, i + kAheadSD);
        if (i & 1) db2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], vb[i >> 1], i == 1 ? f32x16{} : db2, 0, 0, 0);
        else sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], kb[i >> 1], i == 0 ? f32x16{} : sb, 0, 0, 0);
        // P and dS of chunk e: 16 / SD accumulators per step, packed to bf16
        // pairs as the odd element of each pair is done.
#pragma unroll
        for (int k2 = 0; k2 < 16 / SD; ++k2) {
          const int x = i * (16 / SD) + k2;  // accumulator index
          const float arg = __builtin_fmaf(sa[x], a.scale_log2, -lrow[x]);  // (lrow in log2 units)
          float p;
          if constexpr (decltype(masked)::value) {
            // Allowed pairs have a finite LSE (the row has a key).
            const bool ok = (myrows >> (16 * (x >> 3) + (x & 7))) & 1u;
            p = ok ? fexp2(arg) : 0.f;
          } else {
            p = fexp2(arg);
          }
          const float dd = p * (da[x] - drow[x]);
          if (x & 1) {
            pw[x >> 1] = pack_bf16x2(pe, p);
            dw[x >> 1] = pack_bf16x2(de, dd);
          } else {
            pe = p, de = dd;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (__all(rows == 0xffffffffu)) sdp_pass(std::false_type{});
    else sdp_pass(std::true_type{});
    {
      bf16x8 fr[KV];
#pragma unroll
      for (int i = 0; i < kAheadKV; ++i) fr[i] = dkv_frag(tc, i);
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        if (i + kAheadKV < KV) fr[i + kAheadKV] = dkv_frag(tc, i + kAheadKV);
        const int c2 = (i >> 1) / NDB, u = (i >> 1) % NDB;
        if (i & 1) {
          const bf16x8 db = as_bf16x8(dw[4 * c2], dw[4 * c2 + 1], dw[4 * c2 + 2], dw[4 * c2 + 3]);
          dk[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], db, dk[u], 0, 0, 0);
        } else {
          const bf16x8 pb = as_bf16x8(pw[4 * c2], pw[4 * c2 + 1], pw[4 * c2 + 2], pw[4 * c2 + 3]);
          dv[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], pb, dv[u], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    sa = sb, da = db2;
  }

  if (kvalid) {
    uint16_t *kp_ = (uint16_t *)a.dk + b * a.dk_sb + g * a.dk_sh + (int64_t)key * a.dk_ss;
    uint16_t *vp_ = (uint16_t *)a.dv + b * a.dv_sb + g * a.dv_sh + (int64_t)key * a.dv_ss;
#pragma unroll
    for (int u = 0; u < NDB; ++u)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * u + 8 * q4 + 4 * hh;
        *(uint2 *)(kp_ + d0) = make_uint2(pack_bf16x2(dk[u][4 * q4] * a.scale, dk[u][4 * q4 + 1] * a.scale),
                                          pack_bf16x2(dk[u][4 * q4 + 2] * a.scale, dk[u][4 * q4 + 3] * a.scale));
        *(uint2 *)(vp_ + d0) = make_uint2(pack_bf16x2(dv[u][4 * q4], dv[u][4 * q4 + 1]),
                                          pack_bf16x2(dv[u][4 * q4 + 2], dv[u][4 * q4 + 3]));
      }
  }
}

template <int D, int TK>
void launch_dq(const BwdArgs &a, int tq, bool kil, unsigned grid, hipStream_t s) {
  if (tq == 256) hipLaunchKernelGGL((k_bwd_dq<D, TK, 256>), dim3(grid), dim3(512), 0, s, a);
  else if constexpr (TK == 64)
    if (kil) hipLaunchKernelGGL((k_bwd_dq<D, TK, 128, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dq<D, TK, 128>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_bwd_dq<D, TK, 128>), dim3(grid), dim3(256), 0, s, a);
}

template <int D>
void launch_d(const BwdArgs &a, bool kil, unsigned dq_grid, unsigned kv_grid, hipStream_t s) {
  if (dq_grid) {
    if (a.tk == 128) launch_dq<D, 128>(a, a.tq, false, dq_grid, s);
    else launch_dq<D, 64>(a, a.tq, kil, dq_grid, s);
  }
  if (kv_grid) {
    if (a.tk == 128) hipLaunchKernelGGL((k_bwd_dkdv<D, 128>), dim3(kv_grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dkdv<D, 64>), dim3(kv_grid), dim3(256), 0, s, a);
  }
}

}  // namespace

bsa_status backward_launch(const Plan &p, const BwdArgs &a, hipStream_t s) {
  const int64_t kv_items = (int64_t)p.B * p.Hkv * ((p.nkt * p.rg.tk + 127) / 128);
  if (p.nrows > 0x7fffffff || kv_items > 0x7fffffff)
    return fail(BSA_ERR_UNSUPPORTED, "too many tiles for one launch");
  const unsigned dq_grid = (unsigned)p.nrows, kv_grid = (unsigned)kv_items;
  if (p.D == 128) launch_d<128>(a, p.key_interleaved, dq_grid, kv_grid, s);
  else launch_d<64>(a, p.key_interleaved, dq_grid, kv_grid, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BSA_ERR_HIP, std::string("backward launch: ") + hipGetErrorString(e));
  return BSA_OK;
}

}  // namespace bsa
