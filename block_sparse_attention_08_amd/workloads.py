"""Seeded synthetic workloads for block-sparse attention.

This module only draws random inputs: logical block masks, Q/K/V values and
page tables. It holds none of the attention arithmetic, so the tests, the
benchmark and the CPU oracle can all use it without sharing any method code.

Workload shapes follow the workloads the pages evaluate on, none of which
ship here (real video-diffusion masks, model weights, long-context prompts);
the generators below stand in for them:

* ``tiny``: a 4x4-block Bernoulli(0.5) mask with the diagonal forced on, fp32.
* ``video_dit``: a video-DiT latent grid tokenised in 3-D tiles, with a local
  3-D window plus random global blocks per head (Tessera, abstract: masks
  from video diffusion models; Veda: per-head 3-D tile geometry).
* ``chunked_prefill``: a GQA query chunk over a paged KV cache, with per
  query block top-10% key-block selection from random logits under a causal
  constraint (CompactAttention: block mask used as a KV selection signal).
* ``affine``: sliding-window, dilated and window+global patterns at 32/64
  block sizes (SPLAT, abstract: regular sparse-MHSA patterns at 10-50%
  density).
* ``long_video``: per-head block sizes 64/128/256 over a nested 3-D token
  order, 3-D local window plus random tiles, with empty and heavy query rows.

Masks are ``uint8`` arrays laid out as the library expects: for each mask
batch ``bm`` and head ``h`` a row-major ``[nqb_h][nkb_h]`` block, blocks
concatenated in ``(bm, h)`` order. Q/K/V are standard-normal values rounded
to bf16 (round to nearest even) unless the workload is fp32.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# Workload ids used as the first word of every SeedSequence.
WID_TINY, WID_VIDEO, WID_PREFILL, WID_AFFINE, WID_LONG, WID_DECODE, WID_RANDOM = 1, 2, 3, 4, 5, 6, 9
WID_PERIODIC = 10
# Second word: which stream of random numbers.
STREAM_QKV, STREAM_MASK, STREAM_PAGES, STREAM_DOUT = 0, 1, 2, 3


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclasses.dataclass
class Workload:
    """One block-sparse attention problem with its seeded inputs."""

    name: str
    batch: int
    hq: int
    hkv: int
    sq: int
    skv: int
    d: int
    dtype: str                      # "bf16" or "f32"
    bq: List[int]                   # per q-head logical block sizes
    bk: List[int]
    mask: np.ndarray                # uint8, flat, (bm, h, qb, kb) order
    mask_broadcast: bool = False
    causal: bool = False
    causal_offset: int = 0
    gqa_union: bool = False
    paged: bool = False
    page_size: int = 0
    pages_per_seq: int = 0
    num_pages: int = 0
    page_table: Optional[np.ndarray] = None   # int32 [batch][pages_per_seq]
    seed: Tuple[int, ...] = (0,)
    # per head, the pattern as affine runs (row_num, row_den, offset, stride,
    # count) when the workload is defined by one (the input of bsa_plan_acsr)
    acsr: Optional[List[List[Tuple[int, int, int, int, int]]]] = None
    # storage order inside a page of a paged pool: "nhd" (token, head, dim)
    # or "hnd" (head, token, dim: one kv head's rows of a page contiguous);
    # the tensors keep the logical [page][token][head][dim] shape either way
    kv_layout: str = "nhd"

    # ---- geometry helpers (pure bookkeeping, no attention arithmetic) ----
    @property
    def mask_batches(self) -> int:
        return 1 if self.mask_broadcast else self.batch

    def nqb(self, h: int) -> int:
        return cdiv(self.sq, self.bq[h])

    def nkb(self, h: int) -> int:
        return cdiv(self.skv, self.bk[h])

    def head_mask(self, bm: int, h: int) -> np.ndarray:
        """View of the [nqb][nkb] logical mask of mask-batch bm, head h."""
        off = 0
        for b2 in range(self.mask_batches):
            for h2 in range(self.hq):
                n = self.nqb(h2) * self.nkb(h2)
                if b2 == bm and h2 == h:
                    return self.mask[off:off + n].reshape(self.nqb(h), self.nkb(h))
                off += n
        raise IndexError((bm, h))

    def q_shape(self):
        return (self.batch, self.hq, self.sq, self.d)

    def kv_shape(self):
        if self.paged:
            return (self.num_pages, self.page_size, self.hkv, self.d)
        return (self.batch, self.hkv, self.skv, self.d)

    # ---- values ----
    def make_qkv(self, device: str = "cpu"):
        """Q, K, V as torch tensors of the workload dtype.

        On the CPU the values come from numpy PCG64 (stream 0 of the workload
        seed: Q, then K, then V). For large shapes on a GPU, ``device="cuda"``
        draws them with torch's seeded CUDA generator instead, which is far
        faster; callers that need host copies copy the device tensors back.
        """
        import torch

        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        shapes = [self.q_shape(), self.kv_shape(), self.kv_shape()]
        if device == "cpu":
            g = _rng(*self.seed, STREAM_QKV)
            out = []
            for shp in shapes:
                x = g.standard_normal(int(np.prod(shp)), dtype=np.float32)
                if self.dtype == "bf16":
                    t = torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16)
                else:
                    t = torch.from_numpy(x)
                out.append(t.reshape(shp))
            return tuple(self._layout(t, i) for i, t in enumerate(out))

        gen = torch.Generator(device=device)
        gen.manual_seed(int(np.random.SeedSequence(list(self.seed) + [STREAM_QKV]).generate_state(1)[0]))
        out = []
        for shp in shapes:
            x = torch.randn(shp, generator=gen, device=device, dtype=torch.float32)
            out.append(x.to(tdt))
            del x
        return tuple(self._layout(t, i) for i, t in enumerate(out))

    def _layout(self, t, i: int):
        """K and V (i = 1, 2) of a paged pool in the workload's in-page order:
        the same values, stored head-major for "hnd"."""
        if i == 0 or not self.paged or self.kv_layout == "nhd":
            return t
        assert self.kv_layout == "hnd"
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)

    def make_dout(self, device: str = "cpu"):
        """Upstream gradient dL/dO for a backward pass: N(0,1) of Q's shape and
        dtype, from its own stream of the workload seed (numpy on the CPU,
        torch's seeded generator on a GPU, as for make_qkv)."""
        import torch

        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        shp = self.q_shape()
        if device == "cpu":
            x = _rng(*self.seed, STREAM_DOUT).standard_normal(int(np.prod(shp)), dtype=np.float32)
            if self.dtype == "bf16":
                return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).reshape(shp)
            return torch.from_numpy(x).reshape(shp)
        gen = torch.Generator(device=device)
        gen.manual_seed(int(np.random.SeedSequence(list(self.seed) + [STREAM_DOUT]).generate_state(1)[0]))
        return torch.randn(shp, generator=gen, device=device, dtype=torch.float32).to(tdt)

    def make_kv8(self, k, v):
        """K and V quantized to OCP FP8 E4M3 with one fp32 scale per kv head
        (max |x| of the head maps to 448, the largest finite e4m3 value),
        rounded to nearest by torch's float8_e4m3fn conversion. Returns
        (k8, v8, k_scale, v_scale): uint8 tensors of K's layout and fp32 [Hkv]
        scales, on K's device."""
        import torch

        head_axis = 2 if self.paged else 1
        out = []
        for x in (k, v):
            xf = x.float()
            dims = [i for i in range(4) if i != head_axis]
            amax = xf.abs().amax(dim=dims)
            scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
            shp = [1, 1, 1, 1]
            shp[head_axis] = -1
            q8 = (xf / scale.view(shp)).to(torch.float8_e4m3fn).view(torch.uint8)
            out.append((self._layout(q8.contiguous(), 1), scale.contiguous()))
        return out[0][0], out[1][0], out[0][1], out[1][1]

    def problem_dict(self) -> dict:
        return dict(
            batch=self.batch, num_q_heads=self.hq, num_kv_heads=self.hkv,
            seqlen_q=self.sq, seqlen_kv=self.skv, head_dim=self.d, dtype=self.dtype,
            block_q=list(self.bq), block_k=list(self.bk),
            mask_batch_broadcast=int(self.mask_broadcast), causal=int(self.causal),
            causal_kv_offset=self.causal_offset, gqa_union=int(self.gqa_union),
            paged=int(self.paged), page_size=self.page_size,
            pages_per_seq=self.pages_per_seq, num_pages=self.num_pages,
        )


def _concat(blocks: List[np.ndarray]) -> np.ndarray:
    return np.ascontiguousarray(np.concatenate([b.reshape(-1) for b in blocks]).astype(np.uint8))


# --------------------------------------------------------------------------
# Tiny fp32 case
# --------------------------------------------------------------------------
def tiny(seed: int = 0) -> Workload:
    """B=1, H=2, S=256, D=64, fp32; 64x64 blocks; Bernoulli(0.5), diagonal on."""
    h, s, bs = 2, 256, 64
    nb = s // bs
    g = _rng(WID_TINY, seed, STREAM_MASK)
    blocks = []
    for _ in range(h):
        m = (g.random((nb, nb)) < 0.5).astype(np.uint8)
        np.fill_diagonal(m, 1)
        blocks.append(m)
    return Workload("tiny", 1, h, h, s, s, 64, "f32", [bs] * h, [bs] * h, _concat(blocks),
                    seed=(WID_TINY, seed))


# --------------------------------------------------------------------------
# Video-DiT 3-D window + random global blocks
# --------------------------------------------------------------------------
def video_dit(heads: int = 24, grid=(16, 30, 52), tile=(16, 2, 4), d: int = 128,
              window=(1, 2, 2), p_global: float = 0.03, seed: int = 0) -> Workload:
    """Latent grid ``grid`` flattened in 3-D tile order; one logical block per tile.

    With the default grid 16x30x52 and 128-token tiles, the only tiling into
    full tiles is (16, 2, 4), giving a 1x15x13 tile grid and 195 blocks; the
    window in t is then vacuous. Each head draws its own random global blocks.
    """
    gt, gh, gw = (grid[i] // tile[i] for i in range(3))
    assert all(grid[i] % tile[i] == 0 for i in range(3))
    bs = tile[0] * tile[1] * tile[2]
    nb = gt * gh * gw
    s = nb * bs
    idx = np.arange(nb)
    ct, ch, cw = idx // (gh * gw), (idx // gw) % gh, idx % gw
    win = ((np.abs(ct[:, None] - ct[None, :]) <= window[0])
           & (np.abs(ch[:, None] - ch[None, :]) <= window[1])
           & (np.abs(cw[:, None] - cw[None, :]) <= window[2]))
    blocks = []
    for h in range(heads):
        g = _rng(WID_VIDEO, seed, STREAM_MASK, h)
        blocks.append((win | (g.random((nb, nb)) < p_global)).astype(np.uint8))
    return Workload("video_dit", 1, heads, heads, s, s, d, "bf16", [bs] * heads, [bs] * heads,
                    _concat(blocks), seed=(WID_VIDEO, seed))


# --------------------------------------------------------------------------
# Chunked-prefill GQA over a paged cache
# --------------------------------------------------------------------------
def chunked_prefill(hq: int = 32, hkv: int = 8, d: int = 128, chunk: int = 4096,
                    context: int = 65536, page: int = 64, block: int = 128,
                    keep_tenths: int = 1, seed: int = 0) -> Workload:
    """The chunk holds the last ``chunk`` positions of a ``context``-token cache.

    Query i sits at absolute position ``context - chunk + i``; key j is allowed
    only if ``j <= i + (context - chunk)``. For each head and query block the
    candidates are the key blocks whose first key is not after the block's last
    query; the top ceil(n * keep_tenths / 10) by i.i.d. N(0,1) logit are kept
    (ties to the lower block index).
    """
    assert chunk % block == 0 and context % block == 0 and context % page == 0
    off = context - chunk
    nqb, nkb = chunk // block, context // block
    blocks = []
    for h in range(hq):
        g = _rng(WID_PREFILL, seed, STREAM_MASK, h)
        logits = g.standard_normal((nqb, nkb))
        m = np.zeros((nqb, nkb), np.uint8)
        for qb in range(nqb):
            last_q = off + (qb + 1) * block - 1
            ncand = last_q // block + 1
            k = (ncand * keep_tenths + 9) // 10
            order = np.lexsort((np.arange(ncand), -logits[qb, :ncand]))
            m[qb, order[:k]] = 1
        blocks.append(m)
    pps = context // page
    gp = _rng(WID_PREFILL, seed, STREAM_PAGES)
    table = gp.permutation(pps).astype(np.int32).reshape(1, pps)
    return Workload("chunked_prefill", 1, hq, hkv, chunk, context, d, "bf16",
                    [block] * hq, [block] * hq, _concat(blocks), causal=True,
                    causal_offset=off, gqa_union=True, paged=True, page_size=page,
                    pages_per_seq=pps, num_pages=pps, page_table=table,
                    seed=(WID_PREFILL, seed))


# --------------------------------------------------------------------------
# Decode and short chunks over a paged cache
# --------------------------------------------------------------------------
def decode(batch: int = 16, hq: int = 32, hkv: int = 8, d: int = 128, q_len: int = 1,
           context: int = 65536, page: int = 64, block: int = 128, keep_tenths: int = 1,
           kv_layout: str = "nhd",
           seed: int = 0) -> Workload:
    """A batch of sequences, each with ``q_len`` new tokens at the end of a
    ``context``-token paged cache (decode: one token; a short chunk, such as
    speculative verification: a few).

    Query i of a sequence sits at ``context - q_len + i``; key j is allowed
    only if ``j <= i + context - q_len``. Per sequence and head, the query
    block keeps the top ceil(n * keep_tenths / 10) of its n causal candidate
    key blocks by i.i.d. N(0,1) logit (ties to the lower block), and the
    heads of a kv group attend to the union of their selections, as in
    chunked prefill. Every sequence reads its own pages of one pool through
    a random permutation.
    """
    assert context % block == 0 and context % page == 0 and 1 <= q_len <= context
    off = context - q_len
    nqb, nkb = cdiv(q_len, block), context // block
    blocks = []
    for b in range(batch):
        for h in range(hq):
            g = _rng(WID_DECODE, seed, STREAM_MASK, b, h)
            logits = g.standard_normal((nqb, nkb))
            m = np.zeros((nqb, nkb), np.uint8)
            for qb in range(nqb):
                last_q = off + min((qb + 1) * block, q_len) - 1
                ncand = last_q // block + 1
                k = (ncand * keep_tenths + 9) // 10
                order = np.lexsort((np.arange(ncand), -logits[qb, :ncand]))
                m[qb, order[:k]] = 1
            blocks.append(m)
    pps = context // page
    gp = _rng(WID_DECODE, seed, STREAM_PAGES)
    table = gp.permutation(batch * pps).astype(np.int32).reshape(batch, pps)
    return Workload("decode", batch, hq, hkv, q_len, context, d, "bf16", [block] * hq,
                    [block] * hq, _concat(blocks), causal=True, causal_offset=off, gqa_union=True,
                    paged=True, page_size=page, pages_per_seq=pps, num_pages=batch * pps,
                    page_table=table, seed=(WID_DECODE, seed, q_len), kv_layout=kv_layout)


# --------------------------------------------------------------------------
# Regular (affine) patterns
# --------------------------------------------------------------------------
def affine_pattern(kind: int, nb: int, bs: int, window: int, stride: int = 8,
                   n_global: int = 2) -> np.ndarray:
    qb = np.arange(nb)[:, None]
    kb = np.arange(nb)[None, :]
    wb = window // bs
    if kind == 0:
        m = np.abs(qb - kb) <= wb
    elif kind == 1:
        m = ((qb - kb) % stride) == 0
    else:
        m = (np.abs(qb - kb) <= wb) | (kb < n_global)
    return m.astype(np.uint8)


def affine_runs(kind: int, nb: int, bs: int, window: int, stride: int = 8,
                n_global: int = 2) -> List[Tuple[int, int, int, int, int]]:
    """The pattern of affine_pattern(kind, ...) as affine runs (row_num,
    row_den, offset, stride, count): the window |qb - kb| <= w is the run of
    2w + 1 blocks from qb - w; the dilated pattern kb = qb (mod stride) is a
    run of that stride from far enough below 0 to past nb; the global columns
    are a run of slope 0."""
    wb = window // bs
    reach = -(-nb // stride)
    if kind == 0:
        return [(1, 1, -wb, 1, 2 * wb + 1)]
    if kind == 1:
        return [(1, 1, -stride * reach, stride, 2 * reach + 1)]
    return [(1, 1, -wb, 1, 2 * wb + 1), (0, 1, 0, 1, n_global)]


def affine(bs: int = 64, batch: int = 2, heads: int = 16, s: int = 16384, d: int = 64,
           window: int = 1024, seed: int = 0) -> Workload:
    """Per head h the pattern h mod 3: window, stride-8 dilated, window+first-2 columns."""
    nb = cdiv(s, bs)
    blocks = [affine_pattern(h % 3, nb, bs, window) for h in range(heads)]
    return Workload(f"affine_bs{bs}", batch, heads, heads, s, s, d, "bf16", [bs] * heads,
                    [bs] * heads, _concat(blocks), mask_broadcast=True,
                    seed=(WID_AFFINE, seed, bs, window),
                    acsr=[affine_runs(h % 3, nb, bs, window) for h in range(heads)])


def random_acsr(batch: int = 1, hq: int = 3, hkv: Optional[int] = None, sq: int = 700,
                skv: int = 900, d: int = 64, bq=64, bk=64, max_runs: int = 3,
                causal: bool = False, causal_offset: int = 0, seed: int = 0) -> Workload:
    """Random affine runs per head (slopes 0, 1/2, 1, 3/2, 2 and -1, offsets,
    strides 1..5, counts, overlapping runs). The mask is left empty: it is
    what the runs expand to, which the oracle computes."""
    hkv = hq if hkv is None else hkv
    bqs = list(bq) if isinstance(bq, (list, tuple)) else [bq] * hq
    bks = list(bk) if isinstance(bk, (list, tuple)) else [bk] * hq
    g = _rng(WID_RANDOM, seed, STREAM_MASK)
    slopes = [(0, 1), (1, 2), (1, 1), (3, 2), (2, 1), (-1, 1)]
    heads = []
    for h in range(hq):
        nk = cdiv(skv, bks[h])
        runs = []
        for _ in range(int(g.integers(1, max_runs + 1))):
            num, den = slopes[int(g.integers(0, len(slopes)))]
            st = int(g.integers(1, 6))
            cnt = int(g.integers(1, max(2, nk // st + 2)))
            off = int(g.integers(-nk, nk))
            runs.append((num, den, off, st, cnt))
        heads.append(runs)
    return Workload("random_acsr", batch, hq, hkv, sq, skv, d, "bf16", bqs, bks,
                    np.zeros(0, np.uint8), mask_broadcast=True, causal=causal,
                    causal_offset=causal_offset, seed=(WID_RANDOM, seed, 77), acsr=heads)


# --------------------------------------------------------------------------
# Long-video mixed geometry
# --------------------------------------------------------------------------
def _long_video_coords(bs: int, l2grid):
    """3-D coordinates of each logical block in the head's own tile grid.

    Tokens are ordered by level-2 tiles of (2, 8, 16) in raster order; each
    level-2 tile holds two (2, 8, 8) halves along w, each half holds two
    (1, 8, 8) slices along t. Blocks of 256/128/64 tokens are these tiles.
    """
    t2n, h2n, w2n = l2grid
    if bs == 256:
        c = np.arange(t2n * h2n * w2n)
        return np.stack(np.unravel_index(c, l2grid), 1)
    if bs == 128:
        c = np.arange(2 * t2n * h2n * w2n)
        t2, h2, w2 = np.unravel_index(c >> 1, l2grid)
        return np.stack([t2, h2, 2 * w2 + (c & 1)], 1)
    if bs == 64:
        c = np.arange(4 * t2n * h2n * w2n)
        t2, h2, w2 = np.unravel_index(c >> 2, l2grid)
        return np.stack([2 * t2 + (c & 1), h2, 2 * w2 + ((c >> 1) & 1)], 1)
    raise ValueError(bs)


LONG_VIDEO_P = {64: 0.053, 128: 0.041, 256: 0.020}


def long_video(heads: int = 40, grid=(30, 48, 80), d: int = 128, p_empty: float = 0.10,
               p_heavy: float = 0.05, heavy_density: float = 0.40, seed: int = 0) -> Workload:
    """Per-head block size [64, 128, 256][h % 3] over a nested 3-D token order."""
    l2 = (grid[0] // 2, grid[1] // 8, grid[2] // 16)
    assert grid[0] % 2 == 0 and grid[1] % 8 == 0 and grid[2] % 16 == 0
    s = grid[0] * grid[1] * grid[2]
    bsz = [(64, 128, 256)[h % 3] for h in range(heads)]
    blocks = []
    for h in range(heads):
        bs = bsz[h]
        c = _long_video_coords(bs, l2)
        nb = c.shape[0]
        win = np.ones((nb, nb), bool)
        for ax in range(3):
            win &= np.abs(c[:, None, ax] - c[None, :, ax]) <= 1
        g = _rng(WID_LONG, seed, STREAM_MASK, h)
        u = g.random(nb)
        r = g.random((nb, nb))
        heavy = (u >= p_empty) & (u < p_empty + p_heavy)
        empty = u < p_empty
        p = np.where(heavy, heavy_density, LONG_VIDEO_P[bs])[:, None]
        m = (win | (r < p)) & ~empty[:, None]
        blocks.append(m.astype(np.uint8))
    return Workload("long_video", 1, heads, heads, s, s, d, "bf16", bsz, bsz, _concat(blocks),
                    seed=(WID_LONG, seed))


# --------------------------------------------------------------------------
# Periodic rows (dilated patterns of several periods) with random blocks
# --------------------------------------------------------------------------
def periodic(batch: int = 2, bq=(32, 64, 64, 32), sq: int = 2048, skv: int = 1024, bk: int = 64,
             d: int = 64, periods=(2, 4, 8, 1), p_random: float = 0.03, causal: bool = False,
             causal_offset: int = 0, seed: int = 0) -> Workload:
    """Per head h, key block kb is selected in query block qb when
    (kb - qb) is a multiple of periods[h] (period 1: a band |kb - qb/2| <= 2),
    plus Bernoulli(p_random) blocks; one mask per batch element."""
    g = _rng(WID_PERIODIC, seed, STREAM_MASK)
    hq = len(bq)
    blocks = []
    for _ in range(batch):
        for h in range(hq):
            nq, nk = cdiv(sq, bq[h]), cdiv(skv, bk)
            qb = np.arange(nq)[:, None]
            kb = np.arange(nk)[None, :]
            per = periods[h]
            m = ((kb - qb) % per == 0) if per > 1 else (np.abs(kb - qb // 2) <= 2)
            m = m | (g.random((nq, nk)) < p_random)
            blocks.append(m.astype(np.uint8))
    return Workload("periodic", batch, hq, hq, sq, skv, d, "bf16", list(bq), [bk] * hq, _concat(blocks),
                    causal=causal, causal_offset=causal_offset, seed=(WID_PERIODIC, seed))


# --------------------------------------------------------------------------
# Random problems for edge cases (ragged lengths, GQA, causal, paged, empty)
# --------------------------------------------------------------------------
def random_problem(batch=1, hq=2, hkv=None, sq=300, skv=333, d=64, dtype="bf16", bq=64,
                   bk=64, density=0.5, mask_broadcast=False, causal=False, causal_offset=0,
                   gqa_union=False, paged=False, page_size=64, empty_rows=0.0,
                   seed=0) -> Workload:
    """A small random problem; ``bq``/``bk`` may be ints or per-head lists."""
    hkv = hq if hkv is None else hkv
    bqs = list(bq) if isinstance(bq, (list, tuple)) else [bq] * hq
    bks = list(bk) if isinstance(bk, (list, tuple)) else [bk] * hq
    g = _rng(WID_RANDOM, seed, STREAM_MASK)
    bm = 1 if mask_broadcast else batch
    blocks = []
    for _ in range(bm):
        for h in range(hq):
            nq, nk = cdiv(sq, bqs[h]), cdiv(skv, bks[h])
            m = g.random((nq, nk)) < density
            m &= (g.random(nq) >= empty_rows)[:, None]
            blocks.append(m.astype(np.uint8))
    w = Workload("random", batch, hq, hkv, sq, skv, d, dtype, bqs, bks, _concat(blocks),
                 mask_broadcast=mask_broadcast, causal=causal, causal_offset=causal_offset,
                 gqa_union=gqa_union, seed=(WID_RANDOM, seed))
    if paged:
        pps = cdiv(skv, page_size)
        gp = _rng(WID_RANDOM, seed, STREAM_PAGES)
        npages = batch * pps + 3
        perm = gp.permutation(npages)[: batch * pps]
        w.paged, w.page_size, w.pages_per_seq, w.num_pages = True, page_size, pps, npages
        w.page_table = perm.astype(np.int32).reshape(batch, pps)
    return w
