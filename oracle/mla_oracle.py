"""Plain fp64 CPU oracle for DeepSeek MLA decode.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The GPU library never
calls it, and it shares no code with the GPU library.

What it computes (one query token per sequence, one shared latent KV head):

* Sources.  "用 TileLang 编写高性能 DeepSeek MLA 内核" (the TileLang MLA guide),
  sections "先看核心难点" (Q/K head dim 576 = 512 latent + 64 RoPE, V head dim
  512) and "参考实现与正确性验证" (the reference joins q with q_pe and kv with
  k_pe along the last axis, forms scores with an einsum, applies softmax and
  takes the weighted sum of the value rows).  "DeepSeek开源周第一天：FlashMLA
  深度分析" (the FlashMLA analysis), last section, states the same Q=576 / V=512
  split.  V is the latent slice of the same cache row.
* For sequence b with L = cache_seqlens[b] valid rows, row j of the cache is
  K_j = latent_j ‖ rope_j (576 values) and V_j = latent_j (512 values).
* z[h, j] = softmax_scale * (q_nope[b,h] · latent_j + q_pe[b,h] · rope_j)
* lse[b, h] = ln Σ_j exp(z[h, j])            (natural log; -inf when L = 0)
* out[b, h] = Σ_j exp(z[h, j] - lse[b, h]) V_j   (zero when L = 0)

Paged layout: the TileLang guide's "变体内核" section (paged variant: rows are
found through block_table and positions at or past cache_seqlens are masked)
and the FlashMLA analysis's parameter struct (block_table, page_block_size).
Logical row j of sequence b lives in physical page block_table[b, j // page]
at offset j % page.

Split mode follows the guide's "Split Kernel" and "Combine Kernel" sections:
each KV range yields a normalised partial output and a base-2 log-sum-exp of
the scaled scores; the combine takes the largest partial lse as anchor, forms
the base-2 log of the summed exponentials, and weights each partial by
exp2(lse_k - lse_total).  How ranges are cut is a reading (the pages' paged
variant speaks of blocks_per_split and remaining_blocks): the valid length is
cut into 64-row blocks, split k of s gets floor(nb/s) blocks plus one more when
k < nb mod s, in order.

Several query tokens per sequence (speculative / multi-token decode): the
FlashMLA analysis's parameter struct carries seqlen_q and is_causal.  Reading:
the s = seqlen_q new tokens are the last s rows of the cache, and query token t
(0-based, the newest last) sees rows j < L - (s - 1 - t); its H heads are query
rows t*H .. t*H + H - 1 of the sequence (token-major).  s = 1 is plain decode.

Readings where the pages are silent:
* lse is returned in natural-log units (the kernel's base-2 value times ln 2).
* L = 0 gives out = 0 and lse = -inf; an empty split contributes nothing.  A
  negative L counts as 0.

Every function here is fp64 NumPy; matrix products and exp/log are library
primitives.  No blocking, fusion or reordering beyond what the definition and
the split/combine steps above state.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

D_LATENT = 512
D_ROPE = 64
SPLIT_BLOCK_ROWS = 64


# ---------------------------------------------------------------------------
# Storage decoding (fp16 / bf16 bit patterns -> exact float64)
# ---------------------------------------------------------------------------

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of fp16 (numpy float16), bf16 (uint16 bits) or
    fp8 (uint8 bytes, OCP E4M3) storage."""
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_to_f64(a)
    raise ValueError(dtype)


def e4m3_to_f64(a: np.ndarray) -> np.ndarray:
    """OCP 8-bit E4M3 bytes to exact float64: sign bit 7, exponent bits 6..3
    (bias 7), mantissa bits 2..0.  Exponent 0 is subnormal, (m / 8) * 2^-6;
    otherwise (1 + m / 8) * 2^(e - 7).  Exponent 15 with mantissa 7 is NaN
    (0x7F, 0xFF); the format has no infinities, so the largest finite
    magnitude is 1.75 * 2^8 = 448.  The FP8 cache the TileLang guide lists
    among its variant kernels ("变体内核") gives no format; this is the
    reading this library takes (one fp32 scale per cache tensor)."""
    b = np.asarray(a, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (b & 0x7 == 7), np.nan, mag)
    return sign * mag


# ---------------------------------------------------------------------------
# Cache row gathering
# ---------------------------------------------------------------------------

def cache_rows(b: int, L: int, dtype: str, *, kv_latent=None, k_pe=None, pool=None,
               block_table=None, page_block_size: int = 0, kv_scale: float = 1.0) -> np.ndarray:
    """Rows 0..L-1 of sequence b as float64 ``[L, 576]`` (latent then RoPE).
    ``dtype`` is the cache's storage; an fp8 cache's values are the decoded
    bytes times ``kv_scale``."""
    if L == 0:
        return np.zeros((0, D_LATENT + D_ROPE))
    if pool is None:
        lat = to_f64(kv_latent[b, :L, 0, :], dtype)
        pe = to_f64(k_pe[b, :L, 0, :], dtype)
        rows = np.concatenate([lat, pe], axis=1)
    else:
        j = np.arange(L)
        pages = np.asarray(block_table)[b, j // page_block_size]
        if pages.min() < 0 or pages.max() >= pool.shape[0]:
            raise IndexError("block_table references a page outside the pool")
        rows = to_f64(pool[pages, j % page_block_size, 0, :], dtype)
    return rows * kv_scale if dtype == "fp8" else rows


# ---------------------------------------------------------------------------
# Attention over one set of rows
# ---------------------------------------------------------------------------

def scores(qn: np.ndarray, qp: np.ndarray, K: np.ndarray, softmax_scale: float) -> np.ndarray:
    """z[h, j] = scale * (q_nope[h]·latent_j + q_pe[h]·rope_j), shape [H, L]."""
    return softmax_scale * (qn @ K[:, :D_LATENT].T + qp @ K[:, D_LATENT:].T)


def softmax_stats(z: np.ndarray) -> np.ndarray:
    """Natural-log LSE per row of z ([H, L]); -inf for an empty row set."""
    H, L = z.shape
    if L == 0:
        return np.full(H, -np.inf)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def weighted_values(z: np.ndarray, lse: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Σ_j exp(z[h, j] - lse[h]) V_j, shape [H, 512]; zero for an empty row set."""
    if z.shape[1] == 0:
        return np.zeros((z.shape[0], D_LATENT))
    return np.exp(z - lse[:, None]) @ V


def attend(qn: np.ndarray, qp: np.ndarray, K: np.ndarray, softmax_scale: float):
    """(out [H, 512], lse [H]) of one query block over rows K ([L, 576])."""
    z = scores(qn, qp, K, softmax_scale)
    lse = softmax_stats(z)
    return weighted_values(z, lse, K[:, :D_LATENT]), lse


# ---------------------------------------------------------------------------
# Whole-batch direct definition
# ---------------------------------------------------------------------------

def _layout_kwargs(inp) -> dict:
    kw = dict(kv_scale=float(getattr(inp, "kv_scale", 1.0)))
    if inp.pool is not None:
        kw.update(pool=inp.pool, block_table=inp.block_table, page_block_size=inp.page_block_size)
    else:
        kw.update(kv_latent=inp.kv_latent, k_pe=inp.k_pe)
    return kw


def _cache_dtype(inp) -> str:
    return getattr(inp, "kv_dtype", "") or inp.dtype


def visible_rows(L: int, seqlen_q: int, t: int) -> int:
    """Cache rows that query token t of seqlen_q sees in a sequence of L rows:
    rows j < L - (seqlen_q - 1 - t), none when that is below 1."""
    return max(0, max(int(L), 0) - (seqlen_q - 1 - t))


def mla_decode_ref(inp, batches: Optional[Sequence[int]] = None,
                   heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Direct fp64 MLA decode of an ``MlaInputs``-like object.

    Returns ``out [nb, nh, 512]`` and ``lse [nb, nh]`` for the selected
    sequences (default all) and query rows (default all), in that order.  Query
    row v belongs to token v // heads_per_token (``inp.seqlen_q`` tokens,
    default 1), which sees the rows given by ``visible_rows``.
    """
    sq = int(getattr(inp, "seqlen_q", 1))
    hpt = inp.heads // sq
    bsel = list(range(inp.batch)) if batches is None else list(batches)
    hsel = np.arange(inp.heads) if heads is None else np.asarray(list(heads))
    out = np.zeros((len(bsel), len(hsel), D_LATENT))
    lse = np.zeros((len(bsel), len(hsel)))
    kw = _layout_kwargs(inp)
    for i, b in enumerate(bsel):
        L = max(int(inp.cache_seqlens[b]), 0)
        K = cache_rows(b, L, _cache_dtype(inp), **kw)
        for t in range(sq):
            idx = np.nonzero(hsel // hpt == t)[0]
            if idx.size == 0:
                continue
            rows = hsel[idx]
            qn = to_f64(inp.q_nope[b][rows], inp.dtype)
            qp = to_f64(inp.q_pe[b][rows], inp.dtype)
            out[i, idx], lse[i, idx] = attend(qn, qp, K[:visible_rows(L, sq, t)], inp.softmax_scale)
    return out, lse


# ---------------------------------------------------------------------------
# Split-KV partials and the LSE combine
# ---------------------------------------------------------------------------

def split_ranges(L: int, s: int, block_rows: int = SPLIT_BLOCK_ROWS) -> List[Tuple[int, int]]:
    """Row ranges of the s splits of a length-L sequence (block-granular, in order).

    nb = ceil(L / block_rows) blocks; split k gets floor(nb / s) blocks plus one
    when k < nb mod s.  Ranges are clipped to L; surplus splits are empty.
    """
    if s < 1:
        raise ValueError("s must be >= 1")
    nb = -(-L // block_rows)
    per, rem = divmod(nb, s)
    out, blk = [], 0
    for k in range(s):
        n = per + (1 if k < rem else 0)
        r0 = min(blk * block_rows, L)
        r1 = min((blk + n) * block_rows, L)
        out.append((r0, r1))
        blk += n
    return out


def split_partial(qn, qp, K, softmax_scale):
    """(O_k [H, 512] normalised, lse2_k [H]) of one split; lse2 in base 2."""
    o, lse = attend(qn, qp, K, softmax_scale)
    return o, lse / math.log(2.0)


def combine(partials: Sequence[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Merge (O_k, lse2_k) partials; returns (out, natural-log lse).

    Anchor M = max_k lse2_k over non-empty splits; Λ = log2 Σ_k 2^(lse2_k - M) + M;
    out = Σ_k 2^(lse2_k - Λ) O_k.  All-empty gives (0, -inf).
    """
    lses = np.stack([p[1] for p in partials])       # [s, H]
    outs = np.stack([p[0] for p in partials])       # [s, H, 512]
    M = lses.max(axis=0)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    with np.errstate(invalid="ignore"):
        total = np.log2(np.exp2(lses - Ms).sum(axis=0)) + Ms
        w = np.exp2(lses - total)                   # [s, H]
    w = np.where(np.isneginf(lses), 0.0, w)
    out = (w[:, :, None] * outs).sum(axis=0)
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, total * math.log(2.0))
    return out, lse


def mla_decode_split_ref(inp, splits, batches: Optional[Sequence[int]] = None,
                         heads: Optional[Sequence[int]] = None, block_rows: int = SPLIT_BLOCK_ROWS):
    """Split-KV form: per-range partials then the LSE combine.

    ``splits`` is one int (same count for every sequence) or a per-sequence list.
    """
    bsel = list(range(inp.batch)) if batches is None else list(batches)
    hsel = np.arange(inp.heads) if heads is None else np.asarray(list(heads))
    out = np.zeros((len(bsel), len(hsel), D_LATENT))
    lse = np.zeros((len(bsel), len(hsel)))
    kw = _layout_kwargs(inp)
    sq = int(getattr(inp, "seqlen_q", 1))
    hpt = inp.heads // sq
    for i, b in enumerate(bsel):
        s = splits if np.isscalar(splits) else splits[b]
        L = max(int(inp.cache_seqlens[b]), 0)
        K = cache_rows(b, L, _cache_dtype(inp), **kw)
        for t in range(sq):
            idx = np.nonzero(hsel // hpt == t)[0]
            if idx.size == 0:
                continue
            rows = hsel[idx]
            qn = to_f64(inp.q_nope[b][rows], inp.dtype)
            qp = to_f64(inp.q_pe[b][rows], inp.dtype)
            Lt = visible_rows(L, sq, t)
            parts = [split_partial(qn, qp, K[r0:max(r0, min(r1, Lt))], inp.softmax_scale)
                     for r0, r1 in split_ranges(L, int(s), block_rows)]
            out[i, idx], lse[i, idx] = combine(parts)
    return out, lse

