"""Seeded synthetic inputs for MLA decode.

This module is shared by the CPU oracle side (tests, baseline timing) and the
GPU side (tests, bench).  It only *makes* inputs: it holds no part of the
attention arithmetic.  Every array is produced on the host from a NumPy
``default_rng`` seed, so both sides see bit-identical values.

Storage conventions
-------------------
* ``f16`` arrays are ``numpy.float16``.
* ``bf16`` arrays are ``numpy.uint16`` holding bfloat16 bit patterns (NumPy has
  no bfloat16); the fp32 -> bf16 cast is round-to-nearest-even.
* Contiguous caches are ``kv_latent [B, S, 1, 512]`` and ``k_pe [B, S, 1, 64]``.
* Paged caches are one pool ``[P, page, 1, 576]`` (latent 512 followed by RoPE
  64 in each row) plus ``block_table int32 [B, max_blocks]``; entries past a
  sequence's last page are -1.

Value distribution: i.i.d. N(0, 1) drawn in fp32 and cast, as in the random
normal supply the TileLang MLA guide uses for its correctness check
("参考实现与正确性验证" section).
"""
from __future__ import annotations

import concurrent.futures as _fut
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE

# Rows per generator chunk: each chunk gets its own child seed so the large
# caches can be filled by several threads and still be reproducible.
_CHUNK_ROWS = 4096


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest-even) and return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def cast_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp32 values to the storage format named by ``dtype``."""
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_np_dtype(dtype: str):
    return {"f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}[dtype]


# FP8 cache: OCP E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
# bits; no infinities; 0x7F / 0xFF are NaN; largest finite 448), one fp32
# scale per cache tensor: a stored byte stands for decode(byte) * kv_scale.
E4M3_MAX = 448.0
DEFAULT_KV_SCALE = 0.0125   # N(0,1) values up to about 5.6 land below 448 / scale


def _e4m3_magnitudes() -> np.ndarray:
    """Magnitudes of the finite non-negative E4M3 codes 0x00..0x7E, ascending."""
    out = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        out[code] = np.ldexp(m, -9) if e == 0 else np.ldexp(8 + m, e - 10)
    return out


def f32_to_e4m3_bits(x: np.ndarray, kv_scale: float) -> np.ndarray:
    """Quantise x / kv_scale to E4M3 bytes: round to nearest, ties to an even
    code, magnitudes beyond 448 saturate to 448 (input generation only)."""
    a = np.abs(np.asarray(x, dtype=np.float64) / kv_scale)
    mags = _e4m3_magnitudes()
    hi = np.clip(np.searchsorted(mags, a), 1, 126)
    lo = hi - 1
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= mags[126], 126, code).astype(np.uint8)
    sign = (np.signbit(np.asarray(x, dtype=np.float64))).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def _normal_rows(seed_seq: np.random.SeedSequence, n_rows: int, width: int, dtype: str,
                 kv_scale: Optional[float] = None) -> np.ndarray:
    """``n_rows x width`` N(0,1) values in storage format, filled chunk-wise in
    parallel.  ``dtype="fp8"``: the values drawn as for fp16, then quantised
    to E4M3 bytes of value / kv_scale."""
    out = np.empty((n_rows, width), dtype=storage_np_dtype(dtype))
    n_chunks = (n_rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    children = seed_seq.spawn(n_chunks)

    def fill(i: int) -> None:
        r0 = i * _CHUNK_ROWS
        r1 = min(n_rows, r0 + _CHUNK_ROWS)
        g = np.random.default_rng(children[i])
        x = g.standard_normal((r1 - r0, width), dtype=np.float32)
        if dtype == "fp8":
            out[r0:r1] = f32_to_e4m3_bits(cast_storage(x, "f16").astype(np.float32), kv_scale)
        else:
            out[r0:r1] = cast_storage(x, dtype)

    if n_chunks <= 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with _fut.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


@dataclass
class MlaInputs:
    """One MLA decode problem: queries, KV cache (contiguous or paged), lengths."""

    dtype: str
    q_nope: np.ndarray            # [B, H, 512] (H = seqlen_q x heads per token, token-major)
    q_pe: np.ndarray              # [B, H, 64]
    cache_seqlens: np.ndarray     # int32 [B]
    softmax_scale: float
    kv_latent: Optional[np.ndarray] = None   # contiguous: [B, S, 1, 512]
    k_pe: Optional[np.ndarray] = None        # contiguous: [B, S, 1, 64]
    pool: Optional[np.ndarray] = None        # paged: [P, page, 1, 576]
    block_table: Optional[np.ndarray] = None  # paged: int32 [B, max_blocks]
    page_block_size: int = 0
    seqlen_q: int = 1             # query tokens per sequence (rows of q are token-major)
    kv_dtype: str = ""            # cache storage: "" = as the queries, or "fp8" (E4M3 bytes)
    kv_scale: float = 1.0         # fp8 cache: value = decode(byte) * kv_scale
    meta: dict = field(default_factory=dict)

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def paged(self) -> bool:
        return self.pool is not None

    @property
    def batch(self) -> int:
        return self.q_nope.shape[0]

    @property
    def heads(self) -> int:
        """Query rows per sequence: seqlen_q x heads_per_token."""
        return self.q_nope.shape[1]

    @property
    def heads_per_token(self) -> int:
        return self.q_nope.shape[1] // self.seqlen_q


def default_scale() -> float:
    """softmax_scale = 1/sqrt(576): the QK head dim of MLA."""
    return 1.0 / float(np.sqrt(D_QK))


def make_queries(ss: np.random.SeedSequence, batch: int, heads: int, dtype: str):
    q = _normal_rows(ss, batch * heads, D_QK, dtype).reshape(batch, heads, D_QK)
    return np.ascontiguousarray(q[:, :, :D_LATENT]), np.ascontiguousarray(q[:, :, D_LATENT:])


def _cache_rows(seed_seq, n_rows: int, dtype: str, kv_dtype: str, kv_scale: float) -> np.ndarray:
    """N(0,1) cache rows in the storage format: 16-bit as the queries, or E4M3
    bytes of value / kv_scale."""
    if kv_dtype != "fp8":
        return _normal_rows(seed_seq, n_rows, D_QK, dtype)
    return _normal_rows(seed_seq, n_rows, D_QK, "fp8", kv_scale)


def _kv_args(kv_dtype, kv_scale):
    kv_dtype = kv_dtype or ""
    if kv_dtype not in ("", "fp8"):
        raise ValueError(f"unknown cache dtype {kv_dtype!r}")
    if kv_dtype == "fp8":
        return kv_dtype, float(DEFAULT_KV_SCALE if kv_scale is None else kv_scale)
    return kv_dtype, 1.0


def make_contiguous(batch: int, heads: int, max_seqlen: int, cache_seqlens, dtype: str = "f16",
                    seed: int = 0, scale: Optional[float] = None, seqlen_q: int = 1,
                    kv_dtype: Optional[str] = None, kv_scale: Optional[float] = None) -> MlaInputs:
    """Contiguous cache ``[B, S, 1, 512] + [B, S, 1, 64]``, all rows N(0,1).

    With ``seqlen_q`` > 1 each sequence has that many query tokens of ``heads``
    heads each, stored as ``seqlen_q * heads`` query rows, token-major.
    ``kv_dtype="fp8"`` stores the cache as E4M3 bytes of value / kv_scale
    (the rows drawn as for fp16, then quantised)."""
    kv_dtype, kv_scale = _kv_args(kv_dtype, kv_scale)
    lens = np.asarray(cache_seqlens, dtype=np.int32).reshape(batch)
    if lens.size and (lens.min() < 0 or lens.max() > max_seqlen):
        raise ValueError("cache_seqlens must lie in [0, max_seqlen]")
    root = np.random.SeedSequence(seed)
    sq, skv = root.spawn(2)
    q_nope, q_pe = make_queries(sq, batch, heads * seqlen_q, dtype)
    rows = _cache_rows(skv, batch * max_seqlen, dtype, kv_dtype, kv_scale).reshape(batch, max_seqlen, 1, D_QK)
    return MlaInputs(
        dtype=dtype, q_nope=q_nope, q_pe=q_pe, cache_seqlens=lens,
        softmax_scale=default_scale() if scale is None else float(scale),
        kv_latent=np.ascontiguousarray(rows[..., :D_LATENT]),
        k_pe=np.ascontiguousarray(rows[..., D_LATENT:]), seqlen_q=seqlen_q,
        kv_dtype=kv_dtype, kv_scale=kv_scale,
        meta={"layout": "contiguous", "seed": seed, "max_seqlen": max_seqlen},
    )


def make_paged(batch: int, heads: int, cache_seqlens, dtype: str = "bf16", seed: int = 0,
               page_block_size: int = 64, max_blocks: Optional[int] = None, shuffle: bool = True,
               spare_pages: int = 0, scale: Optional[float] = None, seqlen_q: int = 1,
               kv_dtype: Optional[str] = None, kv_scale: Optional[float] = None) -> MlaInputs:
    """Paged pool ``[P, page, 1, 576]`` with a block_table.

    Each sequence owns ``ceil(L_b / page)`` logical pages.  Physical pages are a
    random permutation of ``0..P-1`` (``shuffle``) handed to logical pages in
    order; unused block_table entries are -1.  ``spare_pages`` adds pool pages
    that no sequence references.  ``kv_dtype="fp8"``: E4M3 pool bytes (see
    make_contiguous).
    """
    kv_dtype, kv_scale = _kv_args(kv_dtype, kv_scale)
    lens = np.asarray(cache_seqlens, dtype=np.int32).reshape(batch)
    if lens.size and lens.min() < 0:
        raise ValueError("cache_seqlens must be >= 0")
    pages_per_seq = (lens.astype(np.int64) + page_block_size - 1) // page_block_size
    need = int(pages_per_seq.max()) if batch else 0
    if max_blocks is None:
        max_blocks = max(1, need)
    if need > max_blocks:
        raise ValueError("max_blocks too small for cache_seqlens")
    n_used = int(pages_per_seq.sum())
    n_pages = n_used + spare_pages
    root = np.random.SeedSequence(seed)
    sq, skv, sperm = root.spawn(3)
    q_nope, q_pe = make_queries(sq, batch, heads * seqlen_q, dtype)
    pool = _cache_rows(skv, max(n_pages, 1) * page_block_size, dtype, kv_dtype, kv_scale)
    pool = pool.reshape(max(n_pages, 1), page_block_size, 1, D_QK)
    perm = np.random.default_rng(sperm).permutation(n_pages) if shuffle else np.arange(n_pages)
    table = np.full((batch, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b in range(batch):
        k = int(pages_per_seq[b])
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return MlaInputs(
        dtype=dtype, q_nope=q_nope, q_pe=q_pe, cache_seqlens=lens,
        softmax_scale=default_scale() if scale is None else float(scale),
        pool=pool, block_table=table, page_block_size=page_block_size, seqlen_q=seqlen_q,
        kv_dtype=kv_dtype, kv_scale=kv_scale,
        meta={"layout": "paged", "seed": seed, "n_pages": n_pages},
    )


def scale_random_rows(inp: MlaInputs, fraction: float, factor: float, seed: int) -> np.ndarray:
    """Multiply ``round(fraction * L_b)`` distinct logical rows of each sequence by ``factor``.

    The whole 576-wide row (latent and RoPE) is scaled, so the V row scales too.
    With a power-of-two factor the result is exact in fp16/bf16 storage.
    Returns the chosen logical positions as an int array ``[B, k_max]`` (-1 padded).
    """
    if inp.cache_dtype == "fp8":
        raise ValueError("scale_random_rows works on 16-bit caches (an E4M3 row times 8 may saturate)")
    rng = np.random.default_rng(seed)
    chosen = []
    for b in range(inp.batch):
        L = int(inp.cache_seqlens[b])
        k = int(round(fraction * L))
        pos = np.sort(rng.choice(L, size=k, replace=False)) if k else np.zeros(0, np.int64)
        chosen.append(pos)
        for j in pos:
            if inp.paged:
                p = inp.block_table[b, j // inp.page_block_size]
                row = inp.pool[p, j % inp.page_block_size, 0]
                inp.pool[p, j % inp.page_block_size, 0] = _scaled(row, factor, inp.dtype)
            else:
                inp.kv_latent[b, j, 0] = _scaled(inp.kv_latent[b, j, 0], factor, inp.dtype)
                inp.k_pe[b, j, 0] = _scaled(inp.k_pe[b, j, 0], factor, inp.dtype)
    kmax = max((len(c) for c in chosen), default=0)
    out = np.full((inp.batch, kmax), -1, dtype=np.int64)
    for b, c in enumerate(chosen):
        out[b, :len(c)] = c
    return out


def _scaled(row: np.ndarray, factor: float, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return (row.astype(np.float32) * np.float32(factor)).astype(np.float16)
    f = (row.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return f32_to_bf16_bits(f)


# ---------------------------------------------------------------------------
# The five workloads used for parity and measurement.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    0: "tiny_b2_h16_l256_f16",
    1: "b64_h128_l4096_f16",
    2: "b128_h128_l8192_f16",
    3: "paged_b64_h128_lU1-16384_bf16",
    4: "stress_paged_b2_h128_l131072_bf16",
}


def make_config(idx: int, batch_subset: Optional[int] = None, seqlen_q: int = 1,
                heads: Optional[int] = None, kv_dtype: Optional[str] = None) -> MlaInputs:
    """Build workload ``idx`` (0..4).  ``batch_subset`` keeps only the first sequences;
    ``seqlen_q`` > 1 gives every sequence that many query tokens (of H heads each);
    ``heads`` replaces H (e.g. one tensor-parallel shard's heads); ``kv_dtype="fp8"``
    stores the same N(0,1) cache rows as E4M3 bytes with DEFAULT_KV_SCALE (configs
    0..3; the stress pattern's x8 rows would saturate E4M3), named with a
    ``_kvfp8`` suffix.

    0: B=2, H=16, L=256, fp16, contiguous.
    1: B=64, H=128, L=4096, fp16, contiguous.
    2: B=128, H=128, L=8192, fp16, contiguous.
    3: B=64, H=128, L_b ~ U{1..16384}, bf16, paged (64), shuffled block_table.
    4: B=2, H=128, L=131072, bf16, paged (64), shuffled, 1% of rows x8.
    """
    Hx = heads
    fp8 = kv_dtype == "fp8"
    if fp8 and idx == 4:
        raise ValueError("the stress workload scales rows x8, beyond what E4M3 at the default scale holds")
    suffix = "_kvfp8" if fp8 else ""
    if idx == 0:
        B, H, L, dt = 2, 16, 256, "f16"
    elif idx == 1:
        B, H, L, dt = 64, 128, 4096, "f16"
    elif idx == 2:
        B, H, L, dt = 128, 128, 8192, "f16"
    elif idx == 3:
        B, H = 64, Hx or 128
        lens = np.random.default_rng(np.random.SeedSequence([3, 1])).integers(1, 16384, size=B, endpoint=True)
        if batch_subset is not None:
            lens = lens[:batch_subset]
            B = batch_subset
        inp = make_paged(B, H, lens, "bf16", seed=3, page_block_size=64, max_blocks=256, seqlen_q=seqlen_q,
                         kv_dtype=kv_dtype)
        inp.meta["config"] = CONFIG_NAMES[3] + suffix
        return inp
    elif idx == 4:
        B, H, L = 2, Hx or 128, 131072
        if batch_subset is not None:
            B = batch_subset
        inp = make_paged(B, H, [L] * B, "bf16", seed=4, page_block_size=64, max_blocks=L // 64, seqlen_q=seqlen_q)
        inp.meta["scaled_rows"] = scale_random_rows(inp, 0.01, 8.0, seed=40)
        inp.meta["config"] = CONFIG_NAMES[4]
        return inp
    else:
        raise ValueError(idx)
    if batch_subset is not None:
        B = batch_subset
    H = Hx or H
    inp = make_contiguous(B, H, L, [L] * B, dt, seed=idx, seqlen_q=seqlen_q, kv_dtype=kv_dtype)
    inp.meta["config"] = CONFIG_NAMES[idx] + suffix
    return inp
