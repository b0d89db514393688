"""MI355X (gfx950) DeepSeek MLA decode.

Thin Python binding over the C ABI of ``libmla_decode.so``: it reads shapes and
strides off PyTorch tensors, allocates outputs and workspace with PyTorch, and
passes raw device pointers and the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

from . import _lib
from ._lib import (  # noqa: F401
    D_LATENT,
    D_ROPE,
    MAX_SPLITS,
    NOALLOC_SCRATCH_BYTES,
    MLA_DTYPE_BF16,
    MLA_DTYPE_F16,
    MLA_KV_AS_DTYPE,
    MLA_KV_FP8_E4M3,
    SPLIT_BLOCK_ROWS,
    MlaDesc,
    MlaError,
)

__all__ = [
    "mla_decode", "mla_decode_noalloc", "mla_decode_planned", "mla_plan_host", "mla_plan_device", "mla_workspace_size", "mla_max_work",
    "mla_num_cus", "mla_last_error", "mla_timing_enable", "mla_timing_read", "make_desc",
    "mla_check_block_table",
    "MlaDesc", "MlaError",
]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return MLA_DTYPE_F16
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float16 or bfloat16")


def _is_fp8_cache(t) -> bool:
    """E4M3 cache bytes: a uint8 tensor, or PyTorch's float8_e4m3fn (the same
    OCP E4M3 format)."""
    torch = _torch()
    return t.dtype == torch.uint8 or t.dtype == getattr(torch, "float8_e4m3fn", None)


def _as4(t, last: int, name: str):
    """View a cache tensor as [N, rows, 1, last] (accepts [N, rows, last] too)."""
    if t.dim() == 3:
        t = t.unsqueeze(2)
    if t.dim() != 4 or t.shape[2] != 1 or t.shape[3] != last:
        raise ValueError(f"{name} must be [N, rows, 1, {last}] (one KV head), got {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise ValueError(f"{name} last dimension must be contiguous")
    return t


def mla_last_error() -> str:
    return _lib.lib().mla_last_error().decode(errors="replace")


def mla_num_cus(device: Optional[int] = None) -> int:
    torch = _torch()
    dev = torch.cuda.current_device() if device is None else int(device)
    n = ctypes.c_int32()
    _lib.check(_lib.lib().mla_num_cus(dev, ctypes.byref(n)))
    return n.value


def make_desc(q_nope, q_pe, kv_latent, k_pe, block_table, out, seqlen_q: int = 1,
              kv_scale: Optional[float] = None) -> MlaDesc:
    """Fill an ``MlaDesc`` from tensors (strides in elements).  With
    ``seqlen_q`` > 1 the H query rows are seqlen_q tokens x H / seqlen_q heads,
    token-major.  An FP8 cache (``uint8`` or ``float8_e4m3fn`` E4M3 bytes)
    stands for decode(byte) * ``kv_scale`` (default 1); a 16-bit cache takes
    no scale."""
    if q_nope.dim() != 3 or q_nope.shape[2] != D_LATENT or q_nope.stride(2) != 1:
        raise ValueError(f"q_nope must be [B, H, 512] with contiguous last dim, got {tuple(q_nope.shape)}")
    B, H = q_nope.shape[0], q_nope.shape[1]
    if tuple(q_pe.shape) != (B, H, D_ROPE) or q_pe.stride(2) != 1:
        raise ValueError(f"q_pe must be [B, H, 64], got {tuple(q_pe.shape)}")
    if tuple(out.shape) != (B, H, D_LATENT) or out.stride(2) != 1:
        raise ValueError(f"out must be [B, H, 512], got {tuple(out.shape)}")
    kv = _as4(kv_latent, D_LATENT, "kv_latent")
    kp = _as4(k_pe, D_ROPE, "k_pe")
    if kv.shape[:2] != kp.shape[:2]:
        raise ValueError("kv_latent and k_pe disagree on [N, rows]")
    d = MlaDesc()
    d.batch, d.heads = B, H
    d.seqlen_q = int(seqlen_q)
    d.d_latent, d.d_rope = D_LATENT, D_ROPE
    d.dtype = _dtype_code(q_nope)
    fp8 = _is_fp8_cache(kv)
    if fp8 != _is_fp8_cache(kp):
        raise TypeError(f"kv_latent ({kv.dtype}) and k_pe ({kp.dtype}) must share one storage type")
    cache = () if fp8 else ((kv, "kv_latent"), (kp, "k_pe"))
    for t, nm in ((q_pe, "q_pe"), (out, "out"), *cache):
        if t.dtype != q_nope.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} differs from q_nope dtype {q_nope.dtype}")
    if fp8:
        d.kv_dtype = MLA_KV_FP8_E4M3
        d.kv_scale = 1.0 if kv_scale is None else float(kv_scale)
    elif kv_scale is not None and float(kv_scale) != 1.0:
        raise ValueError("kv_scale applies to an FP8 cache only")
    if block_table is None:
        if kv.shape[0] != B:
            raise ValueError("contiguous cache must have batch as its first dimension")
        d.max_seqlen = kv.shape[1]
    else:
        d.page_block_size = kv.shape[1]
        d.block_table_stride = block_table.stride(0)
        d.num_pages = kv.shape[0]
    d.q_nope_sb, d.q_nope_sh = q_nope.stride(0), q_nope.stride(1)
    d.q_pe_sb, d.q_pe_sh = q_pe.stride(0), q_pe.stride(1)
    d.kv_sb, d.kv_sr = kv.stride(0), kv.stride(1)
    d.kpe_sb, d.kpe_sr = kp.stride(0), kp.stride(1)
    d.out_sb, d.out_sh = out.stride(0), out.stride(1)
    return d


def mla_max_work(desc: MlaDesc, num_split: int, num_cus: int) -> int:
    n = ctypes.c_int32()
    _lib.check(_lib.lib().mla_max_work(ctypes.byref(desc), int(num_split), int(num_cus), ctypes.byref(n)))
    return n.value


def mla_workspace_size(desc: MlaDesc, num_split: int, num_cus: int) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.lib().mla_workspace_size(ctypes.byref(desc), int(num_split), int(num_cus), ctypes.byref(n)))
    return n.value


_workspaces = {}


def _workspace(device, stream_id: int, nbytes: int):
    torch = _torch()
    key = (device, stream_id)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def mla_decode_noalloc(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale: float,
                       num_split: int = 0, out=None, lse=None, stream=None,
                       kv_scale: Optional[float] = None) -> Tuple["object", "object"]:
    """``mla_decode`` through the C ABI's no-allocation entry point: the
    library's static per-GPU scratch array replaces the workspace (at most
    ``NOALLOC_SCRATCH_BYTES``; calls that overlap on one GPU race).  Pass
    ``out`` and ``lse`` to keep the call free of allocations."""
    return mla_decode(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale, num_split, out,
                      lse, stream=stream, kv_scale=kv_scale, _noalloc=True)


def mla_decode_planned(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale: float, plan,
                       num_split: int = 0, num_cus: Optional[int] = None, out=None, lse=None, workspace=None,
                       stream=None, kv_scale: Optional[float] = None) -> Tuple["object", "object"]:
    """mla_decode with a plan made beforehand: ``plan`` is the ``(num_splits,
    split_offset, work)`` that ``mla_plan_device(cache_seqlens, heads,
    num_split, num_cus, seqlen_q=...)`` returned for these lengths; pass the
    same ``num_split`` and ``num_cus`` (default: this GPU's CU count), which
    size the workspace.  One plan serves every layer of a decode step; the
    kernels read the plan and clamp what they read, so a plan made for other
    lengths gives wrong results, not faults."""
    return mla_decode(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale, num_split, out,
                      lse, workspace, stream, kv_scale, _plan=(plan, num_cus))


def mla_decode(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale: float,
               num_split: int = 0, out=None, lse=None, workspace=None,
               stream=None, kv_scale: Optional[float] = None, _noalloc: bool = False,
               _plan=None) -> Tuple["object", "object"]:
    """MLA decode through the C ABI; returns ``(out [B,H,512], lse fp32 [B,H])``.

    Contiguous cache: ``kv_latent [B, S, 1, 512]``, ``k_pe [B, S, 1, 64]``,
    ``block_table=None``.  Paged cache: ``kv_latent`` / ``k_pe`` are views of a
    pool ``[P, page, 1, 576]`` (``pool[..., :512]`` and ``pool[..., 512:]``)
    and ``block_table`` is int32 ``[B, max_blocks]``.  ``num_split=0`` lets the
    planner choose the splits.  Work is enqueued on ``stream`` (default: the
    current stream) and nothing synchronises.

    FP8 cache: ``kv_latent`` / ``k_pe`` hold OCP E4M3 bytes (``uint8`` or
    ``float8_e4m3fn``), standing for decode(byte) * ``kv_scale``; queries and
    output stay float16 / bfloat16.

    Several query tokens per sequence: ``q_nope [B, s, H, 512]`` and ``q_pe
    [B, s, H, 64]`` (the s new tokens are the last s cache rows; token t sees
    rows j < L - (s - 1 - t)); then ``out`` is ``[B, s, H, 512]`` and ``lse``
    ``[B, s, H]``.
    """
    torch = _torch()
    if not q_nope.is_cuda:
        raise ValueError("tensors must live on the GPU")
    _check_placement(q_nope, dict(q_pe=q_pe, kv_latent=kv_latent, k_pe=k_pe, block_table=block_table,
                                  cache_seqlens=cache_seqlens, out=out, lse=lse, workspace=workspace))
    seqlen_q, four_d = 1, q_nope.dim() == 4
    if four_d:
        B, seqlen_q, Hq = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
        if q_pe.dim() != 4 or tuple(q_pe.shape[:3]) != (B, seqlen_q, Hq):
            raise ValueError("q_pe must be [B, s, H, 64] like q_nope")
        if out is None:
            out = torch.empty((B, seqlen_q, Hq, D_LATENT), dtype=q_nope.dtype, device=q_nope.device)
        if lse is None:
            lse = torch.empty((B, seqlen_q, Hq), dtype=torch.float32, device=q_nope.device)
        out4, lse4 = out, lse
        # Query rows token-major: views only (the kernel writes through out/lse).
        q_nope, q_pe, out, lse = (_rows_view(q_nope, "q_nope"), _rows_view(q_pe, "q_pe"), _rows_view(out, "out"),
                                  _rows_view(lse, "lse"))
    B, H = q_nope.shape[0], q_nope.shape[1]
    if out is None:
        out = torch.empty((B, H, D_LATENT), dtype=q_nope.dtype, device=q_nope.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H):
        raise ValueError("lse must be a contiguous float32 [B, H] tensor")
    _check_batch_arrays(B, cache_seqlens, block_table)
    desc = make_desc(q_nope, q_pe, kv_latent, k_pe, block_table, out, seqlen_q, kv_scale)
    s = torch.cuda.current_stream(q_nope.device) if stream is None else stream
    kv = _as4(kv_latent, D_LATENT, "kv_latent")
    kp = _as4(k_pe, D_ROPE, "k_pe")
    bt = None if block_table is None else block_table.data_ptr()
    if _noalloc:
        st = _lib.lib().mla_decode_noalloc(
            q_nope.data_ptr(), q_pe.data_ptr(), kv.data_ptr(), kp.data_ptr(), bt, cache_seqlens.data_ptr(),
            float(softmax_scale), int(num_split), out.data_ptr(), lse.data_ptr(), ctypes.byref(desc), s.cuda_stream)
        _lib.check(st)
        return (out4, lse4) if four_d else (out, lse)
    plan = None
    if _plan is not None:
        plan, cus = _plan
        num_cus = mla_num_cus(q_nope.device.index) if cus is None else int(cus)
        ns, off, work = _check_plan(plan, B, q_nope)
    else:
        num_cus = mla_num_cus(q_nope.device.index)
    if workspace is None:
        need = mla_workspace_size(desc, num_split, num_cus)
        workspace = _workspace(q_nope.device, s.cuda_stream, need)
    elif not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    if plan is not None:
        st = _lib.lib().mla_decode_planned(
            q_nope.data_ptr(), q_pe.data_ptr(), kv.data_ptr(), kp.data_ptr(), bt, cache_seqlens.data_ptr(),
            float(softmax_scale), ns.data_ptr(), off.data_ptr(), work.data_ptr(), int(work.shape[0]),
            out.data_ptr(), lse.data_ptr(), ctypes.byref(desc), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), s.cuda_stream)
        _lib.check(st)
        return (out4, lse4) if four_d else (out, lse)
    st = _lib.lib().mla_decode(
        q_nope.data_ptr(), q_pe.data_ptr(), kv.data_ptr(), kp.data_ptr(), bt, cache_seqlens.data_ptr(),
        float(softmax_scale), int(num_split), out.data_ptr(), lse.data_ptr(), ctypes.byref(desc),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), s.cuda_stream)
    _lib.check(st)
    if four_d:
        return out4, lse4
    return out, lse


def _check_placement(q_nope, tensors) -> None:
    """Every tensor argument must live on q_nope's GPU: the C ABI takes raw
    device addresses, so a host tensor's pointer would reach the kernels as a
    host address (a GPU memory fault), and another GPU's as a foreign one."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != q_nope.device:
            raise ValueError(f"{name} is on {t.device}; every tensor must be on q_nope's device {q_nope.device}")


def _check_plan(plan, batch: int, q_nope):
    """(num_splits [B], split_offset [B + 1], work [max_work, 4]): contiguous
    int32 tensors on q_nope's GPU, as mla_plan_device returns them."""
    import torch
    try:
        ns, off, work = plan
    except (TypeError, ValueError):
        raise ValueError("plan must be the (num_splits, split_offset, work) of mla_plan_device") from None
    _check_placement(q_nope, dict(num_splits=ns, split_offset=off, work=work))
    for name, t, shape in (("num_splits", ns, (batch,)), ("split_offset", off, (batch + 1,))):
        if t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError(f"plan {name} must be a contiguous int32 tensor of shape {shape}")
    if work.dtype != torch.int32 or not work.is_contiguous() or work.dim() != 2 or work.shape[1] != 4 \
            or work.shape[0] < 1:
        raise ValueError("plan work must be a contiguous int32 tensor [max_work, 4]")
    return ns, off, work


def _check_batch_arrays(batch: int, cache_seqlens, block_table) -> None:
    """cache_seqlens: contiguous int32 with exactly `batch` entries; block_table
    (paged): int32 [rows >= batch, max_blocks] with contiguous rows.  The
    kernels read cache_seqlens[0..B) and block_table rows 0..B-1, so shorter
    arrays would be read past their end."""
    import torch
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_contiguous():
        raise ValueError("cache_seqlens must be a contiguous int32 tensor")
    if cache_seqlens.dim() != 1 or cache_seqlens.shape[0] != batch:
        raise ValueError(f"cache_seqlens must have shape [{batch}], got {tuple(cache_seqlens.shape)}")
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise ValueError("block_table must be a 2-D int32 tensor with contiguous rows")
        if block_table.shape[0] < batch:
            raise ValueError(f"block_table has {block_table.shape[0]} rows for a batch of {batch}")


def _rows_view(t, name):
    """[B, s, H, ...] -> [B, s*H, ...] as a view (token-major query rows)."""
    if t.stride(1) != t.shape[2] * t.stride(2):
        raise ValueError(f"{name}: the token and head dimensions must be mergeable into one (token-major rows)")
    return t.view(t.shape[0], t.shape[1] * t.shape[2], *t.shape[3:])


def _plan_capacity(batch: int, heads: int, num_split: int, num_cus: int, seqlen_q: int) -> int:
    """Split entries a plan can need (the library's own count, via mla_max_work)."""
    d = MlaDesc()
    d.batch, d.heads, d.d_latent, d.d_rope, d.dtype, d.seqlen_q = int(batch), int(heads), 512, 64, 0, int(seqlen_q)
    return mla_max_work(d, num_split, num_cus)


def mla_plan_host(cache_seqlens, heads: int, num_split: int, num_cus: int, seqlen_q: int = 1):
    """Host twin of the planner.  Returns (num_splits [B], split_offset [B+1], work [W, 4]) as numpy.
    ``heads`` counts query rows (seqlen_q x heads per token)."""
    import numpy as np
    lens = np.ascontiguousarray(cache_seqlens, dtype=np.int32)
    B = lens.shape[0]
    max_work = _plan_capacity(B, heads, num_split, num_cus, seqlen_q)
    ns = np.zeros(B, np.int32)
    off = np.zeros(B + 1, np.int32)
    work = np.zeros((max(max_work, 1), 4), np.int32)
    _lib.check(_lib.lib().mla_plan_host(
        lens.ctypes.data, B, int(heads), int(seqlen_q), int(num_split), int(num_cus), ns.ctypes.data,
        off.ctypes.data, work.ctypes.data, int(max_work)))
    return ns, off, work[:off[B]]


def mla_plan_device(cache_seqlens, heads: int, num_split: int, num_cus: int, stream=None, seqlen_q: int = 1):
    """Device planner; returns (num_splits, split_offset, work) as torch tensors on the GPU."""
    torch = _torch()
    B = cache_seqlens.shape[0]
    max_work = _plan_capacity(B, heads, num_split, num_cus, seqlen_q)
    dev = cache_seqlens.device
    ns = torch.zeros(B, dtype=torch.int32, device=dev)
    off = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    work = torch.zeros((max(max_work, 1), 4), dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    _lib.check(_lib.lib().mla_plan_device(
        cache_seqlens.data_ptr(), B, int(heads), int(seqlen_q), int(num_split), int(num_cus), ns.data_ptr(),
        off.data_ptr(), work.data_ptr(), int(max_work), s.cuda_stream))
    return ns, off, work


def mla_check_block_table(block_table, cache_seqlens, num_pages: int, page_block_size: int, stream=None):
    """Entries of a paged cache's block table that mla_decode reads (j <
    ceil(L_b / page_block_size)) and that lie outside [0, num_pages), per
    sequence: an int32 tensor [B] on the GPU.  mla_decode itself clamps such
    entries into the pool (valid memory, wrong rows); this makes them
    visible.  Enqueued on ``stream``; nothing synchronises."""
    torch = _torch()
    if not block_table.is_cuda:
        raise ValueError("block_table must live on the GPU")
    _check_placement(block_table, dict(cache_seqlens=cache_seqlens))
    B = cache_seqlens.shape[0] if cache_seqlens.dim() == 1 else -1
    _check_batch_arrays(B, cache_seqlens, block_table)
    d = MlaDesc()
    d.batch = B
    d.page_block_size = int(page_block_size)
    d.block_table_stride = block_table.stride(0)
    d.num_pages = int(num_pages)
    bad = torch.empty(max(B, 1), dtype=torch.int32, device=block_table.device)[:B]
    s = torch.cuda.current_stream(block_table.device) if stream is None else stream
    _lib.check(_lib.lib().mla_check_block_table(block_table.data_ptr(), cache_seqlens.data_ptr(), ctypes.byref(d),
                                                bad.data_ptr(), s.cuda_stream))
    return bad


def mla_timing_enable(enable: bool = True) -> None:
    _lib.check(_lib.lib().mla_timing_enable(1 if enable else 0))


def mla_timing_read():
    """(split_ms, combine_ms, calls) summed since the last read."""
    a, c = ctypes.c_float(), ctypes.c_float()
    n = ctypes.c_int32()
    _lib.check(_lib.lib().mla_timing_read(ctypes.byref(a), ctypes.byref(c), ctypes.byref(n)))
    return a.value, c.value, n.value
