"""Move an ``MlaInputs`` problem to GPU tensors (storage bits copied exactly)."""
from __future__ import annotations

import numpy as np


def _t(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "fp8":   # E4M3 bytes, as uint8
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)
    raise ValueError(dtype)


def to_device(inp, device="cuda"):
    """Dict of device tensors: q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens (+ pool), and
    the cache's kv_scale (None for a 16-bit cache)."""
    import torch
    d = {
        "q_nope": _t(inp.q_nope, inp.dtype, device),
        "q_pe": _t(inp.q_pe, inp.dtype, device),
        "cache_seqlens": torch.from_numpy(np.ascontiguousarray(inp.cache_seqlens, dtype=np.int32)).to(device),
    }
    cdt = getattr(inp, "cache_dtype", inp.dtype)
    d["kv_scale"] = float(inp.kv_scale) if cdt == "fp8" else None
    if inp.paged:
        pool = _t(inp.pool, cdt, device)
        d["pool"] = pool
        d["kv_latent"] = pool[..., :512]
        d["k_pe"] = pool[..., 512:]
        d["block_table"] = torch.from_numpy(np.ascontiguousarray(inp.block_table, dtype=np.int32)).to(device)
    else:
        d["kv_latent"] = _t(inp.kv_latent, cdt, device)
        d["k_pe"] = _t(inp.k_pe, cdt, device)
        d["block_table"] = None
    return d


def from_device(t) -> np.ndarray:
    """Device tensor (fp16/bf16/fp32) -> float64 numpy."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
