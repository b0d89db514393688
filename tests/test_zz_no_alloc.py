"""The no-allocation entry point (mla_decode_noalloc) through the C ABI: its
results equal mla_decode's (same kernels and plan, so bit for bit) and the
oracle's, on two calls in a row, the second with a smaller problem; a problem
whose workspace exceeds the static scratch is refused before anything runs."""
import ctypes

import numpy as np
import pytest

import mla_inputs as mi
import oracle

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3


@pytest.fixture(scope="module")
def mla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import deepseek_mla_decode_amd as m
    m._lib.lib()
    return m


def _both(mla, inp, num_split):
    """(noalloc out, lse), (workspace out, lse) on the same device inputs."""
    import torch
    from mla_inputs.torch_io import from_device, to_device
    d = to_device(inp, "cuda")
    args = (d["q_nope"], d["q_pe"], d["kv_latent"], d["k_pe"], d["block_table"], d["cache_seqlens"],
            inp.softmax_scale)
    B, H = inp.batch, inp.heads
    out_n = torch.full((B, H, 512), float("nan"), dtype=d["q_nope"].dtype, device="cuda")
    lse_n = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_noalloc(*args, num_split=num_split, out=out_n, lse=lse_n, kv_scale=d["kv_scale"])
    torch.cuda.synchronize()
    out_w, lse_w = mla.mla_decode(*args, num_split=num_split, kv_scale=d["kv_scale"])
    torch.cuda.synchronize()
    return (from_device(out_n), from_device(lse_n)), (from_device(out_w), from_device(lse_w))


def _check(mla, inp, num_split, what):
    (on, ln), (ow, lw) = _both(mla, inp, num_split)
    assert np.array_equal(on, ow), f"{what}: output differs from mla_decode's"
    assert np.array_equal(np.nan_to_num(ln), np.nan_to_num(lw)) and np.array_equal(np.isneginf(ln), np.isneginf(lw))
    ro, rl = oracle.mla_decode_ref(inp)
    excess = np.abs(on - ro) - (ATOL + RTOL * np.abs(ro))
    assert excess.max() <= 0, f"{what}: out off by {excess.max():.3e}"
    both_inf = np.isneginf(ln) & np.isneginf(rl)
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(ln - rl))
    assert err.max() <= LSE_TOL, f"{what}: lse err {err.max():.3e}"


def test_noalloc_matches_mla_decode_on_two_calls(mla):
    """A large call (planner, 256 work items of 128 heads, close to the
    scratch limit), then a smaller paged one with forced splits: the second
    must not see anything the first left in the shared scratch."""
    lens = np.random.default_rng(160).integers(0, 4097, size=64)
    lens[[3, 40]] = 0
    big = mi.make_contiguous(64, 128, 4096, lens, "f16", seed=161)
    _check(mla, big, 0, "noalloc large, planner")
    small = mi.make_paged(3, 16, [700, 1, 2000], "bf16", seed=162, page_block_size=64, spare_pages=2)
    _check(mla, small, 4, "noalloc small, 4 splits")


def test_noalloc_fp8_cache_on_two_calls(mla):
    """The same entry point over an E4M3 cache: a paged call with the planner,
    then a smaller contiguous one with forced splits."""
    lens = np.random.default_rng(163).integers(1, 3000, size=24)
    big = mi.make_paged(24, 128, lens, "bf16", seed=164, page_block_size=64, spare_pages=3, kv_dtype="fp8")
    _check(mla, big, 0, "noalloc fp8 paged, planner")
    small = mi.make_contiguous(2, 32, 400, [400, 57], "f16", seed=165, kv_dtype="fp8")
    _check(mla, small, 3, "noalloc fp8 small, 3 splits")


def test_noalloc_refuses_problems_beyond_the_scratch(mla):
    """B = 300 sequences of 128 heads (300 work items, 38,400 partial rows,
    about 113 MiB of workspace) exceed the 100 MiB scratch: MLA_ERR_WORKSPACE,
    and nothing is launched (the data pointers are never read)."""
    L = mla._lib.lib()
    d = mla.MlaDesc()
    B, H = 300, 128
    d.batch, d.heads, d.d_latent, d.d_rope, d.dtype = B, H, 512, 64, 0
    d.max_seqlen = 64
    d.q_nope_sb, d.q_nope_sh, d.q_pe_sb, d.q_pe_sh = H * 512, 512, H * 64, 64
    d.kv_sb, d.kv_sr, d.kpe_sb, d.kpe_sr = 64 * 512, 512, 64 * 64, 64
    d.out_sb, d.out_sh = H * 512, 512
    need = mla.mla_workspace_size(d, 0, mla.mla_num_cus(0))
    assert need > mla.NOALLOC_SCRATCH_BYTES
    fake = 0x100000   # aligned, never dereferenced: the call fails before any launch
    st = L.mla_decode_noalloc(fake, fake, fake, fake, None, fake, ctypes.c_float(1 / 24), 0, fake, fake,
                              ctypes.byref(d), None)
    assert st == mla._lib.MLA_ERR_WORKSPACE
    assert "no-allocation scratch" in mla.mla_last_error()
