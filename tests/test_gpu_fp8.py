"""GPU parity of the FP8 (E4M3) KV cache: the HIP path through the C ABI
against the fp64 oracle, which decodes every byte by the format's definition
and multiplies by kv_scale (the TileLang MLA guide lists the FP8 KV-cache
variant among its kernels, "变体内核"; the format and the per-tensor scale are
this library's reading, stated in include/mla_decode.h).

Same tolerance as the 16-bit path: |out - ref| <= 2e-3 + 1e-2 |ref| and
|lse - ref| <= 1e-3 elementwise; the cache values are exact in both 16-bit
types, so only the kernel's own arithmetic differs from the oracle's.
"""
import numpy as np
import pytest

import mla_inputs as mi
import oracle
from tests.test_gpu_parity import _full_inputs, _run, _run_tokens, assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import deepseek_mla_decode_amd as m
    m._lib.lib()   # loud failure if the library is missing
    return m


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("num_split", [1, 4, 0])
def test_tiny(mla, dtype, num_split):
    inp = mi.make_contiguous(2, 16, 256, [256, 256], dtype, seed=0, kv_dtype="fp8")
    out, lse = _run(mla, inp, num_split)
    ro, rl = oracle.mla_decode_ref(inp)
    assert_parity(out, lse, ro, rl, f"fp8 tiny {dtype} split={num_split}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("num_split", [0, 1, 3, 8])
def test_ragged_lengths(mla, dtype, num_split):
    """Lengths around the 32-row tile and 64-row block edges; 0 gives out = 0,
    lse = -inf.  Tiles past the end re-read the last one into staging slots
    that are widened but never read."""
    lens = [0, 1, 31, 32, 33, 100, 64, 65, 96, 97, 200, 257]
    inp = mi.make_contiguous(len(lens), 128, 260, lens, dtype, seed=201, kv_dtype="fp8")
    out, lse = _run(mla, inp, num_split)
    ro, rl = oracle.mla_decode_ref(inp)
    assert_parity(out, lse, ro, rl, f"fp8 ragged {dtype} split={num_split}")
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()


@pytest.mark.parametrize("page", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_paged(mla, page, dtype):
    """Paged pool [P, page, 1, 576] of E4M3 bytes (rows 576 bytes apart, the
    RoPE part at byte 512), shuffled block table with spare pages."""
    lens = [1, 64, 129, 500, 1000, 33]
    inp = mi.make_paged(len(lens), 128, lens, dtype, seed=203, page_block_size=page, spare_pages=5,
                        kv_dtype="fp8")
    for ns in (0, 1, 5):
        out, lse = _run(mla, inp, ns)
        ro, rl = oracle.mla_decode_ref(inp)
        assert_parity(out, lse, ro, rl, f"fp8 paged page={page} {dtype} split={ns}")


@pytest.mark.parametrize("heads", [1, 16, 33, 96, 160, 256])
def test_head_counts(mla, heads):
    """Fewer heads than a group: waves with no heads only load and widen their
    share of every tile; 160 and 256 heads take two head groups, each widening
    the same tiles in a workgroup of its own."""
    inp = mi.make_contiguous(3, heads, 150, [150, 77, 5], "f16", seed=202, kv_dtype="fp8")
    for ns in (0, 2):
        out, lse = _run(mla, inp, ns)
        ro, rl = oracle.mla_decode_ref(inp)
        assert_parity(out, lse, ro, rl, f"fp8 heads={heads} split={ns}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_code_value(mla, dtype):
    """Cache bytes drawn uniformly from all 254 finite E4M3 codes (zeros of
    both signs, subnormals, 448), kv_scale = 1/448 so values lie in [-1, 1]:
    every code passes through the kernel's widening."""
    lens = [300, 47]
    inp = mi.make_contiguous(len(lens), 64, 300, lens, dtype, seed=204, kv_dtype="fp8", kv_scale=1.0 / 448)
    rng = np.random.default_rng(205)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    inp.kv_latent[...] = rng.choice(codes, size=inp.kv_latent.shape)
    inp.k_pe[...] = rng.choice(codes, size=inp.k_pe.shape)
    assert set(np.unique(inp.kv_latent)) == set(codes.tolist())
    for ns in (1, 4):
        out, lse = _run(mla, inp, ns)
        ro, rl = oracle.mla_decode_ref(inp)
        assert_parity(out, lse, ro, rl, f"fp8 all codes {dtype} split={ns}")


@pytest.mark.parametrize("kv_scale", [1.0, 0.0125, 3.0e-3])
def test_kv_scale(mla, kv_scale):
    """The scale multiplies scores and values: the same bytes under three
    scales, each against the oracle's decode(byte) * kv_scale."""
    inp = mi.make_contiguous(2, 128, 500, [500, 260], "bf16", seed=206, kv_dtype="fp8", kv_scale=0.0125)
    inp.kv_scale = kv_scale
    for ns in (1, 3):
        out, lse = _run(mla, inp, ns)
        ro, rl = oracle.mla_decode_ref(inp)
        assert_parity(out, lse, ro, rl, f"fp8 kv_scale={kv_scale} split={ns}")


@pytest.mark.parametrize("seqlen_q", [2, 4])
def test_several_query_tokens(mla, seqlen_q):
    lens = [0, 1, 3, 33, 64, 65, 300]
    inp = mi.make_paged(len(lens), 64, lens, "bf16", seed=207, page_block_size=64, seqlen_q=seqlen_q,
                        kv_dtype="fp8")
    for ns in (0, 2):
        out, lse = _run_tokens(mla, inp, ns)
        ro, rl = oracle.mla_decode_ref(inp)
        assert_parity(out, lse, ro, rl, f"fp8 {seqlen_q} tokens split={ns}")


def test_float8_tensor_type_is_accepted(mla):
    """PyTorch's float8_e4m3fn tensors are the same bytes as uint8 ones."""
    import torch
    from mla_inputs.torch_io import from_device, to_device
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("no float8_e4m3fn in this PyTorch")
    inp = mi.make_contiguous(2, 32, 100, [100, 40], "f16", seed=208, kv_dtype="fp8")
    d = to_device(inp, "cuda")
    o8, l8 = mla.mla_decode(d["q_nope"], d["q_pe"], d["kv_latent"], d["k_pe"], None, d["cache_seqlens"],
                            inp.softmax_scale, kv_scale=inp.kv_scale)
    of, lf = mla.mla_decode(d["q_nope"], d["q_pe"], d["kv_latent"].view(torch.float8_e4m3fn),
                            d["k_pe"].view(torch.float8_e4m3fn), None, d["cache_seqlens"], inp.softmax_scale,
                            kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    assert torch.equal(o8, of) and torch.equal(l8, lf)
    ro, rl = oracle.mla_decode_ref(inp)
    assert_parity(from_device(of), from_device(lf), ro, rl, "float8_e4m3fn")


def test_bad_scales_are_rejected(mla):
    import torch
    from mla_inputs.torch_io import to_device
    inp = mi.make_contiguous(1, 16, 64, [64], "f16", seed=209, kv_dtype="fp8")
    d = to_device(inp, "cuda")
    args = (d["q_nope"], d["q_pe"], d["kv_latent"], d["k_pe"], None, d["cache_seqlens"], inp.softmax_scale)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(mla.MlaError, match="kv_scale"):
            mla.mla_decode(*args, kv_scale=bad)
    inp16 = mi.make_contiguous(1, 16, 64, [64], "f16", seed=209)
    d16 = to_device(inp16, "cuda")
    with pytest.raises(ValueError, match="kv_scale"):
        mla.mla_decode(d16["q_nope"], d16["q_pe"], d16["kv_latent"], d16["k_pe"], None, d16["cache_seqlens"],
                       inp16.softmax_scale, kv_scale=0.5)
    torch.cuda.synchronize()


def test_full_b64_l4096_f16_kvfp8(mla):
    """The headline shape with an FP8 cache: every sequence and head."""
    _full_inputs(mla, mi.make_config(1, kv_dtype="fp8"), (0, 1), "b64_h128_l4096_f16_kvfp8")


def test_full_b128_l8192_f16_kvfp8(mla):
    _full_inputs(mla, mi.make_config(2, kv_dtype="fp8"), (0,), "b128_h128_l8192_f16_kvfp8")


def test_full_paged_variable_bf16_kvfp8(mla):
    _full_inputs(mla, mi.make_config(3, kv_dtype="fp8"), (0, 4), "paged_b64_h128_lU1-16384_bf16_kvfp8")
