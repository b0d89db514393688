"""Decode with a plan made beforehand (mla_decode_planned): one mla_plan_device
call per decode step serves every layer, as FlashMLA's metadata call does
(FlashMLA analysis, "内存访问优化" section).  The planned call runs the same
work items as mla_decode (its own planner, or forced splits) and so gives
the same bits; with several query tokens the items run in another order,
which changes no item's arithmetic.  A plan made for other lengths, or one
holding arbitrary integers, is clamped by the kernels: the call completes
and touches nothing outside its buffers.
"""
import ctypes

import numpy as np
import pytest

import mla_inputs as mi
import oracle
from tests.test_gpu_parity import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import deepseek_mla_decode_amd as m
    m._lib.lib()   # loud failure if the library is missing
    return m


def _args(d, inp):
    return (d["q_nope"], d["q_pe"], d["kv_latent"], d["k_pe"], d["block_table"], d["cache_seqlens"],
            inp.softmax_scale)


def _both(mla, inp, num_split):
    """(planned out, lse), (mla_decode out, lse) as device tensors."""
    import torch
    from mla_inputs.torch_io import to_device
    d = to_device(inp, "cuda")
    cus = mla.mla_num_cus(0)
    plan = mla.mla_plan_device(d["cache_seqlens"], inp.heads, num_split, cus, seqlen_q=inp.seqlen_q)
    if inp.seqlen_q > 1:
        B, s, H = inp.batch, inp.seqlen_q, inp.heads // inp.seqlen_q
        qn, qp = d["q_nope"].view(B, s, H, 512), d["q_pe"].view(B, s, H, 64)
        a = (qn, qp) + _args(d, inp)[2:]
    else:
        a = _args(d, inp)
    op, lp = mla.mla_decode_planned(*a, plan, num_split=num_split, num_cus=cus, kv_scale=d["kv_scale"])
    od, ld = mla.mla_decode(*a, num_split=num_split, kv_scale=d["kv_scale"])
    torch.cuda.synchronize()
    return (op, lp), (od, ld)


@pytest.mark.parametrize("case", ["contiguous_f16", "paged_bf16_varlen", "forced_5", "kv_fp8", "two_tokens",
                                  "forced_3_four_tokens", "two_head_groups", "kv_fp8_paged_f16",
                                  "kv_fp8_paged_bf16_two_tokens", "kv_fp8_contiguous_bf16"])
def test_planned_matches_mla_decode_bitwise(mla, case):
    import torch
    from mla_inputs.torch_io import from_device
    num_split = 0
    if case == "contiguous_f16":
        inp = mi.make_config(1, batch_subset=16)
    elif case == "paged_bf16_varlen":
        inp = mi.make_config(3, batch_subset=16)
    elif case == "forced_5":
        inp = mi.make_paged(6, 64, [1, 64, 129, 500, 3000, 0], "bf16", seed=301, page_block_size=64)
        num_split = 5
    elif case == "kv_fp8":
        inp = mi.make_contiguous(8, 128, 2000, [2000, 1, 33, 700, 1999, 64, 65, 1000], "f16", seed=302,
                                 kv_dtype="fp8")
    elif case == "two_tokens":
        inp = mi.make_paged(5, 64, [3, 64, 65, 700, 2500], "f16", seed=303, page_block_size=64, seqlen_q=2)
    elif case == "forced_3_four_tokens":
        # forced prefix splits plus the two tail splits per sequence in the plan
        inp = mi.make_paged(4, 128, [4, 40, 333, 1500], "bf16", seed=304, page_block_size=64, seqlen_q=4)
        num_split = 3
    elif case == "two_head_groups":
        inp = mi.make_contiguous(3, 256, 900, [900, 17, 450], "bf16", seed=305)
    elif case == "kv_fp8_paged_f16":
        inp = mi.make_paged(6, 128, [1, 64, 65, 1500, 0, 3100], "f16", seed=306, page_block_size=64,
                            kv_dtype="fp8")
    elif case == "kv_fp8_paged_bf16_two_tokens":
        inp = mi.make_paged(5, 64, [2, 33, 640, 2047, 2500], "bf16", seed=307, page_block_size=128, seqlen_q=2,
                            kv_dtype="fp8")
    else:
        inp = mi.make_contiguous(4, 128, 1800, [1800, 1, 900, 95], "bf16", seed=308, kv_dtype="fp8")
    (op, lp), (od, ld) = _both(mla, inp, num_split)
    assert torch.equal(op, od), f"{case}: planned output differs from mla_decode's"
    assert torch.equal(torch.nan_to_num(lp), torch.nan_to_num(ld)) and torch.equal(torch.isneginf(lp),
                                                                                   torch.isneginf(ld))
    ro, rl = oracle.mla_decode_ref(inp)
    o, l = from_device(op), from_device(lp)
    if inp.seqlen_q > 1:
        o, l = o.reshape(ro.shape), l.reshape(rl.shape)
    assert_parity(o, l, ro, rl, f"planned {case}")


def test_one_plan_serves_several_layers(mla):
    """Three layers (their own queries and caches, the same lengths) decoded with
    one plan: each equals its own mla_decode call."""
    import torch
    from mla_inputs.torch_io import to_device
    lens = np.random.default_rng(310).integers(1, 6000, size=24)
    cus = mla.mla_num_cus(0)
    inps = [mi.make_paged(24, 128, lens, "bf16", seed=311 + i, page_block_size=64) for i in range(3)]
    layers = [to_device(inp, "cuda") for inp in inps]
    plan = mla.mla_plan_device(layers[0]["cache_seqlens"], 128, 0, cus)
    for i, (inp, d) in enumerate(zip(inps, layers)):
        a = _args(d, inp)
        op, lp = mla.mla_decode_planned(*a, plan)
        od, ld = mla.mla_decode(*a)
        torch.cuda.synchronize()
        assert torch.equal(op, od) and torch.equal(lp, ld), f"layer {i}"


def test_plan_for_other_lengths_stays_in_bounds(mla):
    """A plan made for longer sequences, and one of arbitrary integers: the
    kernels clamp every field they read (sequence and split index, row
    range, item count, split offsets), so each call completes and leaves the
    rows outside out untouched (out is a slice of a larger NaN-filled
    buffer whose guard rows must stay NaN)."""
    import torch
    from mla_inputs.torch_io import to_device
    inp = mi.make_paged(6, 64, [10, 200, 64, 1000, 1, 333], "f16", seed=320, page_block_size=64, spare_pages=3)
    d = to_device(inp, "cuda")
    cus = mla.mla_num_cus(0)
    longer = torch.tensor([4000, 9000, 64, 20000, 1, 7000], dtype=torch.int32, device="cuda")
    stale = mla.mla_plan_device(longer, 64, 0, cus)
    rng = np.random.default_rng(321)
    max_work = stale[2].shape[0]
    garbage = (torch.tensor(rng.integers(-2**31, 2**31 - 1, size=6), dtype=torch.int32, device="cuda"),
               torch.tensor(rng.integers(-2**31, 2**31 - 1, size=7), dtype=torch.int32, device="cuda"),
               torch.tensor(rng.integers(-2**31, 2**31 - 1, size=(max_work, 4)), dtype=torch.int32,
                            device="cuda"))
    for name, plan in (("stale", stale), ("arbitrary", garbage)):
        big = torch.full((8, 64, 512), float("nan"), dtype=torch.float16, device="cuda")
        out = big[1:7]
        op, lp = mla.mla_decode_planned(*_args(d, inp), plan, out=out, num_cus=cus)
        torch.cuda.synchronize()
        assert torch.isnan(big[0]).all() and torch.isnan(big[7]).all(), f"{name}: write outside out"


def test_planned_argument_errors(mla):
    """NULL plan arrays and a capacity below one are refused before any launch;
    the binding checks the plan tensors' device, type and shape."""
    import torch
    from mla_inputs.torch_io import to_device
    inp = mi.make_contiguous(2, 16, 64, [64, 10], "f16", seed=330)
    d = to_device(inp, "cuda")
    cus = mla.mla_num_cus(0)
    plan = mla.mla_plan_device(d["cache_seqlens"], 16, 0, cus)
    ns, off, work = plan
    with pytest.raises(ValueError, match="split_offset"):
        mla.mla_decode_planned(*_args(d, inp), (ns, off[:-1], work))
    with pytest.raises(ValueError, match="work"):
        mla.mla_decode_planned(*_args(d, inp), (ns, off, work.view(-1)))
    with pytest.raises(ValueError, match="device"):
        mla.mla_decode_planned(*_args(d, inp), (ns.cpu(), off, work))
    L = mla._lib.lib()
    desc = mla.make_desc(d["q_nope"], d["q_pe"], d["kv_latent"], d["k_pe"], None, torch.empty_like(d["q_nope"]))
    ws = torch.empty(mla.mla_workspace_size(desc, 0, cus), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q_nope"])
    lse = torch.empty((2, 16), dtype=torch.float32, device="cuda")
    common = (d["q_nope"].data_ptr(), d["q_pe"].data_ptr(), d["kv_latent"].data_ptr(), d["k_pe"].data_ptr(), None,
              d["cache_seqlens"].data_ptr(), ctypes.c_float(inp.softmax_scale))
    tail = (out.data_ptr(), lse.data_ptr(), ctypes.byref(desc), ws.data_ptr(), ws.numel(), None)
    st = L.mla_decode_planned(*common, None, off.data_ptr(), work.data_ptr(), work.shape[0], *tail)
    assert st == mla._lib.MLA_ERR_INVALID_ARG and "plan" in mla.mla_last_error()
    st = L.mla_decode_planned(*common, ns.data_ptr(), off.data_ptr(), work.data_ptr(), 0, *tail)
    assert st == mla._lib.MLA_ERR_INVALID_ARG and "max_work" in mla.mla_last_error()
    torch.cuda.synchronize()


def test_graph_of_plan_and_layers_follows_new_lengths(mla):
    """A decode step as a serving loop captures it: the plan (mla_plan_device)
    and two layers' planned decodes in one HIP graph, replayed after the
    lengths tensor has been rewritten in place (a step that appended a token
    to every sequence, then back).  The plan is made inside the graph, so each
    replay follows the current lengths: every layer's output equals an eager
    mla_decode call on the same lengths bit for bit, and the longer step
    matches the oracle."""
    import torch
    from mla_inputs.torch_io import to_device, from_device
    lens1 = [700, 1, 2000, 64, 0, 1500]
    lens2 = [701, 2, 2001, 65, 1, 1501]
    inps = [mi.make_paged(6, 128, lens2, "bf16", seed=340 + i, page_block_size=64) for i in range(2)]
    layers = [to_device(inp, "cuda") for inp in inps]
    cus = mla.mla_num_cus(0)
    seqlens = torch.tensor(lens1, dtype=torch.int32, device="cuda")
    outs = [torch.empty((6, 128, 512), dtype=torch.bfloat16, device="cuda") for _ in layers]
    lses = [torch.empty((6, 128), dtype=torch.float32, device="cuda") for _ in layers]
    d0 = layers[0]
    desc = mla.make_desc(d0["q_nope"], d0["q_pe"], d0["kv_latent"], d0["k_pe"], d0["block_table"], outs[0])
    ws = torch.empty(mla.mla_workspace_size(desc, 0, cus), dtype=torch.uint8, device="cuda")
    scale = inps[0].softmax_scale

    def step():
        plan = mla.mla_plan_device(seqlens, 128, 0, cus)
        for d, o, l in zip(layers, outs, lses):
            mla.mla_decode_planned(d["q_nope"], d["q_pe"], d["kv_latent"], d["k_pe"], d["block_table"], seqlens,
                                   scale, plan, num_cus=cus, out=o, lse=l, workspace=ws)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    for r, lens in enumerate((lens2, lens1, lens2)):
        seqlens.copy_(torch.tensor(lens, dtype=torch.int32))
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (d, o, l) in enumerate(zip(layers, outs, lses)):
            eo, el = mla.mla_decode(d["q_nope"], d["q_pe"], d["kv_latent"], d["k_pe"], d["block_table"], seqlens,
                                    scale)
            torch.cuda.synchronize()
            assert torch.equal(o, eo), f"replay {r} layer {i}: output differs from eager"
            assert torch.equal(torch.nan_to_num(l), torch.nan_to_num(el)) and torch.equal(
                torch.isneginf(l), torch.isneginf(el)), f"replay {r} layer {i}: lse differs from eager"
    ro, rl = oracle.mla_decode_ref(inps[1])
    assert_parity(from_device(outs[1]), from_device(lses[1]), ro, rl, "graph replay, longer step")
