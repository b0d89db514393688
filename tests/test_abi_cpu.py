"""C ABI checks that need no GPU: symbols, argument validation, workspace sizes,
and the host twin of the split planner against the oracle's split ranges."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from deepseek_mla_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    return _lib.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*|size_t)\s+\**(mla_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in mla_decode.h but not exported"
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def _desc(B=2, H=16, dtype=0, **kw):
    d = _lib.MlaDesc()
    d.batch, d.heads, d.d_latent, d.d_rope, d.dtype = B, H, 512, 64, dtype
    d.max_seqlen = 256
    d.q_nope_sb, d.q_nope_sh = H * 512, 512
    d.q_pe_sb, d.q_pe_sh = H * 64, 64
    d.kv_sb, d.kv_sr = 256 * 512, 512
    d.kpe_sb, d.kpe_sr = 256 * 64, 64
    d.out_sb, d.out_sh = H * 512, 512
    for k, v in kw.items():
        setattr(d, k, v)
    return d


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation first


def _decode(L, desc, num_split=0, scale=1 / 24, ptrs=None, block_table=None, ws=FAKE, ws_bytes=1 << 40):
    p = dict(q=FAKE, qp=FAKE, kv=FAKE, kpe=FAKE, lens=FAKE, out=FAKE, lse=FAKE)
    if ptrs:
        p.update(ptrs)
    return L.mla_decode(p["q"], p["qp"], p["kv"], p["kpe"], block_table, p["lens"], scale, num_split, p["out"],
                        p["lse"], None if desc is None else ctypes.byref(desc), ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", _lib.MLA_ERR_INVALID_ARG),
    ("neg_batch", _lib.MLA_ERR_INVALID_ARG),
    ("zero_heads", _lib.MLA_ERR_INVALID_ARG),
    ("dims", _lib.MLA_ERR_UNSUPPORTED),
    ("dtype", _lib.MLA_ERR_UNSUPPORTED),
    ("neg_seqlen_q", _lib.MLA_ERR_INVALID_ARG),
    ("big_seqlen_q", _lib.MLA_ERR_UNSUPPORTED),
    ("heads_not_multiple_of_seqlen_q", _lib.MLA_ERR_INVALID_ARG),
    ("neg_split", _lib.MLA_ERR_INVALID_ARG),
    ("huge_split", _lib.MLA_ERR_INVALID_ARG),
    ("nan_scale", _lib.MLA_ERR_INVALID_ARG),
    ("null_q", _lib.MLA_ERR_INVALID_ARG),
    ("null_lens", _lib.MLA_ERR_INVALID_ARG),
    ("stride_not_8", _lib.MLA_ERR_UNSUPPORTED),
    ("neg_stride", _lib.MLA_ERR_INVALID_ARG),
    ("misaligned_kv", _lib.MLA_ERR_UNSUPPORTED),
    ("misaligned_lse", _lib.MLA_ERR_INVALID_ARG),
    ("page_16", _lib.MLA_ERR_UNSUPPORTED),
    ("page_stride0", _lib.MLA_ERR_INVALID_ARG),
    ("neg_max_seqlen", _lib.MLA_ERR_INVALID_ARG),
    ("zero_scale", _lib.MLA_ERR_INVALID_ARG),
    ("neg_scale", _lib.MLA_ERR_INVALID_ARG),
    ("huge_row_stride", _lib.MLA_ERR_UNSUPPORTED),
    ("huge_q_head_stride", _lib.MLA_ERR_UNSUPPORTED),
])
def test_validation_errors(L, case, expect):
    d = _desc()
    kw = {}
    if case == "null_desc":
        d = None
    elif case == "neg_batch":
        d.batch = -1
    elif case == "zero_heads":
        d.heads = 0
    elif case == "dims":
        d.d_latent = 448
    elif case == "dtype":
        d.dtype = 7
    elif case == "neg_seqlen_q":
        d.seqlen_q = -1
    elif case == "big_seqlen_q":
        d.seqlen_q = 17
    elif case == "heads_not_multiple_of_seqlen_q":
        d.seqlen_q = 3
    elif case == "neg_split":
        kw["num_split"] = -1
    elif case == "huge_split":
        kw["num_split"] = _lib.MAX_SPLITS + 1
    elif case == "nan_scale":
        kw["scale"] = float("nan")
    elif case == "null_q":
        kw["ptrs"] = {"q": None}
    elif case == "null_lens":
        kw["ptrs"] = {"lens": None}
    elif case == "stride_not_8":
        d.kv_sr = 516
    elif case == "neg_stride":
        d.out_sh = -512
    elif case == "misaligned_kv":
        kw["ptrs"] = {"kv": FAKE + 2}
    elif case == "misaligned_lse":
        kw["ptrs"] = {"lse": FAKE + 2}
    elif case == "page_16":
        d.page_block_size, d.block_table_stride, d.num_pages = 16, 4, 8
        kw["block_table"] = FAKE
    elif case == "page_stride0":
        d.page_block_size, d.block_table_stride, d.num_pages = 64, 0, 8
        kw["block_table"] = FAKE
    elif case == "neg_max_seqlen":
        d.max_seqlen = -1
    elif case == "zero_scale":
        kw["scale"] = 0.0
    elif case == "neg_scale":
        kw["scale"] = -0.04
    elif case == "huge_row_stride":
        d.kpe_sr = 1 << 22
    elif case == "huge_q_head_stride":
        d.q_pe_sh = 1 << 22
    st = _decode(L, d, **kw)
    assert st == expect, (case, st, L.mla_last_error())
    assert L.mla_last_error().decode()


@pytest.mark.parametrize("case,expect", [
    ("kv_dtype", _lib.MLA_ERR_UNSUPPORTED),
    ("fp8_zero_scale", _lib.MLA_ERR_INVALID_ARG),
    ("fp8_neg_scale", _lib.MLA_ERR_INVALID_ARG),
    ("fp8_inf_scale", _lib.MLA_ERR_INVALID_ARG),
    ("fp8_nan_scale", _lib.MLA_ERR_INVALID_ARG),
    ("fp8_row_stride_not_16", _lib.MLA_ERR_UNSUPPORTED),
    ("fp8_page_stride_not_16", _lib.MLA_ERR_UNSUPPORTED),
    ("scale_on_16bit_cache", _lib.MLA_ERR_INVALID_ARG),
])
def test_kv_cache_format_validation(L, case, expect):
    """An FP8 cache needs a finite positive kv_scale and cache strides in
    multiples of 16 bytes (rows 16-byte aligned); a 16-bit cache takes no
    scale (0 and 1 mean none); other kv_dtype values are unsupported."""
    d = _desc(kv_dtype=_lib.MLA_KV_FP8_E4M3, kv_scale=0.5)
    kw = {}
    if case == "kv_dtype":
        d.kv_dtype = 2
    elif case == "fp8_zero_scale":
        d.kv_scale = 0.0
    elif case == "fp8_neg_scale":
        d.kv_scale = -0.5
    elif case == "fp8_inf_scale":
        d.kv_scale = float("inf")
    elif case == "fp8_nan_scale":
        d.kv_scale = float("nan")
    elif case == "fp8_row_stride_not_16":
        d.kv_sr = 520   # a multiple of 8 (fine for a 16-bit cache), not of 16 bytes
    elif case == "fp8_page_stride_not_16":
        d.page_block_size, d.block_table_stride, d.num_pages = 64, 4, 8
        d.kv_sb, d.kv_sr, d.kpe_sb, d.kpe_sr = 64 * 576 + 8, 576, 64 * 576, 576
        kw["block_table"] = FAKE
    elif case == "scale_on_16bit_cache":
        d.kv_dtype, d.kv_scale = _lib.MLA_KV_AS_DTYPE, 0.5
    st = _decode(L, d, **kw)
    assert st == expect, (case, st, L.mla_last_error())
    assert L.mla_last_error().decode()
    # the same description with a good scale and 16-byte strides passes validation (MLA_ERR_WORKSPACE:
    # the fake workspace size is checked after every argument)
    good = _desc(kv_dtype=_lib.MLA_KV_FP8_E4M3, kv_scale=0.5)
    assert _decode(L, good, ws=None, ws_bytes=0) in (_lib.MLA_ERR_WORKSPACE, _lib.MLA_ERR_HIP)


def test_empty_batch_is_ok_without_touching_memory(L):
    d = _desc(B=0)
    assert _decode(L, d, ptrs={k: None for k in ("q", "qp", "kv", "kpe", "lens", "out", "lse")}) == _lib.MLA_OK


def test_workspace_size_formula(L):
    for B, H, ns, cus, sq in [(2, 16, 1, 256, 1), (64, 128, 0, 256, 1), (2, 128, 64, 256, 1), (3, 200, 0, 256, 1),
                              (500, 128, 0, 256, 1), (64, 256, 0, 256, 2), (3, 96, 5, 256, 3), (200, 128, 0, 256, 4),
                              (2, 256, 0, 256, 2), (16, 128, 0, 256, 4)]:
        d = _desc(B=B, H=H, dtype=(B + H) % 2)   # fp16 and bf16 both covered
        d.seqlen_q = sq
        w = ctypes.c_int32()
        assert L.mla_max_work(ctypes.byref(d), ns, cus, ctypes.byref(w)) == 0
        hg = -(-H // 128)
        tail = 2 if sq > 1 else 0
        C = -(-cus // hg)
        if tail and 4 * B * tail <= C:
            C -= B * tail
        want_w = B * (ns + tail) if ns else max(B, C) + B * tail
        assert w.value == want_w
        n = ctypes.c_size_t()
        assert L.mla_workspace_size(ctypes.byref(d), ns, cus, ctypes.byref(n)) == 0
        r = lambda x: -(-x // 256) * 256  # noqa: E731
        plan = 4 * B + 4 * (B + 1) + 16 * want_w
        part_lse = r(plan)
        part16 = r(part_lse + 4 * want_w * H)
        part32 = r(part16 + 512 * 2 * want_w * H)
        assert n.value == r(part32 + 512 * 4 * want_w * H)   # fp16 rows, fp32 copies of the wide ones


def _plan(lens, heads, ns, cus, sq=1):
    from deepseek_mla_decode_amd import mla_plan_host
    return mla_plan_host(np.asarray(lens, np.int32), heads, ns, cus, seqlen_q=sq)


def _check_ranges_against_oracle(lens, ns_arr, off, work):
    for b, L_b in enumerate(lens):
        s = int(ns_arr[b])
        want = oracle.split_ranges(int(max(L_b, 0)), s)
        got = [(int(work[off[b] + k, 2]), int(work[off[b] + k, 3])) for k in range(s)]
        assert got == want, (b, L_b, s)
        assert all(int(work[off[b] + k, 0]) == b and int(work[off[b] + k, 1]) == k for k in range(s))


@pytest.mark.parametrize("lens,heads,ns", [
    ([256, 256], 16, 1), ([256, 256], 16, 4), ([4096] * 64, 128, 0), ([8192] * 128, 128, 0),
    ([131072] * 2, 128, 0), ([131072] * 2, 128, 64), ([1, 0, 65, 64, 63, 300], 128, 0),
    ([0, 0, 0], 128, 0), ([5, 7], 128, 8),
])
def test_host_planner_matches_oracle_ranges(lens, heads, ns):
    nsa, off, work = _plan(lens, heads, ns, 256)
    assert off[0] == 0 and int(off[-1]) == work.shape[0]
    if ns:
        assert (nsa == ns).all()
    _check_ranges_against_oracle(lens, nsa, off, work)


def test_planner_fills_the_cus_for_uniform_lengths():
    for lens, want in (([4096] * 64, 4), ([8192] * 128, 2), ([131072] * 2, 128)):
        nsa, off, _ = _plan(lens, 128, 0, 256)
        assert (nsa == want).all() and int(off[-1]) == 256


def test_planner_budget_is_minimal_on_random_lengths():
    rng = np.random.default_rng(0)
    for trial in range(20):
        B = int(rng.integers(1, 300))
        lens = rng.integers(0, 20000, size=B).astype(np.int32)
        heads = int(rng.choice([16, 64, 128, 256]))
        cus = int(rng.choice([80, 256, 304]))
        nsa, off, work = _plan(lens, heads, 0, cus)
        hg = -(-heads // 128)
        cap = max(B, -(-cus // hg))
        assert int(off[-1]) <= cap and (nsa >= 1).all()
        nb = -(-lens.astype(np.int64) // 64)
        # the largest work item is at most t blocks, and with t - 1 the split total would exceed cap
        t = max(int(max(-(-n // s) for n, s in zip(nb, nsa))), 1)
        if t > 1:
            assert sum(max(1, -(-int(n) // (t - 1))) for n in nb) > cap
        _check_ranges_against_oracle(lens, nsa, off, work)


@pytest.mark.parametrize("lens,heads,ns,sq", [
    ([4096] * 64, 256, 0, 2), ([1, 0, 2, 3, 65, 66, 300], 96, 0, 3), ([100, 5], 64, 4, 4), ([0, 0], 32, 2, 2),
    ([131072] * 2, 512, 0, 4),
])
def test_host_planner_tail_splits(lens, heads, ns, sq):
    """Several query tokens: the splits cut the prefix -- rows every token sees,
    down to a multiple of 32 -- as the oracle's split_ranges does, and two
    single-tile tail splits take the rest."""
    nsa, off, work = _plan(lens, heads, ns, 256, sq)
    assert int(off[-1]) == work.shape[0]
    for b, L in enumerate(lens):
        s = int(nsa[b])
        if ns:
            assert s == ns + 2
        Lp = max(L - (sq - 1), 0) // 32 * 32
        mid = min(Lp + 32, L)
        assert L - Lp <= 32 + 31 and Lp <= max(L - (sq - 1), 0)
        want = oracle.split_ranges(Lp, s - 2) + [(Lp, mid), (mid, L)]
        got = [(int(work[off[b] + k, 2]), int(work[off[b] + k, 3])) for k in range(s)]
        assert got == want, (b, L, got, want)


def test_split_starts_keep_tiles_inside_pages():
    """Every nonempty split starts at a multiple of 32 rows, for any lengths,
    query-token counts and split modes: a 32-row tile then never crosses a
    page (page sizes are multiples of 32), which the paged tile loads rely
    on."""
    rng = np.random.default_rng(5)
    for trial in range(60):
        B = int(rng.integers(1, 120))
        lens = rng.integers(0, 9000, size=B).astype(np.int32)
        sq = int(rng.choice([1, 2, 3, 4, 8, 16]))
        heads = sq * int(rng.choice([16, 32, 64, 128]))
        ns = int(rng.choice([0, 0, 1, 3, 7]))
        nsa, off, work = _plan(lens, heads, ns, int(rng.choice([80, 256, 304])), sq)
        nonempty = work[:, 3] > work[:, 2]
        assert (work[nonempty, 2] % 32 == 0).all(), (sq, ns, work[nonempty][work[nonempty, 2] % 32 != 0][:3])


def test_xcd_mapping_with_two_kinds_is_a_bijection():
    """The split kernel's workgroup order (restated): workgroup f runs on XCD
    f % 8 as its (f // 8)-th; each XCD takes its even share of the nb prefix
    workgroups first, then the rest of its workgroups are tails.  For every
    total and tail count this must hit each work-item index exactly once,
    tails in [0, nt) and prefix splits in [nt, total)."""
    def before(n, x):
        return x * (n // 8) + min(x, n % 8)

    for total in list(range(1, 130)) + [255, 256, 257, 264, 512, 768, 1031]:
        for nt in sorted({0, 1, 2, 7, 8, 9, total // 3, total // 2, total - 1, total} & set(range(total + 1))):
            nb = total - nt
            seen = []
            for f in range(total):
                x, idx = f % 8, f // 8
                nb_x = before(nb, x + 1) - before(nb, x)
                if idx < nb_x:
                    lin = nt + before(nb, x) + idx
                    assert nt <= lin < total
                else:
                    lin = before(total, x) - before(nb, x) + (idx - nb_x)
                    assert 0 <= lin < nt
                seen.append(lin)
            assert sorted(seen) == list(range(total)), (total, nt)


def test_combine_xcd_order_is_a_bijection_matching_the_split_order():
    """The combine kernels' workgroup order (restated): workgroup (x, y) with
    flat id f = x + y * gx runs on XCD f % 8 as its (f // 8)-th and takes grid
    position lin = before(total, f % 8) + f // 8 in y-major order.  It must hit
    every (x, y) exactly once, and with equal splits per sequence each XCD must
    merge the sequences whose splits the split kernel gave it (the same
    contiguous run of sequences)."""
    def before(n, x):
        return x * (n // 8) + min(x, n % 8)

    for gx in (1, 2, 3, 8, 13, 32, 33, 128):
        for gy in (1, 2, 5, 7, 8, 64, 100, 129):
            total = gx * gy
            seen = set()
            for f in range(total):
                lin = before(total, f % 8) + f // 8
                seen.add((lin % gx, lin // gx))
            assert seen == {(x, y) for x in range(gx) for y in range(gy)}, (gx, gy)
    # B sequences of s splits: split workgroup f works on item before(B s, f % 8)
    # + f // 8, sequence item // s; combine workgroups of sequence b sit on the
    # XCDs whose split workgroups hold b.
    for B, s, gx in ((64, 4, 32), (128, 2, 32), (2, 128, 128), (40, 6, 32)):
        W = B * s
        split_xcd = {}
        for f in range(W):
            item = before(W, f % 8) + f // 8
            split_xcd.setdefault(item // s, set()).add(f % 8)
        total = gx * B
        for f in range(total):
            b = (before(total, f % 8) + f // 8) // gx
            if len(split_xcd[b]) == 1:
                assert f % 8 in split_xcd[b], (B, s, b)


def test_block_table_check_validation(L):
    """mla_check_block_table rejects a missing description, NULL arrays and
    bad paging fields before launching anything; an empty batch is a no-op."""
    d = _desc(B=2, page_block_size=64, block_table_stride=4, num_pages=8)
    chk = lambda desc, bt=FAKE, lens=FAKE, bad=FAKE: L.mla_check_block_table(  # noqa: E731
        bt, lens, None if desc is None else ctypes.byref(desc), bad, None)
    assert chk(None) == _lib.MLA_ERR_INVALID_ARG
    for kw in ({"bt": None}, {"lens": None}, {"bad": None}, {"bad": FAKE + 2}):
        assert chk(d, **kw) == _lib.MLA_ERR_INVALID_ARG, kw
    for field, value, want in (("page_block_size", 16, _lib.MLA_ERR_UNSUPPORTED),
                               ("block_table_stride", 0, _lib.MLA_ERR_INVALID_ARG),
                               ("num_pages", 0, _lib.MLA_ERR_INVALID_ARG), ("batch", -1, _lib.MLA_ERR_INVALID_ARG)):
        bad_desc = _desc(B=2, page_block_size=64, block_table_stride=4, num_pages=8)
        setattr(bad_desc, field, value)
        assert chk(bad_desc) == want, field
        assert L.mla_last_error().decode()
    assert chk(_desc(B=0), bt=None, lens=None, bad=None) == _lib.MLA_OK


@pytest.mark.parametrize("case", ["null_num_splits", "null_split_offset", "null_work", "zero_capacity",
                                  "misaligned_work", "zero_heads"])
def test_planned_decode_validation(L, case):
    """mla_decode_planned refuses NULL or misaligned plan arrays and a capacity
    below one before anything else (no device call); a well-formed call gets
    past them to the device checks."""
    d = _desc()
    ns, off, work, cap = FAKE, FAKE, FAKE, 256
    if case == "null_num_splits":
        ns = None
    elif case == "null_split_offset":
        off = None
    elif case == "null_work":
        work = None
    elif case == "zero_capacity":
        cap = 0
    elif case == "misaligned_work":
        work = FAKE + 4
    elif case == "zero_heads":
        d.heads = 0

    def call(desc, ns, off, work, cap, ws=FAKE, ws_bytes=1 << 40):
        return L.mla_decode_planned(FAKE, FAKE, FAKE, FAKE, None, FAKE, ctypes.c_float(1 / 24), ns, off, work,
                                    cap, FAKE, FAKE, ctypes.byref(desc), ws, ws_bytes, None)

    st = call(d, ns, off, work, cap)
    assert st == _lib.MLA_ERR_INVALID_ARG, (case, st, L.mla_last_error())
    assert L.mla_last_error().decode()
    assert call(_desc(), FAKE, FAKE, FAKE, 256, ws=None, ws_bytes=0) in (_lib.MLA_ERR_WORKSPACE, _lib.MLA_ERR_HIP)
