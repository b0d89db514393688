"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes the oracle module (so that the mutation test can
hand in a deliberately broken copy) and raises ``AssertionError`` when the
oracle disagrees with:

* a pure-Python brute force that evaluates the definition differently
  (softmax weights as 1 / Σ_i exp(z_i - z_j), dot products with math.fsum,
  fp16/bf16 decoded with ``struct``), on tiny shapes;
* closed forms (seqlen 1, uniform attention, a dominant key, the stored
  hand-derived fixtures under ``tests/golden``);
* invariants (shift of all scores, normalisation, permutation of rows and of
  pages, number of splits, independence of sequences).

The definition being pinned: TileLang MLA guide, sections "先看核心难点" and
"参考实现与正确性验证"; split/combine: the same guide's "Split Kernel" and
"Combine Kernel" sections.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

import mla_inputs as mi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Independent brute force (pure Python)
# ---------------------------------------------------------------------------

def _py_value(x, dtype):
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", int(np.asarray(x, np.float16).view(np.uint16))))[0]
    return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]


def _py_row(inp, b, j):
    """Row j of sequence b as a Python list of 576 floats."""
    if inp.paged:
        p = int(inp.block_table[b][j // inp.page_block_size])
        raw = inp.pool[p][j % inp.page_block_size][0]
        return [_py_value(v, inp.dtype) for v in raw]
    lat = [_py_value(v, inp.dtype) for v in inp.kv_latent[b][j][0]]
    pe = [_py_value(v, inp.dtype) for v in inp.k_pe[b][j][0]]
    return lat + pe


def brute_force(inp, b, h):
    """(out list[512], lse) for one (sequence, head), straight from the definition."""
    L = int(inp.cache_seqlens[b])
    q = [_py_value(v, inp.dtype) for v in inp.q_nope[b][h]] + [_py_value(v, inp.dtype) for v in inp.q_pe[b][h]]
    if L == 0:
        return [0.0] * 512, -math.inf
    rows = [_py_row(inp, b, j) for j in range(L)]
    z = [inp.softmax_scale * math.fsum(qi * ki for qi, ki in zip(q, row)) for row in rows]
    # p_j = 1 / Σ_i exp(z_i - z_j): no running max, a different route to the same number.
    p = [1.0 / math.fsum(math.exp(zi - zj) for zi in z) for zj in z]
    lse = z[0] + math.log(math.fsum(math.exp(zi - z[0]) for zi in z))
    out = [math.fsum(p[j] * rows[j][d] for j in range(L)) for d in range(512)]
    return out, lse


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(same_inf, 0.0, np.abs(a - b))
    lim = atol + rtol * np.where(same_inf, 0.0, np.abs(b))
    bad = ~(err <= lim)
    assert not bad.any(), f"{what}: max err {np.nanmax(np.where(same_inf, 0, err)):.3e}, {int(bad.sum())} bad"


def tiny_cases():
    """Tiny workloads for the brute force: lengths 1, 2, 63, 64, 65, 130; both layouts."""
    cases = [
        mi.make_contiguous(2, 3, 130, [1, 130], "f16", seed=11),
        mi.make_contiguous(2, 2, 65, [63, 65], "f16", seed=12),
        mi.make_paged(2, 2, [64, 2], "bf16", seed=13, page_block_size=32, spare_pages=3),
        mi.make_paged(1, 4, [70], "bf16", seed=14, page_block_size=64),
    ]
    return cases


def pin_bruteforce(orc, cases=None, heads_per_case=2):
    for inp in (cases or tiny_cases()):
        out, lse = orc.mla_decode_ref(inp)
        for b in range(inp.batch):
            for h in range(min(inp.heads, heads_per_case)):
                bo, bl = brute_force(inp, b, h)
                _close(out[b, h], bo, 1e-11, 1e-12, "brute force out")
                _close(lse[b, h], bl, 1e-12, 1e-12, "brute force lse")


def pin_seqlen1(orc):
    """L = 1: out is exactly V_0 and lse is exactly z_0."""
    for dt in ("f16", "bf16"):
        inp = mi.make_contiguous(2, 4, 8, [1, 1], dt, seed=21)
        out, lse = orc.mla_decode_ref(inp)
        for b in range(2):
            v0 = orc.to_f64(inp.kv_latent[b, 0, 0], dt)
            assert np.array_equal(out[b], np.broadcast_to(v0, out[b].shape)), "seqlen-1 out != V_0"
            for h in range(4):
                _, z0 = brute_force(inp, b, h)
                _close(lse[b, h], z0, 1e-13, 1e-14, "seqlen-1 lse")


def pin_uniform(orc):
    """q_nope = 0 and identical RoPE rows: every score equals z, so out = mean V, lse = z + ln L."""
    L = 37
    inp = mi.make_contiguous(1, 3, L, [L], "f16", seed=22)
    inp.q_nope[:] = 0
    inp.k_pe[0, :, 0, :] = inp.k_pe[0, 0, 0, :]
    out, lse = orc.mla_decode_ref(inp)
    V = inp.kv_latent[0, :L, 0, :].astype(np.float64)
    kpe = inp.k_pe[0, 0, 0, :].astype(np.float64)
    for h in range(3):
        z = inp.softmax_scale * math.fsum(float(a) * float(b) for a, b in
                                          zip(inp.q_pe[0, h].astype(np.float64), kpe))
        _close(out[0, h], V.mean(axis=0), 1e-12, 1e-13, "uniform out")
        _close(lse[0, h], z + math.log(L), 1e-13, 1e-13, "uniform lse")


def pin_onehot(orc):
    """A dominant key j*: out = V_{j*} up to e^-100, lse = z_{j*} up to e^-100."""
    L = 50
    inp = mi.make_contiguous(1, 2, L, [L], "f16", seed=23)
    inp.q_nope[:] = 0
    inp.q_pe[:] = np.abs(inp.q_pe).astype(np.float16) + np.float16(1.0)
    inp.k_pe[:] = 0
    jstar = 17
    inp.k_pe[0, jstar, 0, :] = np.float16(64.0)
    out, lse = orc.mla_decode_ref(inp)
    for h in range(2):
        zstar = inp.softmax_scale * 64.0 * float(inp.q_pe[0, h].astype(np.float64).sum())
        assert zstar > 100
        _close(out[0, h], inp.kv_latent[0, jstar, 0].astype(np.float64), 1e-12, 1e-12, "one-hot out")
        _close(lse[0, h], zstar, 1e-13, 1e-12, "one-hot lse")


def pin_shift(orc):
    """Adding the same amount to every score of a head leaves out unchanged and shifts lse."""
    L = 40
    base = mi.make_contiguous(1, 3, L, [L], "f16", seed=24)
    shifted = mi.make_contiguous(1, 3, L, [L], "f16", seed=24)
    base.k_pe[0, :, 0, 0] = 0
    shifted.k_pe[0, :, 0, 0] = np.float16(4.0)      # adds 4 * q_pe[h, 0] * scale to all scores
    o0, l0 = orc.mla_decode_ref(base)
    o1, l1 = orc.mla_decode_ref(shifted)
    _close(o1, o0, 1e-11, 1e-12, "shift out")
    delta = 4.0 * base.q_pe[0, :, 0].astype(np.float64) * base.softmax_scale
    _close(l1[0], l0[0] + delta, 1e-12, 1e-12, "shift lse")


def pin_normalisation(orc):
    """Σ_j exp(z_j - lse) = 1 with z from the brute-force dot products."""
    inp = mi.make_paged(1, 2, [90], "bf16", seed=25, page_block_size=32)
    _, lse = orc.mla_decode_ref(inp)
    for h in range(2):
        q = [_py_value(v, "bf16") for v in inp.q_nope[0][h]] + [_py_value(v, "bf16") for v in inp.q_pe[0][h]]
        z = [inp.softmax_scale * math.fsum(a * b for a, b in zip(q, _py_row(inp, 0, j))) for j in range(90)]
        s = math.fsum(math.exp(zj - float(lse[0, h])) for zj in z)
        assert abs(s - 1.0) < 1e-12, f"normalisation {s}"


def pin_row_permutation(orc):
    """Permuting the order of the cache rows does not change out or lse."""
    L = 77
    inp = mi.make_contiguous(1, 4, L, [L], "f16", seed=26)
    o0, l0 = orc.mla_decode_ref(inp)
    perm = np.random.default_rng(5).permutation(L)
    inp.kv_latent[0, :L] = inp.kv_latent[0, perm]
    inp.k_pe[0, :L] = inp.k_pe[0, perm]
    o1, l1 = orc.mla_decode_ref(inp)
    _close(o1, o0, 1e-12, 1e-13, "row permutation out")
    _close(l1, l0, 1e-13, 1e-13, "row permutation lse")


def pin_page_permutation(orc):
    """Moving physical pages and rewriting block_table gives identical results."""
    inp = mi.make_paged(2, 3, [100, 33], "bf16", seed=27, page_block_size=32, spare_pages=2)
    o0, l0 = orc.mla_decode_ref(inp)
    P = inp.pool.shape[0]
    perm = np.random.default_rng(6).permutation(P)          # new slot of old page p is perm[p]
    pool2 = np.empty_like(inp.pool)
    pool2[perm] = inp.pool
    table2 = np.where(inp.block_table >= 0, perm[np.maximum(inp.block_table, 0)], -1).astype(np.int32)
    inp.pool, inp.block_table = pool2, table2
    o1, l1 = orc.mla_decode_ref(inp)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1), "page permutation changed the result"


def pin_split_invariance(orc):
    """Split-KV partials + combine equal the direct form for any number of splits."""
    inp = mi.make_paged(3, 3, [300, 64, 1], "bf16", seed=28, page_block_size=64)
    o0, l0 = orc.mla_decode_ref(inp)
    for s in (1, 2, 3, 4, 7):
        o1, l1 = orc.mla_decode_split_ref(inp, s)
        _close(o1, o0, 1e-11, 1e-12, f"split {s} out")
        _close(l1, l0, 1e-12, 1e-12, f"split {s} lse")
    o2, l2 = orc.mla_decode_split_ref(inp, [5, 1, 3])
    _close(o2, o0, 1e-11, 1e-12, "per-sequence splits out")
    _close(l2, l0, 1e-12, 1e-12, "per-sequence splits lse")


def pin_split_ranges(orc):
    """Ranges cover [0, L) once, in order, with sizes differing by at most one
    block; and three cases worked by hand from the rule (nb = ceil(L / 64)
    blocks, split k takes floor(nb / s) of them plus one while k < nb mod s):
    L = 300, s = 2 has 5 blocks, 3 then 2; L = 65, s = 3 has 2 blocks, one
    each for the first two splits and none for the third; L = 4096, s = 4
    gives 16 blocks to each."""
    assert orc.split_ranges(300, 2) == [(0, 192), (192, 300)]
    assert orc.split_ranges(65, 3) == [(0, 64), (64, 65), (65, 65)]
    assert orc.split_ranges(4096, 4) == [(0, 1024), (1024, 2048), (2048, 3072), (3072, 4096)]
    for L in (0, 1, 63, 64, 65, 300, 4096, 131072):
        for s in (1, 2, 3, 4, 7, 64, 128):
            r = orc.split_ranges(L, s)
            assert len(r) == s
            pos = 0
            for a, b in r:
                assert a == pos and b >= a, (L, s, r)
                pos = b
            assert pos == L
            nblk = [-(-(b - a) // 64) if b > a else 0 for a, b in r]
            full = [(b - a + 63) // 64 for a, b in r]
            assert max(full) - min(full) <= 1 or L % 64 != 0, (L, s)
            assert nblk == sorted(nblk, reverse=True) or L % 64 != 0


def pin_multi_token(orc):
    """Three query tokens per sequence: token t's rows (t*H .. t*H + H - 1) give
    exactly plain one-token decode over the first L - (2 - t) cache rows
    (lengths written out by hand below), in the direct and the split form."""
    H = 4
    lens = [40, 3, 1, 0]
    inp = mi.make_contiguous(len(lens), H, 40, lens, "f16", seed=33, seqlen_q=3)
    o3, l3 = orc.mla_decode_ref(inp)
    visible = {0: [38, 1, 0, 0], 1: [39, 2, 0, 0], 2: [40, 3, 1, 0]}   # per token t, per sequence
    for t, vis in visible.items():
        one = mi.MlaInputs(dtype="f16", q_nope=inp.q_nope[:, t * H:(t + 1) * H].copy(),
                           q_pe=inp.q_pe[:, t * H:(t + 1) * H].copy(),
                           cache_seqlens=np.array(vis, np.int32), softmax_scale=inp.softmax_scale,
                           kv_latent=inp.kv_latent, k_pe=inp.k_pe)
        o1, l1 = orc.mla_decode_ref(one)
        assert np.array_equal(o3[:, t * H:(t + 1) * H], o1), t
        assert np.array_equal(l3[:, t * H:(t + 1) * H], l1), t
    for s in (1, 2, 5):
        os_, ls_ = orc.mla_decode_split_ref(inp, s)
        _close(os_, o3, 1e-11, 1e-12, f"multi-token split {s} out")
        both = np.isneginf(ls_) & np.isneginf(l3)
        _close(np.where(both, 0, ls_), np.where(both, 0, l3), 1e-12, 1e-12, f"multi-token split {s} lse")


def pin_batch_independence(orc):
    """Changing one sequence's cache leaves every other sequence bit-identical."""
    inp = mi.make_contiguous(3, 2, 50, [50, 20, 35], "f16", seed=29)
    o0, l0 = orc.mla_decode_ref(inp)
    inp.kv_latent[1] = (inp.kv_latent[1].astype(np.float32) * 2 + 1).astype(np.float16)
    o1, l1 = orc.mla_decode_ref(inp)
    for b in (0, 2):
        assert np.array_equal(o0[b], o1[b]) and np.array_equal(l0[b], l1[b])
    assert not np.array_equal(o0[1], o1[1])


def _golden_inputs(case):
    """Build an input object from a sparse golden-fixture description."""
    dt = case["dtype"]
    B, H, L = 1, case["heads"], len(case["rows"])
    inp = mi.make_contiguous(B, H, max(L, 1), [L], dt, seed=0, scale=case["softmax_scale"])
    inp.q_nope[:] = 0
    inp.q_pe[:] = 0
    inp.kv_latent[:] = 0
    inp.k_pe[:] = 0
    for h, entries in enumerate(case["q"]):
        for d, v in entries:
            if d < 512:
                inp.q_nope[0, h, d] = v
            else:
                inp.q_pe[0, h, d - 512] = v
    for j, entries in enumerate(case["rows"]):
        for d, v in entries:
            if d < 512:
                inp.kv_latent[0, j, 0, d] = v
            else:
                inp.k_pe[0, j, 0, d - 512] = v
    if case.get("paged"):
        rows = np.concatenate([inp.kv_latent[0, :L, 0], inp.k_pe[0, :L, 0]], axis=1)
        page = case["page_block_size"]
        table = case["block_table"]
        npages = max(table) + 1
        pool = np.zeros((npages, page, 1, 576), dtype=np.float16)
        for j in range(L):
            pool[table[j // page], j % page, 0] = rows[j]
        inp.pool = pool
        inp.block_table = np.array([table], dtype=np.int32)
        inp.page_block_size = page
        inp.kv_latent = inp.k_pe = None
    return inp


def pin_golden(orc):
    """Hand-derived closed-form fixtures in tests/golden/closed_forms.json."""
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        inp = _golden_inputs(case)
        if case.get("splits"):
            out, lse = orc.mla_decode_split_ref(inp, case["splits"], block_rows=case.get("block_rows", 64))
        else:
            out, lse = orc.mla_decode_ref(inp)
        for h, exp in enumerate(case["expect"]):
            _close(lse[0, h], exp["lse"], 1e-14, 1e-14, f"golden {case['name']} lse")
            want = np.zeros(512)
            for d, v in exp["out"]:
                want[d] = v
            _close(out[0, h], want, 1e-14, 1e-15, f"golden {case['name']} out")
    for case in data["combine_cases"]:
        parts = [(np.array(o, dtype=np.float64)[None, :], np.array([l], dtype=np.float64))
                 for o, l in zip(case["partial_out"], case["partial_lse2"])]
        out, lse = orc.combine(parts)
        _close(out[0], case["out"], 1e-14, 1e-15, f"golden {case['name']} out")
        _close(lse[0], case["lse"], 1e-14, 1e-15, f"golden {case['name']} lse")


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) cache with a per-tensor scale
# ---------------------------------------------------------------------------

# Bytes decoded by hand from the format (sign | 4 exponent bits, bias 7 | 3
# mantissa bits; exponent 0 subnormal with 2^-6 * m/8; no infinities).
E4M3_TABLE = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x02, 2.0 ** -8), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x0F, 1.875 * 2.0 ** -6), (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3C, 1.5), (0x40, 2.0),
    (0x48, 4.0), (0x70, 128.0), (0x77, 240.0), (0x78, 256.0), (0x7E, 448.0), (0x80, -0.0),
    (0xB8, -1.0), (0xBC, -1.5), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
]


def pin_fp8_decode(orc):
    """Hand-decoded E4M3 bytes; 0x7F and 0xFF are NaN."""
    codes = np.array([c for c, _ in E4M3_TABLE], dtype=np.uint8)
    vals = orc.to_f64(codes, "fp8")
    for (c, v), got in zip(E4M3_TABLE, vals):
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), f"E4M3 0x{c:02X}: {got} != {v}"
    assert np.isnan(orc.to_f64(np.array([0x7F, 0xFF], dtype=np.uint8), "fp8")).all()


def _fp8_twin(inp8, dtype):
    """The 16-bit problem whose cache holds exactly the fp8 cache's values
    (kv_scale a power of two, so every value is an fp16 / bf16 number): the
    values come from the generator's E4M3 table, not from the oracle."""
    import copy
    mags = mi._e4m3_magnitudes()
    def val(b):
        b = np.asarray(b, dtype=np.int64)
        v = mags[np.minimum(b & 0x7F, 126)] * np.where(b & 0x80, -1.0, 1.0)
        return mi.cast_storage((v * inp8.kv_scale).astype(np.float32), dtype)
    twin = copy.copy(inp8)
    twin.kv_dtype, twin.kv_scale = "", 1.0
    if inp8.paged:
        twin.pool = val(inp8.pool)
    else:
        twin.kv_latent, twin.k_pe = val(inp8.kv_latent), val(inp8.k_pe)
    return twin


def pin_fp8_matches_16bit(orc):
    """An fp8 cache with kv_scale = 2^-3 gives exactly the result of the
    16-bit cache holding the same values, contiguous and paged."""
    for inp8 in (mi.make_contiguous(2, 3, 70, [70, 33], "f16", seed=31, kv_dtype="fp8", kv_scale=0.125),
                 mi.make_paged(2, 2, [40, 65], "bf16", seed=32, page_block_size=32, kv_dtype="fp8",
                               kv_scale=0.125)):
        twin = _fp8_twin(inp8, inp8.dtype)
        o8, l8 = orc.mla_decode_ref(inp8)
        o16, l16 = orc.mla_decode_ref(twin)
        assert np.array_equal(o8, o16) and np.array_equal(l8, l16), "fp8 cache differs from its 16-bit twin"


def pin_fp8_scale(orc):
    """kv_scale s multiplies every cache value: the same as scores scaled by s
    (softmax_scale * s) and the output times s, for a scale that is not a
    power of two."""
    inp = mi.make_contiguous(2, 3, 50, [50, 7], "f16", seed=33, kv_dtype="fp8", kv_scale=0.0123)
    o, l = orc.mla_decode_ref(inp)
    import copy
    unit = copy.copy(inp)
    unit.kv_scale = 1.0
    unit.softmax_scale = inp.softmax_scale * 0.0123
    ou, lu = orc.mla_decode_ref(unit)
    _close(o, 0.0123 * ou, 1e-12, 1e-15, "fp8 scale out")
    _close(l, lu, 1e-12, 1e-12, "fp8 scale lse")


ALL_PINS = [
    pin_fp8_decode,
    pin_fp8_matches_16bit,
    pin_fp8_scale,
    pin_golden,
    pin_seqlen1,
    pin_uniform,
    pin_onehot,
    pin_shift,
    pin_normalisation,
    pin_row_permutation,
    pin_page_permutation,
    pin_split_invariance,
    pin_split_ranges,
    pin_multi_token,
    pin_batch_independence,
    pin_bruteforce,
]
