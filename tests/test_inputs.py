"""The seeded input generator: reproducible, right shapes, right structure."""
import numpy as np

import mla_inputs as mi


def test_reproducible_and_seed_sensitive():
    a = mi.make_contiguous(2, 4, 70, [70, 3], "f16", seed=5)
    b = mi.make_contiguous(2, 4, 70, [70, 3], "f16", seed=5)
    c = mi.make_contiguous(2, 4, 70, [70, 3], "f16", seed=6)
    assert np.array_equal(a.kv_latent, b.kv_latent) and np.array_equal(a.q_pe, b.q_pe)
    assert not np.array_equal(a.kv_latent, c.kv_latent)
    assert a.kv_latent.shape == (2, 70, 1, 512) and a.k_pe.shape == (2, 70, 1, 64)
    assert a.q_nope.shape == (2, 4, 512) and a.q_pe.shape == (2, 4, 64)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    bits = mi.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0.
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6
    assert back[3] == -2.5
    assert np.all(np.abs(back[:5] - x[:5]) <= np.abs(x[:5]) * 2 ** -8)


def test_normal_statistics():
    a = mi.make_contiguous(4, 8, 512, [512] * 4, "f16", seed=1)
    v = a.kv_latent.astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01


def test_paged_block_table_is_a_permutation():
    lens = [1, 64, 65, 300, 0]
    p = mi.make_paged(5, 2, lens, "bf16", seed=9, page_block_size=64, max_blocks=8)
    t = p.block_table
    used = t[t >= 0]
    assert sorted(used.tolist()) == list(range(p.pool.shape[0]))
    for b, L in enumerate(lens):
        n = -(-L // 64)
        assert (t[b, :n] >= 0).all() and (t[b, n:] == -1).all()


def test_scaled_rows_are_exact_and_counted():
    p = mi.make_paged(1, 2, [1000], "bf16", seed=2, page_block_size=64)
    before = p.pool.copy()
    chosen = mi.scale_random_rows(p, 0.01, 8.0, seed=3)
    assert chosen.shape == (1, 10) and len(set(chosen[0].tolist())) == 10
    j = int(chosen[0, 0])
    page, off = p.block_table[0, j // 64], j % 64
    f0 = (before[page, off, 0].astype(np.uint32) << 16).view(np.float32)
    f1 = (p.pool[page, off, 0].astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f1, f0 * 8)


def test_config_shapes_small():
    c0 = mi.make_config(0)
    assert c0.q_nope.shape == (2, 16, 512) and c0.kv_latent.shape == (2, 256, 1, 512)
    assert c0.dtype == "f16" and abs(c0.softmax_scale - 1 / 24) < 1e-15
    c3 = mi.make_config(3, batch_subset=2)
    assert c3.block_table.shape == (2, 256) and c3.dtype == "bf16"
    assert 1 <= c3.cache_seqlens.min() and c3.cache_seqlens.max() <= 16384


def test_e4m3_encoder_round_trip_ties_and_saturation():
    """The generator's E4M3 quantiser: every finite magnitude times the scale
    encodes to its own code; a value halfway between two codes goes to the
    even code; magnitudes beyond 448 saturate; the sign is bit 7."""
    s = 0.5
    mags = mi._e4m3_magnitudes()
    codes = mi.f32_to_e4m3_bits(mags * s, s)
    assert np.array_equal(codes, np.arange(127, dtype=np.uint8))
    assert np.array_equal(mi.f32_to_e4m3_bits(-mags[1:] * s, s), (np.arange(1, 127) | 0x80).astype(np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2 * s
    got = mi.f32_to_e4m3_bits(mids, s).astype(np.int64)
    lo = np.arange(126)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    assert (mi.f32_to_e4m3_bits(np.array([449.0, 1e6, -1e6]) * s, s) == np.array([0x7E, 0x7E, 0xFE])).all()
