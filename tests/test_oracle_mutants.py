"""Plant plausible mistakes in a copy of the oracle; the pins must catch each one.

This shows the pins are strong enough: a dropped term, a wrong sign, a wrong
index or slice, a missing scale, confused log units or an off-by-one in the
split ranges each make at least one pin fail.  Mistakes are planted only in a
private in-memory copy of the CPU oracle.
"""
import importlib.util
import os
import types

import numpy as np
import pytest

from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mla_oracle.py")

MUTANTS = {
    "drop_rope_term": ("qn @ K[:, :D_LATENT].T + qp @ K[:, D_LATENT:].T", "qn @ K[:, :D_LATENT].T"),
    "rope_sign": ("qn @ K[:, :D_LATENT].T + qp @ K[:, D_LATENT:].T", "qn @ K[:, :D_LATENT].T - qp @ K[:, D_LATENT:].T"),
    "no_scale": ("return softmax_scale * (qn", "return (qn"),
    "lse_sign": ("return m + np.log(", "return m - np.log("),
    "wrong_value_slice": ("return weighted_values(z, lse, K[:, :D_LATENT]), lse",
                          "return weighted_values(z, lse, K[:, D_ROPE:D_ROPE + D_LATENT]), lse"),
    "latent_feature_order": ("(qn @ K[:, :D_LATENT].T", "(qn[:, ::-1] @ K[:, :D_LATENT].T"),
    "page_offset": ("pool[pages, j % page_block_size, 0, :]", "pool[pages, (j + 1) % page_block_size, 0, :]"),
    "page_index": ("[b, j // page_block_size]", "[b, (j + 1) // page_block_size]"),
    "row_offset": ("kv_latent[b, :L, 0, :]", "kv_latent[b, 1:L + 1, 0, :]"),
    "bf16_decode": ("astype(np.uint32) << 16", "astype(np.uint32) << 15"),
    "combine_units": ("total * math.log(2.0)", "total"),
    "combine_anchor": ("w = np.exp2(lses - total)", "w = np.exp2(lses - Ms)"),
    "split_remainder": ("1 if k < rem else 0", "1 if k <= rem else 0"),
    "partial_base": ("return o, lse / math.log(2.0)", "return o, lse"),
    "stabiliser_shift": ("np.exp(z - m[:, None]).sum(axis=1)", "np.exp(z - m[:, None] + 1.0).sum(axis=1)"),
    "weights_not_normalised": ("np.exp(z - lse[:, None]) @ V", "np.exp(z) @ V"),
    "causal_direction": ("max(int(L), 0) - (seqlen_q - 1 - t)", "max(int(L), 0) - t"),
    "causal_offset": ("max(int(L), 0) - (seqlen_q - 1 - t)", "max(int(L), 0) - (seqlen_q - t)"),
    "token_major_rows": ("hsel // hpt == t", "hsel % sq == t"),
    "fp8_bias": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "fp8_subnormal": ("m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    "fp8_mantissa": ("(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    "fp8_no_scale": ('return rows * kv_scale if dtype == "fp8" else rows', "return rows"),
    "fp8_sign_bit": ("np.where(b & 0x80, -1.0, 1.0)", "np.where(b & 0x40, -1.0, 1.0)"),
    "fp8_nan_finite": ("mag = np.where((e == 15) & (b & 0x7 == 7), np.nan, mag)", "mag = mag"),
    "fp8_exponent_field": ("e = (b >> 3) & 0xF", "e = (b >> 4) & 0xF"),
    "split_block_rows": ("SPLIT_BLOCK_ROWS = 64", "SPLIT_BLOCK_ROWS = 32"),
    "empty_lse_zero": ("        return np.full(H, -np.inf)", "        return np.zeros(H)"),
    "empty_out_nonzero": ("    out[empty] = 0.0\n", "    out[empty] = 1.0\n"),
    "combine_weight_base": ("w = np.exp2(lses - total)", "w = np.exp(lses - total)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_PINS:
            try:
                pin(mod)
            except (AssertionError, IndexError, ValueError) as e:
                caught.append(pin.__name__)
                break
    assert caught, f"mutant {name} passed every pin"
