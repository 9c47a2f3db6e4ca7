"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a textual edit of oracle/ref.py (a dropped term, a wrong sign,
index or order, a transposed operand), loaded as a separate module on the
CPU.  The real oracle is never modified."""

import os
import types

import pytest

from tests.oracle_pins import ALL_CHECKS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ref.py")

MUTANTS = {
    "nibble_order_reversed": ("(4 * np.arange(8, dtype=np.uint32))", "(28 - 4 * np.arange(8, dtype=np.uint32))"),
    "bias_dropped": ("return s * q + b", "return s * q"),
    "bias_sign": ("return s * q + b", "return s * q - b"),
    "scale_bias_swapped": ("s = np.repeat(bf16_to_f64(scales)", "s = np.repeat(bf16_to_f64(biases)"),
    "group_of_32": ("GROUP = 64", "GROUP = 32"),
    "tie_to_higher_index": ("np.lexsort((np.arange(e), -l[r]))", "np.lexsort((-np.arange(e), -l[r]))"),
    "softmax_unnormalised": ("p = ex / ex.sum()", "p = ex"),
    "renorm_dropped": ("w[r] = w[r] / w[r].sum()", "w[r] = w[r]"),
    "sigmoid_sign": ("p = 1.0 / (1.0 + np.exp(-l[r]))", "p = 1.0 / (1.0 + np.exp(l[r]))"),
    "union_rows_descending": ("        for r in range(k):\n            hits", "        for r in reversed(range(k)):\n            hits"),
    "swiglu_gate_up_swapped": ("return silu(a[..., :i]) * a[..., i:]", "return silu(a[..., i:]) * a[..., :i]"),
    "combine_slot_mismatch": ("y[r] = y[r] + w[r, s] * partial[r, s]", "y[r] = y[r] + w[r, topk - 1 - s] * partial[r, s]"),
    "shared_gate_dropped": ("y[r] = y[r] + gate[r] * shared[r]", "y[r] = y[r] + shared[r]"),
    "gdn_update_transposed": ("np.outer(delta, kt)", "np.outer(kt, delta)"),
    "gdn_decay_dropped": ("S[h] = g[t, h] * S[h]", "S[h] = S[h]"),
    "gdn_head_interleaved": ("c = h // ratio", "c = h % hk"),
    "gdn_delta_sign": ("delta = beta[t, h] * (v[t, h] - m)", "delta = beta[t, h] * (v[t, h] + m)"),
    "gdn_beta_misplaced": ("delta = beta[t, h] * (v[t, h] - m)", "delta = beta[t, h] * v[t, h] - m"),
    "gdn_readout_before_update": ("y[t, h] = S[h] @ qt", "y[t, h] = (S[h] - np.outer(delta, kt)) @ qt"),
    "gdn_kvmem_uses_q": ("m = S[h] @ kt", "m = S[h] @ qt"),
    "rollback_off_by_one": ("else np.array(snaps[j - 1], copy=True)", "else np.array(snaps[min(j, rows - 1)], copy=True)"),
    "sample_ties_to_higher": ("out[r] = valid[z[r][valid] == best][0]", "out[r] = valid[z[r][valid] == best][-1]"),
    "sample_nan_chosen": ("valid = np.flatnonzero(~np.isnan(z[r]))", "valid = np.arange(z.shape[1])"),
    "sample_temperature_dropped": ("(l * np.float32(inv_temp))", "(l * np.float32(1.0))"),
    "sample_noise_subtracted": ("+ np.asarray(noise, dtype=np.float32)", "- np.asarray(noise, dtype=np.float32)"),
    "accept_past_mismatch": ("            n += 1\n        else:\n            break", "            n += 1"),
    "accept_end_of_answer_ignored": ("if drafts[t] == tokens[t] and (eos < 0 or drafts[t] != eos):", "if drafts[t] == tokens[t]:"),
    "accept_compares_next_row": ("if drafts[t] == tokens[t] and", "if drafts[t] == tokens[t + 1] and"),
    "emitted_without_bonus": ("+ [int(tokens[n])]", ""),
    "prefix_off_by_one": ('"prefix": n + 1', '"prefix": n'),
    "conv_taps_reversed": ("conv[t] = conv[t] + w[:, i] * X[t + i]", "conv[t] = conv[t] + w[:, 3 - i] * X[t + i]"),
    "conv_history_misaligned": ("conv[t] = conv[t] + w[:, i] * X[t + i]", "conv[t] = conv[t] + w[:, i] * X[min(t + i + 1, rows + 2)]"),
    "conv_silu_ignored": ("        conv = silu(conv)", "        conv = conv"),
    "qk_norm_without_eps": ("q = q / np.sqrt((q * q).sum(axis=-1, keepdims=True) + eps)", "q = q / np.sqrt((q * q).sum(axis=-1, keepdims=True))"),
    "k_not_normalised": ("k = k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + eps)", "k = k"),
    "decay_A_not_exponentiated": ("g = np.exp(-np.exp(np.asarray(A_log, dtype=np.float64))[None, :] *", "g = np.exp(-(np.asarray(A_log, dtype=np.float64))[None, :] *"),
    "decay_dt_bias_dropped": ("softplus(np.asarray(a, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, :]))", "softplus(np.asarray(a, dtype=np.float64)))"),
    "beta_sign": ("beta = 1.0 / (1.0 + np.exp(-np.asarray(b, dtype=np.float64)))", "beta = 1.0 / (1.0 + np.exp(np.asarray(b, dtype=np.float64)))"),
    "softplus_sign": ("return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))", "return np.maximum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))"),
    "norm_sum_not_mean": ("n = y / np.sqrt((y * y).mean(axis=-1, keepdims=True) + eps)", "n = y / np.sqrt((y * y).sum(axis=-1, keepdims=True) + eps)"),
    "norm_weight_dropped": ("return n * np.asarray(w, dtype=np.float64) * gate", "return n * gate"),
    "gate_silu_for_sigmoid": ("        gate = 1.0 / (1.0 + np.exp(-z))", "        gate = silu(z)"),
    "shared_gate_sign": ("return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))",
                         "return 1.0 / (1.0 + np.exp(np.asarray(z, dtype=np.float64)))"),
    "shared_gate_squared": ("gate = np.ones(k) if z is None else _sigmoid(z)",
                            "gate = np.ones(k) if z is None else 2.0 * _sigmoid(z) ** 2"),
    "norm_silu_sign": ("        gate = silu(z)", "        gate = -silu(z)"),
    "norm_silu_mirrored": ("        gate = silu(z)", "        gate = silu(-z)"),
    "q8_block_64": ("Q8_BLOCK = 32", "Q8_BLOCK = 64"),
    "fp16_exponent_bias": ("np.exp2((e - 15)", "np.exp2((e - 16)"),
    "fp16_subnormal_scale": ("f * 2.0 ** -24", "f * 2.0 ** -25"),
    "q8_codes_unsigned": ("q = np.asarray(qs, dtype=np.int8).astype(np.float64)",
                          "q = np.asarray(qs, dtype=np.int8).view(np.uint8).astype(np.float64)"),
    "q8_scale_block_shift": ("s = np.repeat(fp16_to_f64(d), Q8_BLOCK, axis=-1)",
                             "s = np.roll(np.repeat(fp16_to_f64(d), Q8_BLOCK, axis=-1), 1, axis=-1)"),
    "q3_big_endian_bits": ('bits = np.unpackbits(b, axis=-1, bitorder="little")',
                           'bits = np.unpackbits(b, axis=-1, bitorder="big")'),
    "q3_bit_weights_swapped": ("(trip[..., 0] | (trip[..., 1] << 1) | (trip[..., 2] << 2))",
                               "(trip[..., 1] | (trip[..., 0] << 1) | (trip[..., 2] << 2))"),
    "q3_bias_dropped": ('''    q = unpack_q3(codes).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(biases), GROUP, axis=-1)
    return s * q + b''', '''    q = unpack_q3(codes).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(biases), GROUP, axis=-1)
    return s * q'''),
}


def _load(old, new):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load(*MUTANTS[name])
    failed = []
    for check in ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # AssertionError, or a crash from a broken shape
            failed.append(check.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
