"""Planted mistakes in the oracle (CPU only): each must be caught by at least one pin.

Every mutant replaces one oracle function with a plausible wrong version (a dropped term, a wrong
sign, a wrong index or a transposed operand). The pins are re-run with the mutant patched in, and
the test passes only if some pin fails. The oracle itself is never modified on disk.
"""
import math

import numpy as np
import pytest

from oracle import lla_oracle as O
import tests.test_oracle_pins as P
import tests.test_oracle_gather as G
import tests.test_oracle_q8 as Q
import tests.test_oracle_rope as R


def _encode_no_centre(x_stack, E, mu=None):
    return np.asarray(x_stack, np.float64) @ np.asarray(E, np.float64).T


def _encode_plus_mu(x_stack, E, mu=None):
    x = np.asarray(x_stack, np.float64)
    if mu is not None:
        x = x + mu
    return x @ np.asarray(E, np.float64).T


def _reconstruct_no_mu(z, W_t, mu_t=None):
    return np.asarray(z, np.float64) @ np.asarray(W_t, np.float64).T


def _softmax_no_scale(q, K, V, scale):
    return _orig["softmax_attention"](q, K, V, 1.0)


def _softmax_sqrt_scale(q, K, V, scale):
    return _orig["softmax_attention"](q, K, V, math.sqrt(scale))


def _softmax_lse_no_max(q, K, V, scale):
    o, lse = _orig["softmax_attention"](q, K, V, scale)
    if K.shape[0] == 0:
        return o, lse
    return o, lse - float(np.max(scale * (np.asarray(K) @ np.asarray(q))))


def _softmax_drop_last_key(q, K, V, scale):
    return _orig["softmax_attention"](q, np.asarray(K)[:-1], np.asarray(V)[:-1], scale)


def _loop_slices_wrong_loop(variant, Wk, Wv, mu_k, mu_v, t, h, H, d):
    T = Wk.shape[0]
    return _orig["_loop_slices"](variant, Wk, Wv, mu_k, mu_v, (t + 1) % T, h, H, d)


def _loop_slices_wrong_head(variant, Wk, Wv, mu_k, mu_v, t, h, H, d):
    return _orig["_loop_slices"](variant, Wk, Wv, mu_k, mu_v, t, (h + 1) % H, H, d)


def _loop_slices_2d_head_major(variant, Wk, Wv, mu_k, mu_v, t, h, H, d):
    if variant != "2d":
        return _orig["_loop_slices"](variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
    wk, wv, _, _ = _orig["_loop_slices"](variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
    T = Wk.shape[0]
    base = h * T * d + t * d          # (head, loop, channel) order instead of (loop, head, channel)
    muk = None if mu_k is None else mu_k[base:base + d]
    muv = None if mu_v is None else mu_v[base:base + d]
    return wk, wv, muk, muv


def _gather_drop_last(q, zk, zv, Wk, Wv, t, slots, counts=None, **kw):
    slots = np.asarray(slots)
    c = np.full(slots.shape[0], slots.shape[1]) if counts is None else np.asarray(counts)
    return _orig["attend_decode_gather"](q, zk, zv, Wk, Wv, t, slots, np.maximum(c - 1, 0), **kw)


def _gather_dedup(q, zk, zv, Wk, Wv, t, slots, counts=None, **kw):
    slots = np.asarray(slots).copy()
    for b in range(slots.shape[0]):
        seen = set()
        for j in range(slots.shape[1]):
            if int(slots[b, j]) in seen:
                slots[b, j] = -1
            seen.add(int(slots[b, j]))
    return _orig["attend_decode_gather"](q, zk, zv, Wk, Wv, t, slots, counts, **kw)


def _gather_wraps_out_of_range(q, zk, zv, Wk, Wv, t, slots, counts=None, variant="per_head", **kw):
    n_max = np.asarray(zk).shape[2 if variant == "per_head" else 1]
    return _orig["attend_decode_gather"](q, zk, zv, Wk, Wv, t, np.asarray(slots) % n_max, counts,
                                         variant=variant, **kw)


def _e4m3_truncates(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6, 8)
    step = 2.0 ** (e - 3)
    r = np.floor(a / step) * step
    return np.copysign(np.where(r > 448, np.nan, r), v)


def _e4m3_bias8(v):
    # the exponent bias of the other FP8 E4M3 family (largest finite 240)
    r = _orig["e4m3_round"](np.asarray(v, np.float64) * 2.0) / 2.0
    return np.where(np.abs(r) > 240, np.nan, r)


def _quantize_scale_for_240(z):
    # scale sized for the other family's largest finite value (240) instead of 448
    z32 = np.asarray(z, np.float32)
    s = (np.max(np.abs(z32), axis=-1) / np.float32(240.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    codes = O.e4m3_round((z32 / safe[..., None]).astype(np.float32).astype(np.float64))
    return np.where((s > 0)[..., None], codes, 0.0), s.astype(np.float64)


def _int8_scale_for_128(z):
    z32 = np.asarray(z, np.float32)
    s = (np.max(np.abs(z32), axis=-1) / np.float32(128.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint((z32 / safe[..., None]).astype(np.float64)), -127, 127)
    return np.where((s > 0)[..., None], codes, 0.0), s.astype(np.float64)


def _int8_rounds_half_up(z):
    z32 = np.asarray(z, np.float32)
    s = (np.max(np.abs(z32), axis=-1) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.floor((z32 / safe[..., None]).astype(np.float64) + 0.5), -127, 127)
    return np.where((s > 0)[..., None], codes, 0.0), s.astype(np.float64)


def _int8_truncates(z):
    z32 = np.asarray(z, np.float32)
    s = (np.max(np.abs(z32), axis=-1) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.trunc((z32 / safe[..., None]).astype(np.float64)), -127, 127)
    return np.where((s > 0)[..., None], codes, 0.0), s.astype(np.float64)


def _rope_half_split(x, pos, base=10000.0):
    # pairs (i, i + d/2) instead of RoFormer's (2i, 2i + 1)
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.empty(d, dtype=int)
    perm[0::2], perm[1::2] = np.arange(d // 2), np.arange(d // 2) + d // 2
    y = _orig["rope_rotate"](x[..., perm], pos, base)
    out = np.empty_like(y)
    out[..., perm] = y
    return out


def _rope_decode_query_one_back(q, q_rope, zk, zv, k_rope, Wk, Wv, t, seq_lens=None, mu_k=None,
                                mu_v=None, k_self=None, v_self=None, k_rope_self=None,
                                base=10000.0, scale=None, variant="per_head"):
    return _orig["attend_decode_rope"](q, O.rope_rotate(q_rope, -1, base), zk, zv, k_rope, Wk, Wv,
                                       t, seq_lens, mu_k, mu_v, k_self, v_self, k_rope_self, base,
                                       scale, variant)


def _rope_decode_content_scale(q, q_rope, zk, zv, k_rope, Wk, Wv, t, seq_lens=None, mu_k=None,
                               mu_v=None, k_self=None, v_self=None, k_rope_self=None,
                               base=10000.0, scale=None, variant="per_head"):
    if scale is None:
        scale = 1.0 / math.sqrt(np.asarray(q).shape[-1])
    return _orig["attend_decode_rope"](q, q_rope, zk, zv, k_rope, Wk, Wv, t, seq_lens, mu_k, mu_v,
                                       k_self, v_self, k_rope_self, base, scale, variant)


def _rope_prefill_rows_at_context_start(q, q_rope, zk, zv, k_rope, Wk, Wv, t, ctx_lens,
                                        mu_k=None, mu_v=None, base=10000.0, scale=None,
                                        variant="per_head"):
    # every row's rotary query rotated at ctx instead of ctx + j: undo the extra turn of row j
    qr = np.asarray(q_rope, np.float64).copy()
    for j in range(qr.shape[1]):
        qr[:, j] = O.rope_rotate(qr[:, j], -j, base)
    return _orig["attend_prefill_rope"](q, qr, zk, zv, k_rope, Wk, Wv, t, ctx_lens, mu_k, mu_v,
                                        base, scale, variant)


_orig = {
    "encode_stack": O.encode_stack,
    "reconstruct": O.reconstruct,
    "softmax_attention": O.softmax_attention,
    "_loop_slices": O._loop_slices,
    "attend_decode_gather": O.attend_decode_gather,
    "e4m3_round": O.e4m3_round,
    "quantize_latent_rows": O.quantize_latent_rows,
    "quantize_latent_rows_int8": O.quantize_latent_rows_int8,
    "rope_rotate": O.rope_rotate,
    "attend_decode_rope": O.attend_decode_rope,
    "attend_prefill_rope": O.attend_prefill_rope,
}

MUTANTS = {
    "encode drops the centring": ("encode_stack", _encode_no_centre),
    "encode adds mu instead of subtracting": ("encode_stack", _encode_plus_mu),
    "reconstruct drops mu_t": ("reconstruct", _reconstruct_no_mu),
    "decode reads the next head's factors": ("_loop_slices", _loop_slices_wrong_head),
    "softmax ignores the scale": ("softmax_attention", _softmax_no_scale),
    "softmax uses sqrt(scale)": ("softmax_attention", _softmax_sqrt_scale),
    "lse drops the running max": ("softmax_attention", _softmax_lse_no_max),
    "attention drops the last key": ("softmax_attention", _softmax_drop_last_key),
    "decode reads loop t+1's factors": ("_loop_slices", _loop_slices_wrong_loop),
    "2d mu indexed head-major": ("_loop_slices", _loop_slices_2d_head_major),
    "gather drops the last listed slot": ("attend_decode_gather", _gather_drop_last),
    "gather attends a repeated slot once": ("attend_decode_gather", _gather_dedup),
    "gather wraps out-of-range slots": ("attend_decode_gather", _gather_wraps_out_of_range),
    "e4m3 truncates instead of rounding": ("e4m3_round", _e4m3_truncates),
    "e4m3 uses exponent bias 8": ("e4m3_round", _e4m3_bias8),
    "quantiser scales for 240 instead of 448": ("quantize_latent_rows", _quantize_scale_for_240),
    "int8 quantiser scales for 128": ("quantize_latent_rows_int8", _int8_scale_for_128),
    "int8 quantiser rounds halves up": ("quantize_latent_rows_int8", _int8_rounds_half_up),
    "int8 quantiser truncates": ("quantize_latent_rows_int8", _int8_truncates),
    "rope pairs channels i and i + d/2": ("rope_rotate", _rope_half_split),
    "rope query rotated one position back": ("attend_decode_rope", _rope_decode_query_one_back),
    "rope decode scales by the content width only": ("attend_decode_rope", _rope_decode_content_scale),
    "rope prefill rows rotated at the chunk start": ("attend_prefill_rope", _rope_prefill_rows_at_context_start),
}

PINS = [
    lambda: P.test_full_rank_identity_per_head(True, True),
    lambda: P.test_full_rank_identity_per_head(False, False),
    P.test_full_rank_identity_2d,
    P.test_final_loop_reuse_special_case,
    P.test_zero_query_gives_mean_value,
    P.test_sharp_query_selects_best_key,
    P.test_empty_context_and_length_clamp,
    P.test_prefill_full_rank_identity_causal_offset,
    P.test_brute_force_tiny,
    G.test_full_rank_codec_equals_sdpa_on_kept_tokens,
    G.test_brute_force_tiny_with_duplicates_and_skips,
    G.test_empty_lists,
    Q.test_every_e4m3_value_rounds_to_itself,
    Q.test_rounding_matches_torch_float8_e4m3fn,
    Q.test_quantized_rows_bound_and_extremes,
    Q.test_int8_rows_extremes_bound_and_symmetry,
    Q.test_int8_integer_rows_and_ties_to_even,
    R.test_rotation_closed_form_and_identity,
    R.test_full_rank_codec_equals_sdpa_on_concatenated_keys,
    R.test_common_position_shift_changes_nothing,
    R.test_prefill_full_rank_codec_equals_causal_sdpa_on_concatenated_keys,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin)
    assert caught, f"no pin caught the mutant: {name}"
