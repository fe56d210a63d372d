"""Pins of the oracle's decoupled rotary branch (CPU only).

rope_rotate is pinned to RoFormer's defining properties: a pair at position p turns by p * theta_i
(closed form on one pair), scores of rotated vectors depend only on the position difference, the
norm is kept, and position 0 is the identity. attend_decode_rope is pinned to the contiguous decode
when the rotary query is zero, to torch SDPA on concatenated content + rotary keys under an exact
full-rank codec, and to invariance under a common shift of every position.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import lla_oracle as O


def test_rotation_closed_form_and_identity():
    x = np.array([1.0, 0.0, 0.0, 2.0])
    base = 100.0
    y = O.rope_rotate(x, 3, base)
    th1 = base ** (-2.0 / 4)
    np.testing.assert_allclose(y, [math.cos(3), math.sin(3), -2 * math.sin(3 * th1),
                                   2 * math.cos(3 * th1)], atol=1e-15)
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 64))
    np.testing.assert_array_equal(O.rope_rotate(v, 0), v)
    np.testing.assert_allclose(np.linalg.norm(O.rope_rotate(v, 12345), axis=1),
                               np.linalg.norm(v, axis=1), rtol=1e-13)


def test_scores_depend_only_on_the_position_difference():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    s1 = O.rope_rotate(q, 1000) @ O.rope_rotate(k, 993)
    s2 = O.rope_rotate(q, 262151) @ O.rope_rotate(k, 262144)
    assert abs(s1 - s2) < 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))
    assert abs(s1 - O.rope_rotate(q, 7) @ k) < 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))


def _case(rng, B=2, H=2, d=4, T=2, r=8, n_max=10, dr=4):
    return dict(q=rng.standard_normal((B, H, d)), qr=rng.standard_normal((B, H, dr)),
                zk=rng.standard_normal((B, H, n_max, r)), zv=rng.standard_normal((B, H, n_max, r)),
                kr=rng.standard_normal((B, n_max, dr)), Wk=rng.standard_normal((T, H, d, r)),
                Wv=rng.standard_normal((T, H, d, r)), mu_k=rng.standard_normal((H, T * d)),
                mu_v=rng.standard_normal((H, T * d)), ks=rng.standard_normal((B, H, d)),
                vs=rng.standard_normal((B, H, d)), krs=rng.standard_normal((B, dr)))


def test_zero_rotary_query_is_the_content_decode():
    rng = np.random.default_rng(3)
    c = _case(rng)
    lens = np.array([10, 4])
    o, lse = O.attend_decode_rope(c["q"], 0 * c["qr"], c["zk"], c["zv"], c["kr"], c["Wk"], c["Wv"],
                                  1, lens, c["mu_k"], c["mu_v"], c["ks"], c["vs"], c["krs"],
                                  scale=0.3)
    o2, lse2 = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 1, lens, c["mu_k"],
                               c["mu_v"], c["ks"], c["vs"], scale=0.3)
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-12, rtol=0)


def test_full_rank_codec_equals_sdpa_on_concatenated_keys():
    rng = np.random.default_rng(4)
    B, H, d, T, n, dr = 2, 2, 4, 2, 9, 6
    r = T * d
    E = np.zeros((H, r, r))
    W = np.zeros((T, H, d, r))
    for h in range(H):
        V, _ = np.linalg.qr(rng.standard_normal((r, r)))
        E[h] = V.T
        for t in range(T):
            W[t, h] = V[t * d:(t + 1) * d]
    xk = rng.standard_normal((B, n, T, H, d))
    xv = rng.standard_normal((B, n, T, H, d))
    zk, zv = O.encode_into_cache(np.zeros((B, H, n, r)), np.zeros((B, H, n, r)), xk, xv, E, E,
                                 np.zeros(B, dtype=np.int64))
    kr_raw = rng.standard_normal((B, n, dr))
    kr = O.rope_rotate(kr_raw, np.arange(n)[None, :])  # cached already rotated at slot i
    q, qr = rng.standard_normal((B, H, d)), rng.standard_normal((B, H, dr))
    lens = np.array([9, 5])
    t = 1
    o, _ = O.attend_decode_rope(q, qr, zk, zv, kr, W, W, t, lens, base=10000.0)
    for b in range(B):
        m = int(lens[b])
        for h in range(H):
            K = np.concatenate([xk[b, :m, t, h], O.rope_rotate(kr_raw[b, :m], np.arange(m))], axis=1)
            qq = np.concatenate([q[b, h], O.rope_rotate(qr[b, h], m)])
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(qq)[None, None, None], torch.from_numpy(K)[None, None],
                torch.from_numpy(xv[b, :m, t, h])[None, None])[0, 0, 0].numpy()
            np.testing.assert_allclose(o[b, h], ref, atol=1e-10, rtol=0)


def test_common_position_shift_changes_nothing():
    """Rotating every cached rotary key and the query by the same extra offset leaves the scores
    and so the output unchanged (only position differences matter)."""
    rng = np.random.default_rng(5)
    c = _case(rng)
    lens = np.array([10, 7])
    raw = rng.standard_normal(c["kr"].shape)
    kr0 = O.rope_rotate(raw, np.arange(10)[None, :])
    a = O.attend_decode_rope(c["q"], c["qr"], c["zk"], c["zv"], kr0, c["Wk"], c["Wv"], 0, lens,
                             c["mu_k"], c["mu_v"], c["ks"], c["vs"], c["krs"])
    # shift: keys at i + 50; the query (at N_b) is rotated 50 more by pre-rotating q_rope
    kr1 = O.rope_rotate(raw, np.arange(10)[None, :] + 50)
    qr1 = O.rope_rotate(c["qr"], 50)
    krs1 = O.rope_rotate(c["krs"], 50)
    b_ = O.attend_decode_rope(c["q"], qr1, c["zk"], c["zv"], kr1, c["Wk"], c["Wv"], 0, lens,
                              c["mu_k"], c["mu_v"], c["ks"], c["vs"], krs1)
    np.testing.assert_allclose(a[0], b_[0], atol=1e-11, rtol=0)
    np.testing.assert_allclose(a[1], b_[1], atol=1e-11, rtol=0)


def test_prefill_zero_rotary_query_is_the_content_prefill():
    rng = np.random.default_rng(6)
    B, C, H, d, T, r, n, dr = 2, 3, 2, 4, 2, 6, 9, 4
    zk, zv = rng.standard_normal((B, H, n, r)), rng.standard_normal((B, H, n, r))
    Wk, Wv = rng.standard_normal((T, H, d, r)), rng.standard_normal((T, H, d, r))
    q = rng.standard_normal((B, C, H, d))
    kr = rng.standard_normal((B, n, dr))
    ctx = np.array([5, 0])
    a = O.attend_prefill_rope(q, np.zeros((B, C, H, dr)), zk, zv, kr, Wk, Wv, 1, ctx, scale=0.4)
    b_ = O.attend_prefill(q, zk, zv, Wk, Wv, 1, ctx, scale=0.4)
    np.testing.assert_allclose(a, b_, atol=1e-12, rtol=0)


def test_prefill_full_rank_codec_equals_causal_sdpa_on_concatenated_keys():
    rng = np.random.default_rng(7)
    B, C, H, d, T, dr = 2, 4, 2, 4, 2, 6
    r = T * d
    ctx = np.array([3, 0])
    n = 8
    E = np.zeros((H, r, r))
    W = np.zeros((T, H, d, r))
    for h in range(H):
        V, _ = np.linalg.qr(rng.standard_normal((r, r)))
        E[h] = V.T
        for t in range(T):
            W[t, h] = V[t * d:(t + 1) * d]
    xk = rng.standard_normal((B, n, T, H, d))
    xv = rng.standard_normal((B, n, T, H, d))
    zk, zv = O.encode_into_cache(np.zeros((B, H, n, r)), np.zeros((B, H, n, r)), xk, xv, E, E,
                                 np.zeros(B, dtype=np.int64))
    kr_raw = rng.standard_normal((B, n, dr))
    kr = O.rope_rotate(kr_raw, np.arange(n)[None, :])
    q, qr = rng.standard_normal((B, C, H, d)), rng.standard_normal((B, C, H, dr))
    t = 1
    o = O.attend_prefill_rope(q, qr, zk, zv, kr, W, W, t, ctx)
    for b in range(B):
        m = int(ctx[b]) + C
        for h in range(H):
            K = np.concatenate([xk[b, :m, t, h], O.rope_rotate(kr_raw[b, :m], np.arange(m))], axis=1)
            pos = int(ctx[b]) + np.arange(C)
            Q = np.concatenate([q[b, :, h], O.rope_rotate(qr[b, :, h], pos)], axis=1)
            mask = np.arange(m)[None, :] <= pos[:, None]
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None],
                torch.from_numpy(xv[b, :m, t, h])[None, None],
                attn_mask=torch.from_numpy(mask)[None, None])[0, 0].numpy()
            np.testing.assert_allclose(o[b, :, h], ref, atol=1e-10, rtol=0)
