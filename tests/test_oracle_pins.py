"""Pins of the CPU oracle to things other than itself (CPU only).

* the paper's printed numbers (tests/golden/paper_numbers.json, each entry cited);
* a library routine: torch's scaled_dot_product_attention in float64, under factor choices that
  make the codec the identity (full-rank orthogonal factors, exact low-rank trajectories,
  final-loop reuse);
* closed forms: zero query gives the mean value, constant values give exactly that constant,
  a very sharp query selects the best key, log-sum-exp merges of disjoint token sets;
* invariances: token permutation, LLA-2D with one head against per-head LLA, prefill of one row
  against decode.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import lla_oracle as O
from decode_attention_lla_amd import synth

RNG = np.random.default_rng(12345)


def sdpa(q, K, V, mask=None):
    """torch SDPA in float64 on the CPU: q [m, d], K [n, d], V [n, dv] -> [m, dv]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0, 0].numpy()


def torch_lse(q, K, scale):
    s = torch.from_numpy(np.asarray(K, np.float64)) @ torch.from_numpy(np.asarray(q, np.float64))
    return float(torch.logsumexp(scale * s, dim=0))


def orth(n, rng):
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return Q


def full_rank_per_head(T, H, d, rng):
    """E [H, Td, Td] = V^T and W [T, H, d, Td] = row blocks of V, V orthogonal per head."""
    E = np.zeros((H, T * d, T * d))
    W = np.zeros((T, H, d, T * d))
    for h in range(H):
        V = orth(T * d, rng)
        E[h] = V.T
        for t in range(T):
            W[t, h] = V[t * d:(t + 1) * d]
    return E, W


# --------------------------------------------------------------------------------------------
# printed numbers
# --------------------------------------------------------------------------------------------

def test_compression_ratio_printed_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "paper_numbers.json")))
    for e in g["ratios"]:
        assert O.compression_ratio(e["T"], e["d_head"], e["r_k"], e["r_v"]) == pytest.approx(e["rho"], abs=1e-12), e["cite"]
    # 21.33x at T=4, d_head=128 must come from an integer rank budget (it is 48 = 24 + 24)
    cp = g["capacity_point"]
    o = g["ouro_1p4b"]
    r_sum = 2 * o["T"] * o["d_head"] / cp["rho_printed"]
    assert abs(r_sum - round(r_sum)) < 0.01
    assert abs(O.compression_ratio(o["T"], o["d_head"], 24, 24) - cp["rho_printed"]) < cp["rho_print_tol"]


def test_cache_scalars_printed_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "paper_numbers.json")))
    o = g["ouro_1p4b"]
    full, _ = O.cache_scalars_per_token_layer("per_head", o["H"], o["T"], o["d_head"], 24, 24)
    # a looped model with T loops carries the cache of a D*T-layer decoder (2*H*d per layer)
    eq = g["looped_cache_equivalent_layers"]
    assert full * eq["D"] // (2 * o["H"] * o["d_head"]) == eq["equivalent_layers"]
    # 1M context, 21.3x (r_k + r_v = 48) and a 1024-token eviction budget: 36 MiB
    m = g["million_context_with_eviction"]
    _, comp = O.cache_scalars_per_token_layer("per_head", o["H"], o["T"], o["d_head"], 24, 24)
    total = comp * o["D"] * m["kept_tokens"] * m["bytes_per_scalar"]
    assert total == m["cache_MiB"] * 2 ** 20
    # the reduction is exactly rho
    assert full / comp == pytest.approx(O.compression_ratio(o["T"], o["d_head"], 24, 24))
    # LLA-2D is a factor H below per-head LLA (Section 3, "The LLA-2D variant")
    _, c2 = O.cache_scalars_per_token_layer("2d", o["H"], o["T"], o["d_head"], 256, 256)
    _, ch = O.cache_scalars_per_token_layer("per_head", o["H"], o["T"], o["d_head"], 256, 256)
    assert ch == o["H"] * c2


def test_capacity_shape_cache_bytes():
    """Resident latent bytes of the capacity shape (24 layers, B=768, N=4096, r=24/24, bf16)."""
    s = synth.CASES["capacity"]
    _, comp = O.cache_scalars_per_token_layer("per_head", s.H, s.T, s.d, s.r_k, s.r_v)
    assert comp * s.D * s.B * s.N * 2 == 115_964_116_992


# --------------------------------------------------------------------------------------------
# identity factors against torch SDPA
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("with_mu", [False, True])
@pytest.mark.parametrize("with_self", [False, True])
def test_full_rank_identity_per_head(with_mu, with_self):
    rng = np.random.default_rng(1)
    B, H, d, T, n_max = 2, 3, 4, 3, 7
    lens = np.array([5, 7])
    E, W = full_rank_per_head(T, H, d, rng)
    E2, W2 = full_rank_per_head(T, H, d, rng)
    xk = rng.standard_normal((B, n_max, T, H, d))
    xv = rng.standard_normal((B, n_max, T, H, d))
    mu_k = rng.standard_normal((H, T * d)) if with_mu else None
    mu_v = rng.standard_normal((H, T * d)) if with_mu else None
    zk0 = np.zeros((B, H, n_max, T * d))
    zk, zv = O.encode_into_cache(zk0, zk0, xk, xv, E, E2, [0, 0], mu_k, mu_v)
    q = rng.standard_normal((B, H, d))
    ks = rng.standard_normal((B, H, d)) if with_self else None
    vs = rng.standard_normal((B, H, d)) if with_self else None
    scale = 1 / math.sqrt(d)
    for t in range(T):
        o, lse = O.attend_decode(q, zk, zv, W, W2, t, lens, mu_k, mu_v, ks, vs)
        for b in range(B):
            for h in range(H):
                K = xk[b, :lens[b], t, h]
                V = xv[b, :lens[b], t, h]
                if with_self:
                    K = np.vstack([K, ks[b, h]])
                    V = np.vstack([V, vs[b, h]])
                ref = sdpa(q[b, h][None], K, V)[0]
                np.testing.assert_allclose(o[b, h], ref, atol=1e-10, rtol=0)
                assert lse[b, h] == pytest.approx(torch_lse(q[b, h], K, scale), abs=1e-10)


def test_full_rank_identity_2d():
    rng = np.random.default_rng(2)
    B, H, d, T, n_max = 2, 2, 3, 2, 6
    R = T * H * d
    lens = np.array([6, 4])
    Vk, Vv = orth(R, rng), orth(R, rng)
    Wk = np.stack([Vk[t * H * d:(t + 1) * H * d] for t in range(T)])
    Wv = np.stack([Vv[t * H * d:(t + 1) * H * d] for t in range(T)])
    mu_k = rng.standard_normal(R)
    mu_v = rng.standard_normal(R)
    xk = rng.standard_normal((B, n_max, T, H, d))
    xv = rng.standard_normal((B, n_max, T, H, d))
    z0 = np.zeros((B, n_max, R))
    zk, zv = O.encode_into_cache(z0, z0, xk, xv, Vk.T, Vv.T, [0, 0], mu_k, mu_v, variant="2d")
    q = rng.standard_normal((B, H, d))
    ks = rng.standard_normal((B, H, d))
    vs = rng.standard_normal((B, H, d))
    for t in range(T):
        o, lse = O.attend_decode(q, zk, zv, Wk, Wv, t, lens, mu_k, mu_v, ks, vs, variant="2d")
        for b in range(B):
            for h in range(H):
                K = np.vstack([xk[b, :lens[b], t, h], ks[b, h]])
                V = np.vstack([xv[b, :lens[b], t, h], vs[b, h]])
                np.testing.assert_allclose(o[b, h], sdpa(q[b, h][None], K, V)[0], atol=1e-10, rtol=0)
                assert lse[b, h] == pytest.approx(torch_lse(q[b, h], K, 1 / math.sqrt(d)), abs=1e-10)


def test_final_loop_reuse_special_case():
    """Caching only x_T is LLA with r = d, E = [0 .. 0 I], W_t = I (Section 3, matched baselines).

    Every loop's attention must then equal attention over the final loop's K/V, and the
    footprint is rho = T.
    """
    rng = np.random.default_rng(3)
    B, H, d, T, n = 1, 2, 5, 4, 9
    E = np.zeros((H, d, T * d))
    E[:, :, (T - 1) * d:] = np.eye(d)
    W = np.broadcast_to(np.eye(d), (T, H, d, d)).copy()
    xk = rng.standard_normal((B, n, T, H, d))
    xv = rng.standard_normal((B, n, T, H, d))
    z0 = np.zeros((B, H, n, d))
    zk, zv = O.encode_into_cache(z0, z0, xk, xv, E, E, [0])
    q = rng.standard_normal((B, H, d))
    for t in range(T):
        o, _ = O.attend_decode(q, zk, zv, W, W, t)
        for h in range(H):
            ref = sdpa(q[0, h][None], xk[0, :, T - 1, h], xv[0, :, T - 1, h])[0]
            np.testing.assert_allclose(o[0, h], ref, atol=1e-12, rtol=0)
    assert O.compression_ratio(T, d, d, d) == T


def test_exact_low_rank_trajectories():
    """Rank-<=r trajectories are rebuilt exactly by SVD factors; attention equals SDPA on them."""
    T, d, r, n = 4, 16, 8, 40
    H = 1
    stack_k = synth.trajectories(n, T, d, r, 0.0, 77)
    stack_v = synth.trajectories(n, T, d, r, 0.0, 78)
    Ek, Wk = synth.svd_factors(stack_k, r)
    Ev, Wv = synth.svd_factors(stack_v, r)
    Ek64 = np.linalg.svd(stack_k.reshape(n, T * d).astype(np.float64), full_matrices=False)[2][:r]
    # the float32 factors are accurate to ~1e-7; rebuild float64 factors for an exact check
    Ev64 = np.linalg.svd(stack_v.reshape(n, T * d).astype(np.float64), full_matrices=False)[2][:r]
    for Emat, stack in ((Ek64, stack_k), (Ev64, stack_v)):
        z = O.encode_stack(stack.reshape(n, T * d), Emat)
        for t in range(T):
            xh = O.reconstruct(z, Emat.T[t * d:(t + 1) * d])
            # the stack is stored in float32, so it is rank-r only up to float32 rounding (~6e-8)
            np.testing.assert_allclose(xh, stack[:, t], atol=1e-6 * np.abs(stack).max(), rtol=0)
    # attention with the float32 factors of the generator: exact up to their float32 rounding
    xk = stack_k[None, :, :, None, :]
    xv = stack_v[None, :, :, None, :]
    z0 = np.zeros((1, H, n, r))
    zk, zv = O.encode_into_cache(z0, z0, xk, xv, Ek[None], Ev[None], [0])
    Wk4 = Wk[:, None]
    Wv4 = Wv[:, None]
    q = np.random.default_rng(4).standard_normal((1, H, d))
    for t in range(T):
        o, _ = O.attend_decode(q, zk, zv, Wk4, Wv4, t)
        ref = sdpa(q[0, 0][None], stack_k[:, t], stack_v[:, t])[0]
        np.testing.assert_allclose(o[0, 0], ref, atol=1e-5, rtol=0)


def test_tiny_case_reconstruction_error_is_noise_level():
    """The tiny fp32 case (rank-8 + 1e-3 noise, r=8) rebuilds its trajectories to ~1e-3."""
    c = synth.tiny_fp32_case()
    s = synth.CASES["tiny_fp32"]
    for ax in ("k", "v"):
        x = c["x" + ax][0, :s.N]            # [N, T, H, d]
        for h in range(s.H):
            st = x[:, :, h, :].reshape(s.N, s.T * s.d)
            z = O.encode_stack(st, c["E" + ax][h])
            rec = np.concatenate([O.reconstruct(z, c["W" + ax][t, h]) for t in range(s.T)], axis=1)
            rel = np.linalg.norm(rec - st) / np.linalg.norm(st)
            assert 1e-5 < rel < 1e-2


# --------------------------------------------------------------------------------------------
# closed forms and invariances
# --------------------------------------------------------------------------------------------

def _rand_case(rng, B=2, H=2, d=6, T=3, rk=4, rv=5, n_max=8, variant="per_head"):
    if variant == "per_head":
        zk = rng.standard_normal((B, H, n_max, rk))
        zv = rng.standard_normal((B, H, n_max, rv))
        Wk = rng.standard_normal((T, H, d, rk))
        Wv = rng.standard_normal((T, H, d, rv))
        mu_k = rng.standard_normal((H, T * d))
        mu_v = rng.standard_normal((H, T * d))
    else:
        zk = rng.standard_normal((B, n_max, rk))
        zv = rng.standard_normal((B, n_max, rv))
        Wk = rng.standard_normal((T, H * d, rk))
        Wv = rng.standard_normal((T, H * d, rv))
        mu_k = rng.standard_normal(T * H * d)
        mu_v = rng.standard_normal(T * H * d)
    q = rng.standard_normal((B, H, d))
    ks = rng.standard_normal((B, H, d))
    vs = rng.standard_normal((B, H, d))
    return dict(q=q, zk=zk, zv=zv, Wk=Wk, Wv=Wv, mu_k=mu_k, mu_v=mu_v, k_self=ks, v_self=vs)


@pytest.mark.parametrize("variant", ["per_head", "2d"])
def test_absorbed_equals_explicit(variant):
    """Section 7: moving W^K to the query and applying W^V once after the sum changes nothing."""
    rng = np.random.default_rng(5)
    c = _rand_case(rng, variant=variant)
    lens = np.array([8, 3])
    for t in range(3):
        for kw in ({}, {"k_self": c["k_self"], "v_self": c["v_self"]}):
            args = (c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], t, lens, c["mu_k"], c["mu_v"])
            o1, l1 = O.attend_decode(*args, variant=variant, **kw)
            o2, l2 = O.attend_decode_absorbed(*args, variant=variant, **kw)
            np.testing.assert_allclose(o1, o2, atol=1e-11, rtol=0)
            np.testing.assert_allclose(l1, l2, atol=1e-11, rtol=0)


def test_zero_query_gives_mean_value():
    """q = 0 makes every weight 1/n: o = W^V_t mean(z^V) + mu^V_t and lse = log n."""
    rng = np.random.default_rng(6)
    c = _rand_case(rng)
    lens = np.array([8, 5])
    q0 = np.zeros_like(c["q"])
    d, T = 6, 3
    for t in range(T):
        o, lse = O.attend_decode(q0, c["zk"], c["zv"], c["Wk"], c["Wv"], t, lens, c["mu_k"], c["mu_v"])
        for b in range(2):
            for h in range(2):
                zbar = c["zv"][b, h, :lens[b]].mean(axis=0)
                ref = c["Wv"][t, h] @ zbar + c["mu_v"][h, t * d:(t + 1) * d]
                np.testing.assert_allclose(o[b, h], ref, atol=1e-12, rtol=0)
                assert lse[b, h] == pytest.approx(math.log(lens[b]), abs=1e-12)


def test_constant_values_give_the_constant():
    """If every rebuilt value equals the same vector, o equals it (softmax weights sum to 1)."""
    rng = np.random.default_rng(7)
    c = _rand_case(rng)
    Wv0 = np.zeros_like(c["Wv"])
    cst = rng.standard_normal(6)
    mu_v = np.tile(cst, (2, 3))
    vs = np.broadcast_to(cst, c["v_self"].shape)
    q = 30 * c["q"]
    for t in range(3):
        o, _ = O.attend_decode(q, c["zk"], c["zv"], c["Wk"], Wv0, t, None, c["mu_k"], mu_v, c["k_self"], vs)
        np.testing.assert_allclose(o, np.broadcast_to(cst, o.shape), atol=1e-13, rtol=0)


def test_sharp_query_selects_best_key():
    """Scaling q up drives the softmax to the key with the largest score."""
    rng = np.random.default_rng(8)
    c = _rand_case(rng, B=1, H=1)
    t = 1
    K = c["zk"][0, 0] @ c["Wk"][t, 0].T + c["mu_k"][0, t * 6:(t + 1) * 6]
    V = c["zv"][0, 0] @ c["Wv"][t, 0].T + c["mu_v"][0, t * 6:(t + 1) * 6]
    s = K @ c["q"][0, 0]
    srt = np.sort(s)
    lam = 60.0 / (srt[-1] - srt[-2]) * math.sqrt(6)
    o, lse = O.attend_decode(lam * c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], t, None, c["mu_k"], c["mu_v"])
    np.testing.assert_allclose(o[0, 0], V[np.argmax(s)], atol=1e-9 * np.abs(V).max(), rtol=0)
    assert lse[0, 0] == pytest.approx(lam * srt[-1] / math.sqrt(6), rel=1e-12)


def test_lse_merge_of_disjoint_token_sets():
    """Attention over A u B is the log-sum-exp weighted merge of attention over A and over B."""
    rng = np.random.default_rng(9)
    c = _rand_case(rng, n_max=10)
    split = 4
    zk_b = np.roll(c["zk"], -split, axis=2)
    zv_b = np.roll(c["zv"], -split, axis=2)
    t = 2
    base = (c["Wk"], c["Wv"], t)
    o, l = O.attend_decode(c["q"], c["zk"], c["zv"], *base, None, c["mu_k"], c["mu_v"])
    oa, la = O.attend_decode(c["q"], c["zk"], c["zv"], *base, [split, split], c["mu_k"], c["mu_v"])
    ob, lb = O.attend_decode(c["q"], zk_b, zv_b, *base, [10 - split] * 2, c["mu_k"], c["mu_v"])
    np.testing.assert_allclose(l, np.logaddexp(la, lb), atol=1e-12, rtol=0)
    merged = (np.exp(la - l)[..., None] * oa + np.exp(lb - l)[..., None] * ob)
    np.testing.assert_allclose(o, merged, atol=1e-12, rtol=0)


def test_token_permutation_invariance():
    rng = np.random.default_rng(10)
    c = _rand_case(rng)
    perm = rng.permutation(8)
    o1, l1 = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 0, None, c["mu_k"], c["mu_v"], c["k_self"], c["v_self"])
    o2, l2 = O.attend_decode(c["q"], c["zk"][:, :, perm], c["zv"][:, :, perm], c["Wk"], c["Wv"], 0, None,
                             c["mu_k"], c["mu_v"], c["k_self"], c["v_self"])
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-12, rtol=0)


def test_2d_with_one_head_equals_per_head():
    rng = np.random.default_rng(11)
    c = _rand_case(rng, H=1)
    for t in range(3):
        o1, l1 = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], t, [8, 2], c["mu_k"], c["mu_v"], c["k_self"], c["v_self"])
        o2, l2 = O.attend_decode(c["q"], c["zk"][:, 0], c["zv"][:, 0], c["Wk"][:, 0], c["Wv"][:, 0], t, [8, 2],
                                 c["mu_k"][0], c["mu_v"][0], c["k_self"], c["v_self"], variant="2d")
        np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
        np.testing.assert_allclose(l1, l2, atol=1e-13, rtol=0)
    # encode: per-head with H=1 and LLA-2D write the same latents
    xk = rng.standard_normal((2, 1, 3, 1, 6))
    E = rng.standard_normal((1, 4, 18))
    mu = rng.standard_normal((1, 18))
    a, _ = O.encode_into_cache(np.zeros((2, 1, 3, 4)), np.zeros((2, 1, 3, 4)), xk, xk, E, E, [1, 2], mu, mu)
    b, _ = O.encode_into_cache(np.zeros((2, 3, 4)), np.zeros((2, 3, 4)), xk, xk, E[0], E[0], [1, 2], mu[0], mu[0], variant="2d")
    np.testing.assert_allclose(a[:, 0], b, atol=0, rtol=0)


def test_empty_context_and_length_clamp():
    rng = np.random.default_rng(12)
    c = _rand_case(rng)
    d = 6
    o, lse = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 0, [0, 0], c["mu_k"], c["mu_v"], c["k_self"], c["v_self"])
    np.testing.assert_allclose(o, c["v_self"], atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, np.sum(c["q"] * c["k_self"], -1) / math.sqrt(d), atol=1e-13, rtol=0)
    o, lse = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 0, [0, 0], c["mu_k"], c["mu_v"])
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o1, _ = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 1, [99, -3], c["mu_k"], c["mu_v"])
    o2, _ = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 1, [8, 0], c["mu_k"], c["mu_v"])
    np.testing.assert_array_equal(o1, o2)


# --------------------------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["per_head", "2d"])
def test_prefill_one_row_equals_decode(variant):
    rng = np.random.default_rng(13)
    c = _rand_case(rng, variant=variant)
    ctx = np.array([4, 7])
    for t in range(3):
        o_p = O.attend_prefill(c["q"][:, None], c["zk"], c["zv"], c["Wk"], c["Wv"], t, ctx, c["mu_k"], c["mu_v"], variant=variant)
        o_d, _ = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], t, ctx + 1, c["mu_k"], c["mu_v"], variant=variant)
        np.testing.assert_allclose(o_p[:, 0], o_d, atol=1e-13, rtol=0)


def test_prefill_full_rank_identity_causal_offset():
    """Chunk row j at position ctx + j sees keys 0 .. ctx + j: SDPA with that boolean mask."""
    rng = np.random.default_rng(14)
    B, H, d, T, C = 2, 2, 3, 2, 5
    ctx = np.array([3, 6])
    n_max = 12
    E, W = full_rank_per_head(T, H, d, rng)
    E2, W2 = full_rank_per_head(T, H, d, rng)
    xk = rng.standard_normal((B, n_max, T, H, d))
    xv = rng.standard_normal((B, n_max, T, H, d))
    z0 = np.zeros((B, H, n_max, T * d))
    zk, zv = O.encode_into_cache(z0, z0, xk, xv, E, E2, [0, 0])
    q = rng.standard_normal((B, C, H, d))
    for t in range(T):
        o = O.attend_prefill(q, zk, zv, W, W2, t, ctx)
        for b in range(B):
            n = ctx[b] + C
            mask = np.arange(n)[None, :] <= (ctx[b] + np.arange(C))[:, None]
            for h in range(H):
                ref = sdpa(q[b, :, h], xk[b, :n, t, h], xv[b, :n, t, h], mask)
                np.testing.assert_allclose(o[b, :, h], ref, atol=1e-10, rtol=0)


# --------------------------------------------------------------------------------------------
# brute force on tiny inputs (plain loops over every scalar)
# --------------------------------------------------------------------------------------------

def test_brute_force_tiny():
    rng = np.random.default_rng(15)
    B, H, d, T, rk, rv, n = 1, 2, 3, 2, 2, 3, 4
    c = _rand_case(rng, B=B, H=H, d=d, T=T, rk=rk, rv=rv, n_max=n)
    t = 1
    o, _ = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], t, None, c["mu_k"], c["mu_v"], c["k_self"], c["v_self"])
    for h in range(H):
        keys, vals = [], []
        for i in range(n):
            k = [sum(c["Wk"][t, h, j, a] * c["zk"][0, h, i, a] for a in range(rk)) + c["mu_k"][h, t * d + j] for j in range(d)]
            v = [sum(c["Wv"][t, h, j, a] * c["zv"][0, h, i, a] for a in range(rv)) + c["mu_v"][h, t * d + j] for j in range(d)]
            keys.append(k)
            vals.append(v)
        keys.append(list(c["k_self"][0, h]))
        vals.append(list(c["v_self"][0, h]))
        sc = [sum(c["q"][0, h, j] * k[j] for j in range(d)) / math.sqrt(d) for k in keys]
        w = [math.exp(s) for s in sc]
        tot = sum(w)
        ref = [sum(w[i] * vals[i][j] for i in range(n + 1)) / tot for j in range(d)]
        np.testing.assert_allclose(o[0, h], ref, atol=1e-12, rtol=0)


def test_bf16_rounding_of_rebuilt_kv():
    """round_bf16_via_f32 keeps bf16 values, rounds halfway cases to even, and the rounded decode
    equals the unrounded one when every rebuilt K/V value is already a bf16 value."""
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -7), 3.0 + 2.0 ** -20])
    np.testing.assert_array_equal(O.round_bf16_via_f32(v),
                                  [1.0, 1.0, 1.0 + 2.0 ** -6, -(1.0 + 2.0 ** -7), 3.0])
    rng = np.random.default_rng(21)
    c = _rand_case(rng)
    for k in ("zk", "zv", "Wk", "Wv", "mu_k", "mu_v"):
        c[k] = np.round(c[k] * 2) / 2  # small multiples of 1/2: every rebuilt value is exact in bf16
    a = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 1, None, c["mu_k"], c["mu_v"])
    b = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 1, None, c["mu_k"], c["mu_v"],
                        kv_round_bf16=True)
    np.testing.assert_array_equal(a[0], b[0])
    c2 = _rand_case(rng)
    a = O.attend_decode(c2["q"], c2["zk"], c2["zv"], c2["Wk"], c2["Wv"], 1)
    b = O.attend_decode(c2["q"], c2["zk"], c2["zv"], c2["Wk"], c2["Wv"], 1, kv_round_bf16=True)
    assert 0 < np.max(np.abs(a[0] - b[0])) < 2e-2 * np.max(np.abs(a[0]))
