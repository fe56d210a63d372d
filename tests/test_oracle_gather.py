"""Pins of the oracle's gather-indexed decode and eviction policy (CPU only).

Token eviction composed with LLA (Section 7, "Memory, capacity and latency"; Appendix C): a decode
row attends a listed subset of the cached latents. The oracle's attend_decode_gather is pinned to
* the already-pinned contiguous decode (a list 0 .. n-1 is the same read);
* torch's scaled_dot_product_attention in float64 on the kept tokens' original per-loop K/V, with
  full-rank orthogonal factors that make the codec exact;
* plain loops over every scalar on a tiny case with duplicates, out-of-range slots and counts;
* invariance to the order of the list.
streaming_kept_slots is pinned to its closed form (sink + window, Appendix C, Table 9).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import lla_oracle as O


def _case(rng, B=2, H=2, d=6, T=3, rk=4, rv=5, n_max=9, variant="per_head"):
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
    return dict(q=rng.standard_normal((B, H, d)), zk=zk, zv=zv, Wk=Wk, Wv=Wv, mu_k=mu_k,
                mu_v=mu_v, k_self=rng.standard_normal((B, H, d)),
                v_self=rng.standard_normal((B, H, d)))


def _args(c, with_self):
    return dict(mu_k=c["mu_k"], mu_v=c["mu_v"], k_self=c["k_self"] if with_self else None,
                v_self=c["v_self"] if with_self else None)


@pytest.mark.parametrize("variant", ["per_head", "2d"])
@pytest.mark.parametrize("with_self", [False, True])
def test_identity_list_equals_contiguous_decode(variant, with_self):
    rng = np.random.default_rng(41)
    c = _case(rng, variant=variant)
    lens = np.array([9, 5])
    slots = np.tile(np.arange(9), (2, 1))
    o, lse = O.attend_decode_gather(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 2, slots, lens,
                                    variant=variant, **_args(c, with_self))
    o2, lse2 = O.attend_decode(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 2, lens,
                               variant=variant, **_args(c, with_self))
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-12, rtol=0)


def test_order_of_the_list_does_not_matter():
    rng = np.random.default_rng(42)
    c = _case(rng)
    slots = np.array([[0, 3, 7, 8, 2], [8, 1, 4, 4, 6]])
    perm = np.array([[4, 2, 0, 3, 1], [1, 3, 0, 4, 2]])
    shuffled = np.take_along_axis(slots, perm, axis=1)
    a = O.attend_decode_gather(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 1, slots, None,
                               **_args(c, True))
    b = O.attend_decode_gather(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 1, shuffled, None,
                               **_args(c, True))
    np.testing.assert_allclose(a[0], b[0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(a[1], b[1], atol=1e-12, rtol=0)


def _orth(n, rng):
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return Q


def test_full_rank_codec_equals_sdpa_on_kept_tokens():
    """With r = T*d orthogonal factors the codec is exact, so attention over the kept latents is
    attention over the kept tokens' original loop-t K/V (torch SDPA, float64)."""
    rng = np.random.default_rng(43)
    B, H, d, T, n = 2, 2, 4, 2, 12
    r = T * d
    E = np.zeros((H, r, r))
    W = np.zeros((T, H, d, r))
    for h in range(H):
        V = _orth(r, rng)
        E[h] = V.T
        for t in range(T):
            W[t, h] = V[t * d:(t + 1) * d]
    xk = rng.standard_normal((B, n, T, H, d))
    xv = rng.standard_normal((B, n, T, H, d))
    zk, zv = O.encode_into_cache(np.zeros((B, H, n, r)), np.zeros((B, H, n, r)), xk, xv, E, E,
                                 np.zeros(B, dtype=np.int64))
    q = rng.standard_normal((B, H, d))
    keep = [O.streaming_kept_slots(n, 2, 4), [11, 0, 5]]
    slots = np.full((B, 6), -1)
    for b in range(B):
        slots[b, :len(keep[b])] = keep[b]
    counts = np.array([6, 3])
    t = 1
    o, _ = O.attend_decode_gather(q, zk, zv, W, W, t, slots, counts)
    for b in range(B):
        for h in range(H):
            K = xk[b, keep[b], t, h]
            Vv = xv[b, keep[b], t, h]
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q[b, h])[None, None, None], torch.from_numpy(K)[None, None],
                torch.from_numpy(Vv)[None, None])[0, 0, 0].numpy()
            np.testing.assert_allclose(o[b, h], ref, atol=1e-10, rtol=0)


def test_brute_force_tiny_with_duplicates_and_skips():
    rng = np.random.default_rng(44)
    B, H, d, T, rk, rv, n = 1, 2, 3, 2, 2, 3, 5
    c = _case(rng, B=B, H=H, d=d, T=T, rk=rk, rv=rv, n_max=n)
    t = 0
    slots = np.array([[3, -1, 1, 3, 5, 0, 2]])  # -1 and 5 are skipped; 3 is listed twice; 2 is past count
    counts = np.array([6])
    o, lse = O.attend_decode_gather(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], t, slots, counts,
                                    **_args(c, True))
    used = [3, 1, 3, 0]
    for h in range(H):
        keys, vals = [], []
        for i in used:
            keys.append([sum(c["Wk"][t, h, j, a] * c["zk"][0, h, i, a] for a in range(rk))
                         + c["mu_k"][h, t * d + j] for j in range(d)])
            vals.append([sum(c["Wv"][t, h, j, a] * c["zv"][0, h, i, a] for a in range(rv))
                         + c["mu_v"][h, t * d + j] for j in range(d)])
        keys.append(list(c["k_self"][0, h]))
        vals.append(list(c["v_self"][0, h]))
        sc = [sum(c["q"][0, h, j] * k[j] for j in range(d)) / math.sqrt(d) for k in keys]
        w = [math.exp(s) for s in sc]
        tot = sum(w)
        ref = [sum(w[i] * vals[i][j] for i in range(len(keys))) / tot for j in range(d)]
        np.testing.assert_allclose(o[0, h], ref, atol=1e-12, rtol=0)
        assert abs(lse[0, h] - math.log(tot)) < 1e-12


def test_empty_lists():
    rng = np.random.default_rng(45)
    c = _case(rng)
    slots = np.array([[-3, 100, 9], [1, 2, 3]])  # n_max = 9
    counts = np.array([3, -2])  # row 0: every slot skipped; row 1: count clamps to 0
    o, lse = O.attend_decode_gather(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 0, slots, counts)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, _ = O.attend_decode_gather(c["q"], c["zk"], c["zv"], c["Wk"], c["Wv"], 0, slots, counts,
                                  **_args(c, True))
    np.testing.assert_allclose(o, c["v_self"], atol=1e-12, rtol=0)  # only the self token is left


def test_streaming_kept_slots_closed_form():
    assert O.streaming_kept_slots(0, 4, 256) == []
    assert O.streaming_kept_slots(100, 4, 256) == list(range(100))
    assert O.streaming_kept_slots(260, 4, 256) == list(range(260))
    s = O.streaming_kept_slots(4096, 4, 256)
    assert s == [0, 1, 2, 3] + list(range(4096 - 256, 4096))
    assert len(O.streaming_kept_slots(1 << 20, 4, 1020)) == 1024  # a 1024-token budget at 1M
