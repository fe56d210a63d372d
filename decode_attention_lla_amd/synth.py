"""Seeded synthetic inputs for the LLA latent-cache kernels and their tests.

This module only draws random numbers, rounds them to the storage precision and builds test
factor matrices. It computes none of the codec or attention arithmetic (no encode, no
reconstruction, no softmax): the GPU library and the CPU oracle each do that on their own, and
both receive the arrays produced here.

Workload shapes follow five synthetic cases (the paper's own capacity test fabricates the decode
cache the same way; Section 7, "Serving and compute"):

  tiny_fp32    fp32, H=2, d=16, T=4, r=8/8, B=1, N=64: per-loop K/V are rank-8 trajectories
               plus 1e-3 noise and the factors come from the SVD of the stacked trajectories
               (Section 3, "Initialization and conversion"; here uncentred, mu = 0).
  ouro_layer   bf16, one Ouro-1.4B-shaped layer: H=16, d=128, T=4, r=32/32, B=32, N=4096.
  capacity     bf16, 24 layers, H=16, d=128, T=4, r=24/24 (21.3x), B=768, N=4096.
  deep_loop    bf16, H=40, d=96, T=32, r=96/96 (32x), B=64, N=4096.
  lla2d        bf16 LLA-2D, H=16, d=128, T=4, r=256/256 (32x), B=128, N=8192, prefill C=512.

For the bf16 cases latents, queries and self K/V are N(0,1); each W_t is the orthonormal Q of a
Gaussian d x r matrix; E = (1/T) [W_1^T ... W_T^T], which is the pseudo-inverse of the stacked
[W_1; ...; W_T] when every W_t has orthonormal columns. Seeds are 1000*case + tensor id.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids inside a case's seed block
SEED_Q, SEED_ZK, SEED_ZV, SEED_WK, SEED_WV, SEED_EK, SEED_EV, SEED_XK, SEED_XV, SEED_SELF = range(1, 11)
SEED_MU, SEED_LENS, SEED_SAMPLE, SEED_SLOTS = 11, 12, 13, 14


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    variant: str      # "per_head" or "2d"
    dtype: str        # "f32" or "bf16" (storage of every tensor; accumulation is fp32 on the GPU)
    D: int            # layers
    H: int
    d: int            # d_head
    T: int            # loops
    r_k: int
    r_v: int
    B: int
    N: int            # latent tokens per sequence already in the cache
    C: int = 1        # prefill chunk (1 = decode)
    case: int = 0     # seed block

    @property
    def n_max(self):
        return self.N + self.C

    def with_(self, **kw):
        return dataclasses.replace(self, **kw)


CASES = {
    "tiny_fp32": Shape("tiny_fp32", "per_head", "f32", 1, 2, 16, 4, 8, 8, 1, 64, 1, 1),
    "ouro_layer": Shape("ouro_layer", "per_head", "bf16", 1, 16, 128, 4, 32, 32, 32, 4096, 1, 2),
    "capacity": Shape("capacity", "per_head", "bf16", 24, 16, 128, 4, 24, 24, 768, 4096, 1, 3),
    "deep_loop": Shape("deep_loop", "per_head", "bf16", 1, 40, 96, 32, 96, 96, 64, 4096, 1, 4),
    "lla2d": Shape("lla2d", "2d", "bf16", 1, 16, 128, 4, 256, 256, 128, 8192, 512, 5),
}


def seed(case: int, tensor: int, layer: int = 0) -> int:
    return 1000 * case + tensor + 100000 * layer


# --------------------------------------------------------------------------------------------
# precision helpers
# --------------------------------------------------------------------------------------------

def round_bf16(a):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 holding them."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def to_storage(a, dtype: str):
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a)


def normal(shape, sd: int, dtype: str = "f32", std: float = 1.0):
    g = np.random.default_rng(sd)
    return to_storage(std * g.standard_normal(shape, dtype=np.float32), dtype)


# --------------------------------------------------------------------------------------------
# factor construction (test inputs)
# --------------------------------------------------------------------------------------------

def orthonormal_W(T: int, H: int, d: int, r: int, sd: int, dtype: str):
    """W [T, H, d, r]: each (t, h) slice is the orthonormal Q factor of a Gaussian d x r matrix."""
    g = np.random.default_rng(sd)
    G = g.standard_normal((T, H, d, r))
    Q, R = np.linalg.qr(G)
    # fix signs so the draw is unique (diag(R) > 0)
    sgn = np.sign(np.diagonal(R, axis1=-2, axis2=-1))
    sgn[sgn == 0] = 1.0
    Q = Q * sgn[..., None, :]
    return to_storage(Q, dtype)


def pinv_E_from_W(W, dtype: str):
    """E [H, r, T*d] = (1/T) [W_1^T ... W_T^T] for W [T, H, d, r] with orthonormal columns."""
    W = np.asarray(W, dtype=np.float64)
    T, H, d, r = W.shape
    E = np.transpose(W, (1, 3, 0, 2)).reshape(H, r, T * d) / T
    return to_storage(E, dtype)


def orthonormal_W_2d(T: int, H: int, d: int, r: int, sd: int, dtype: str):
    """LLA-2D W [T, H*d, r]: each loop slice is an orthonormal (H*d) x r matrix."""
    return orthonormal_W(T, 1, H * d, r, sd, dtype)[:, 0]


def pinv_E_from_W_2d(W, dtype: str):
    """LLA-2D E [r, T*H*d] = (1/T) [W_1^T ... W_T^T] for W [T, H*d, r]."""
    return pinv_E_from_W(np.asarray(W)[:, None], dtype)[0]


def trajectories(n_tok: int, T: int, d: int, rank: int, noise: float, sd: int):
    """Per-loop vectors x_t = A_t u + noise * N(0, 1) for n_tok tokens; returns [n_tok, T, d].

    u ~ N(0, I_rank) per token, A_t ~ N(0, 1)/sqrt(rank) (d x rank), one A_t per loop.
    """
    g = np.random.default_rng(sd)
    A = g.standard_normal((T, d, rank)) / math.sqrt(rank)
    u = g.standard_normal((n_tok, rank))
    x = np.einsum("tdk,nk->ntd", A, u) + noise * g.standard_normal((n_tok, T, d))
    return x.astype(np.float32)


def svd_factors(stack, r: int):
    """Test factors from the SVD of a token-by-(T*d) trajectory matrix (uncentred).

    Follows the initialisation recipe of Section 3, "Initialization and conversion": the
    down-projection holds the top-r right singular vectors and each loop's up-projection is the
    matching d-row slice. Returns (E [r, T*d], W [T, d, r]) for a stack of shape [n, T, d].
    """
    n, T, d = stack.shape
    M = np.asarray(stack, dtype=np.float64).reshape(n, T * d)
    _, _, Vt = np.linalg.svd(M, full_matrices=False)
    Vr = Vt[:r].T                      # [T*d, r]
    E = Vr.T                           # [r, T*d]
    W = Vr.reshape(T, d, r)            # rows t*d .. (t+1)*d
    return E.astype(np.float32), W.astype(np.float32)


# --------------------------------------------------------------------------------------------
# whole cases on the host (sizes the oracle handles)
# --------------------------------------------------------------------------------------------

def host_case(s: Shape, with_mu: bool = False, with_self: bool = True, lens=None, t_seed: int = 0):
    """All inputs of one decode step for shape s, as float32 numpy arrays holding storage values.

    Keys: q [T,B,H,d] (one query per loop), zk/zv caches (N filled, slot N.. zero), Wk, Wv,
    Ek, Ev, mu_k/mu_v (or None), k_self/v_self [T,B,H,d], xk/xv [B,1,T,H,d] (the new token's
    per-loop K/V to encode), seq_lens [B].
    """
    c = s.case + 10 * t_seed
    dt = s.dtype
    B, H, d, T, rk, rv = s.B, s.H, s.d, s.T, s.r_k, s.r_v
    out = {}
    if s.variant == "per_head":
        out["Wk"] = orthonormal_W(T, H, d, rk, seed(c, SEED_WK), dt)
        out["Wv"] = orthonormal_W(T, H, d, rv, seed(c, SEED_WV), dt)
        out["Ek"] = pinv_E_from_W(out["Wk"], dt)
        out["Ev"] = pinv_E_from_W(out["Wv"], dt)
        zshape_k = (B, H, s.n_max, rk)
        zshape_v = (B, H, s.n_max, rv)
        mu_shape = (H, T * d)
    else:
        out["Wk"] = orthonormal_W_2d(T, H, d, rk, seed(c, SEED_WK), dt)
        out["Wv"] = orthonormal_W_2d(T, H, d, rv, seed(c, SEED_WV), dt)
        out["Ek"] = pinv_E_from_W_2d(out["Wk"], dt)
        out["Ev"] = pinv_E_from_W_2d(out["Wv"], dt)
        zshape_k = (B, s.n_max, rk)
        zshape_v = (B, s.n_max, rv)
        mu_shape = (T * H * d,)
    zk = np.zeros(zshape_k, np.float32)
    zv = np.zeros(zshape_v, np.float32)
    if s.variant == "per_head":
        zk[:, :, :s.N] = normal((B, H, s.N, rk), seed(c, SEED_ZK), dt)
        zv[:, :, :s.N] = normal((B, H, s.N, rv), seed(c, SEED_ZV), dt)
    else:
        zk[:, :s.N] = normal((B, s.N, rk), seed(c, SEED_ZK), dt)
        zv[:, :s.N] = normal((B, s.N, rv), seed(c, SEED_ZV), dt)
    out["zk"], out["zv"] = zk, zv
    out["q"] = normal((T, B, H, d), seed(c, SEED_Q), dt)
    if with_self:
        kv = normal((2, T, B, H, d), seed(c, SEED_SELF), dt)
        out["k_self"], out["v_self"] = kv[0], kv[1]
    else:
        out["k_self"] = out["v_self"] = None
    if with_mu:
        m = normal((2,) + mu_shape, seed(c, SEED_MU), dt, std=0.5)
        out["mu_k"], out["mu_v"] = m[0], m[1]
    else:
        out["mu_k"] = out["mu_v"] = None
    out["xk"] = normal((B, s.C, T, H, d), seed(c, SEED_XK), dt)
    out["xv"] = normal((B, s.C, T, H, d), seed(c, SEED_XV), dt)
    if lens is None:
        out["seq_lens"] = np.full((B,), s.N, np.int32)
    else:
        out["seq_lens"] = np.asarray(lens, np.int32)
    return out


def tiny_fp32_case(s: Shape = CASES["tiny_fp32"]):
    """The tiny fp32 case: rank-8 trajectories + 1e-3 noise, SVD factors per (head, axis).

    Returns trajectories xk/xv [B, N+1, T, H, d] (N context tokens then the new token), factors
    Ek/Ev [H, r, T*d], Wk/Wv [T, H, d, r], queries q [T, B, H, d] (one per loop).
    """
    B, H, d, T, rk, rv, N = s.B, s.H, s.d, s.T, s.r_k, s.r_v, s.N
    xk = np.zeros((B, N + 1, T, H, d), np.float32)
    xv = np.zeros((B, N + 1, T, H, d), np.float32)
    Ek = np.zeros((H, rk, T * d), np.float32)
    Ev = np.zeros((H, rv, T * d), np.float32)
    Wk = np.zeros((T, H, d, rk), np.float32)
    Wv = np.zeros((T, H, d, rv), np.float32)
    for b in range(B):
        for h in range(H):
            tk = trajectories(N + 1, T, d, rk, 1e-3, seed(s.case, SEED_XK) + 31 * h + 7 * b)
            tv = trajectories(N + 1, T, d, rv, 1e-3, seed(s.case, SEED_XV) + 31 * h + 7 * b)
            xk[b, :, :, h, :] = tk
            xv[b, :, :, h, :] = tv
            if b == 0:
                e, w = svd_factors(tk[:N], rk)
                Ek[h], Wk[:, h] = e, w
                e, w = svd_factors(tv[:N], rv)
                Ev[h], Wv[:, h] = e, w
    q = normal((T, B, H, d), seed(s.case, SEED_Q), "f32")
    return {"xk": xk, "xv": xv, "Ek": Ek, "Ev": Ev, "Wk": Wk, "Wv": Wv, "q": q}


# --------------------------------------------------------------------------------------------
# device fills for the large cases (torch is only plumbing here)
# --------------------------------------------------------------------------------------------

def device_normal_(tensor, sd: int, std: float = 1.0):
    """Fill a device tensor in place with N(0, std^2) from a seeded device generator."""
    import torch
    g = torch.Generator(device=tensor.device)
    g.manual_seed(sd)
    tensor.normal_(0.0, std, generator=g)
    return tensor


def random_case(variant: str, dtype: str, B: int, H: int, d: int, T: int, r_k: int, r_v: int,
                n_max: int, sd: int, with_mu: bool = True, with_self: bool = True,
                q_gain: float = 1.0):
    """Generic seeded inputs for any shape (used by the shape sweeps).

    Latents, queries and self K/V are N(0,1); W entries are N(0, 1/r) so rebuilt K/V have unit
    variance; E entries are N(0, 1/(T*d)); mu (if any) has std 0.5. q_gain scales the query (a
    gain of 8 sharpens the softmax). Returns float32 arrays holding storage values.
    """
    c = sd
    if variant == "per_head":
        zk_s, zv_s = (B, H, n_max, r_k), (B, H, n_max, r_v)
        wk_s, wv_s = (T, H, d, r_k), (T, H, d, r_v)
        ek_s, ev_s = (H, r_k, T * d), (H, r_v, T * d)
        mu_s = (H, T * d)
        K = T * d
    else:
        zk_s, zv_s = (B, n_max, r_k), (B, n_max, r_v)
        wk_s, wv_s = (T, H * d, r_k), (T, H * d, r_v)
        ek_s, ev_s = (r_k, T * H * d), (r_v, T * H * d)
        mu_s = (T * H * d,)
        K = T * H * d
    out = {
        "zk": normal(zk_s, seed(c, SEED_ZK), dtype),
        "zv": normal(zv_s, seed(c, SEED_ZV), dtype),
        "Wk": normal(wk_s, seed(c, SEED_WK), dtype, std=1 / math.sqrt(r_k)),
        "Wv": normal(wv_s, seed(c, SEED_WV), dtype, std=1 / math.sqrt(r_v)),
        "Ek": normal(ek_s, seed(c, SEED_EK), dtype, std=1 / math.sqrt(K)),
        "Ev": normal(ev_s, seed(c, SEED_EV), dtype, std=1 / math.sqrt(K)),
        "q": to_storage(q_gain * normal((T, B, H, d), seed(c, SEED_Q), "f32"), dtype),
    }
    if with_self:
        kv = normal((2, T, B, H, d), seed(c, SEED_SELF), dtype)
        out["k_self"], out["v_self"] = kv[0], kv[1]
    else:
        out["k_self"] = out["v_self"] = None
    if with_mu:
        m = normal((2,) + mu_s, seed(c, SEED_MU), dtype, std=0.5)
        out["mu_k"], out["mu_v"] = m[0], m[1]
    else:
        out["mu_k"] = out["mu_v"] = None
    return out


def random_slots(B: int, budget: int, n_max: int, sd: int, p_skip: float = 0.0,
                 p_repeat: float = 0.0):
    """Seeded slot lists [B, budget] int32 for gather-indexed reads (H2O-like arbitrary subsets).

    Slots are drawn uniformly from [0, n_max) without replacement where budget <= n_max. A fraction
    p_skip is then replaced by out-of-range values (-1 or n_max + k) and a fraction p_repeat by a
    copy of another entry of the same row.
    """
    rng = np.random.default_rng(sd)
    out = np.empty((B, budget), dtype=np.int32)
    for b in range(B):
        if budget <= n_max:
            row = rng.choice(n_max, size=budget, replace=False)
        else:
            row = rng.integers(0, n_max, size=budget)
        skip = rng.random(budget) < p_skip
        row[skip] = np.where(rng.random(int(skip.sum())) < 0.5, -1, n_max + rng.integers(0, 7, int(skip.sum())))
        rep = rng.random(budget) < p_repeat
        row[rep] = row[rng.integers(0, budget, int(rep.sum()))]
        out[b] = row
    return out

