"""CPU oracle for Looped Latent Attention (LLA): encode, per-loop reconstruction and attention.

TEST INFRASTRUCTURE. This module is the slow, obviously correct definition that the GPU library
is checked against. Only the test suite, the smoke check of the entry module and the CPU-baseline
leg of the benchmark may import it. The GPU library never imports it and shares no code with it.

Source of every definition: O'Neill & Reid, "Looped Latent Attention: Cross-Loop KV Compression
for Looped Transformers" (arXiv 2607.15456, HTML version):
  - Section 3, "Teacher cache", Eq. 1: the T per-loop vectors of one (layer, head, axis, token) are
    stacked loop-major into x = [x_1; ...; x_T] of length T*d_head.
  - Section 3, "Cross-loop codec", Eq. 2: latent c = (x - mu) W_down (row-vector form).
  - Section 3, "Cross-loop codec", Eq. 3: loop t is rebuilt as x_hat_t = c W_up,t^T + mu_t.
  - Section 3, "Cross-loop codec", Eq. 4: rho = 2 T d_head / (r_k + r_v); K and V use separate
    latents and ranks.
  - Section 3, "The LLA-2D variant": one latent per token and layer, encoded from the whole
    T*H*d_head stack and rebuilding every head.
  - Section 7, "Per-head LLA versus LLA-2D at inference": the score is bilinear, so the K
    up-projection can move to the query side, and the V up-projection can be applied once to the
    probability-weighted sum of latents (the absorbed form).
  - Appendix A, "Decoding and caching": the latent-store decoder caches only latents and rebuilds
    on read; prefill is two-pass (encode first, then attend).

Column-vector form used here (same mathematics as the row form of the paper):
  E   = W_down^T, shape [r, T*d]      so  z = E (x - mu)
  W_t = W_up,t,   shape [d, r]        so  x_hat_t = W_t z + mu_t

Precision: every input is converted to float64 and every operation runs in float64, so bf16
inputs are upcast exactly and the only rounding is fp64 rounding.

Readings taken where the paper is silent (each is listed with its reason in the design notes):
  * mu is optional (None means zero).
  * the softmax scale defaults to 1/sqrt(d_head).
  * the LLA-2D stack is ordered (loop, head, channel).
  * a decode call may append the querying token's own uncompressed loop-t K/V as one more key.
  * prefill row j of a chunk sits at position ctx_len + j and attends latents 0 .. ctx_len + j.
  * sequence lengths are clamped to [0, n_max]; attention over an empty key set returns o = 0 and
    lse = -inf.

Each public function is exercised against closed forms, special cases and library routines by the
CPU test suite; nothing here is left without such a check.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "compression_ratio",
    "cache_scalars_per_token_layer",
    "encode_stack",
    "reconstruct",
    "softmax_attention",
    "encode_into_cache",
    "attend_decode",
    "attend_decode_absorbed",
    "attend_prefill",
]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------------------------
# Cache accounting (Section 3, Eq. 4 and the surrounding text; Section 3 "The LLA-2D variant")
# --------------------------------------------------------------------------------------------

def compression_ratio(T: int, d_head: int, r_k: int, r_v: int) -> float:
    """rho = 2 T d_head / (r_k + r_v)  (Section 3, Eq. 4).

    Per-head LLA: the uncompressed cache holds 2*T*H*d_head scalars per token and layer and LLA
    holds (r_k + r_v)*H; the H cancels. For LLA-2D pass d_head = H*d_head (the stack the 2D
    latent replaces is the full T*H*d_head vector per axis).
    """
    return 2.0 * T * d_head / float(r_k + r_v)


def cache_scalars_per_token_layer(variant: str, H: int, T: int, d_head: int, r_k: int, r_v: int):
    """(uncompressed, compressed) cached scalars per token per layer.

    Uncompressed: 2*T*H*d_head (Section 3, after Eq. 1). Per-head LLA: (r_k + r_v)*H (text of
    Eq. 4). LLA-2D: (r_k + r_v), a factor H below per-head (Section 3, "The LLA-2D variant").
    """
    full = 2 * T * H * d_head
    if variant == "per_head":
        return full, (r_k + r_v) * H
    if variant == "2d":
        return full, (r_k + r_v)
    raise ValueError(variant)


# --------------------------------------------------------------------------------------------
# Codec (Section 3, Eqs. 1-3)
# --------------------------------------------------------------------------------------------

def encode_stack(x_stack, E, mu=None):
    """Eq. 2 in column form: z = E (x - mu).

    x_stack: [..., T*d] loop-major stack of Eq. 1. E: [r, T*d]. mu: [T*d] or None.
    Returns z: [..., r] (float64).
    """
    x = _f64(x_stack)
    if mu is not None:
        x = x - _f64(mu)
    return x @ _f64(E).T


def reconstruct(z, W_t, mu_t=None):
    """Eq. 3 in column form: x_hat_t = W_t z + mu_t.

    z: [..., r]. W_t: [d, r]. mu_t: [d] or None. Returns [..., d] (float64).
    """
    out = _f64(z) @ _f64(W_t).T
    if mu_t is not None:
        out = out + _f64(mu_t)
    return out


def softmax_attention(q, K, V, scale):
    """Textbook single-query attention: o = sum_i softmax(scale * K q)_i V_i, and its log-sum-exp.

    q: [d]. K: [n, d]. V: [n, dv]. Returns (o [dv], lse). An empty key set gives (0, -inf).
    """
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64), -math.inf
    s = scale * (K @ q)
    m = np.max(s)
    e = np.exp(s - m)
    den = np.sum(e)
    o = (e / den) @ V
    return o, float(m + math.log(den))


# --------------------------------------------------------------------------------------------
# Encode into the latent cache (Eq. 2, applied after loop T to a finished token)
# --------------------------------------------------------------------------------------------

def encode_into_cache(zk, zv, xk, xv, Ek, Ev, pos, mu_k=None, mu_v=None, variant="per_head"):
    """Encode C finished tokens per sequence and write them at cache slots pos[b] .. pos[b]+C-1.

    per_head: x* [B, C, T, H, d]; E* [H, r, T*d]; mu* [H, T*d] or None; cache z* [B, H, n_max, r].
              For each (b, c, h) the Eq. 1 stack is x[b, c, :, h, :] flattened loop-major.
    2d:       x* [B, C, T, H, d]; E* [r, T*H*d]; mu* [T*H*d] or None; cache z* [B, n_max, r].
              The stack is x[b, c] flattened in (loop, head, channel) order.
    Returns new float64 caches (the inputs are not modified).
    """
    zk = _f64(zk).copy()
    zv = _f64(zv).copy()
    xk = _f64(xk)
    xv = _f64(xv)
    B, C, T, H, d = xk.shape
    pos = np.asarray(pos, dtype=np.int64)
    for b in range(B):
        slots = int(pos[b]) + np.arange(C)
        if variant == "per_head":
            for h in range(H):
                # the Eq. 1 stacks of all C tokens of (b, h), loop-major: [C, T*d]
                sk = xk[b, :, :, h, :].reshape(C, T * d)
                sv = xv[b, :, :, h, :].reshape(C, T * d)
                zk[b, h, slots] = encode_stack(sk, Ek[h], None if mu_k is None else mu_k[h])
                zv[b, h, slots] = encode_stack(sv, Ev[h], None if mu_v is None else mu_v[h])
        elif variant == "2d":
            zk[b, slots] = encode_stack(xk[b].reshape(C, T * H * d), Ek, mu_k)
            zv[b, slots] = encode_stack(xv[b].reshape(C, T * H * d), Ev, mu_v)
        else:
            raise ValueError(variant)
    return zk, zv


# --------------------------------------------------------------------------------------------
# Attention over the latent cache, explicit reconstruction (the definition)
# --------------------------------------------------------------------------------------------

def _loop_slices(variant, Wk, Wv, mu_k, mu_v, t, h, H, d):
    """W^K_t, W^V_t, mu^K_t, mu^V_t restricted to head h (Eq. 3; 2D: rows of head h)."""
    if variant == "per_head":
        wk = Wk[t, h]
        wv = Wv[t, h]
        muk = None if mu_k is None else mu_k[h, t * d:(t + 1) * d]
        muv = None if mu_v is None else mu_v[h, t * d:(t + 1) * d]
    else:
        wk = Wk[t, h * d:(h + 1) * d]
        wv = Wv[t, h * d:(h + 1) * d]
        base = t * H * d + h * d
        muk = None if mu_k is None else mu_k[base:base + d]
        muv = None if mu_v is None else mu_v[base:base + d]
    return wk, wv, muk, muv


def _check_variant(variant):
    if variant not in ("per_head", "2d"):
        raise ValueError(variant)


def round_bf16_via_f32(x):
    """Round to float32, then to bfloat16 (both to nearest even): how a float32 accumulation that is
    stored as bf16 rounds. Returns float64 values."""
    import torch
    t = torch.from_numpy(np.asarray(x, np.float64).astype(np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def attend_decode(q, zk, zv, Wk, Wv, t, seq_lens=None, mu_k=None, mu_v=None,
                  k_self=None, v_self=None, scale=None, variant="per_head", kv_round_bf16=False):
    """Decode-time attention of one new token per sequence at loop t, by explicit reconstruction.

    For each (b, h): rebuild k_i = W^K_t z^K_i + mu^K_t and v_i = W^V_t z^V_i + mu^V_t for every
    cached token i < N_b (Eq. 3), optionally append the token's own loop-t (k_self, v_self), and
    run textbook softmax attention with q. With kv_round_bf16 the rebuilt K and V are stored as
    bf16 before attention (round_bf16_via_f32), as a reconstruct-then-attend decoder that
    materialises them in bf16 does (Section 7's comparator).

    Shapes (per_head): q [B,H,d]; z* [B,H,n_max,r*]; W* [T,H,d,r*]; mu* [H,T*d];
                       k_self/v_self [B,H,d]; seq_lens [B] (None = n_max).
    Shapes (2d):       z* [B,n_max,r*]; W* [T,H*d,r*]; mu* [T*H*d]; the rest as per_head.
    Returns (o [B,H,d], lse [B,H]) in float64.
    """
    _check_variant(variant)
    q = _f64(q)
    zk, zv, Wk, Wv = _f64(zk), _f64(zv), _f64(Wk), _f64(Wv)
    mu_k, mu_v, k_self, v_self = _f64(mu_k), _f64(mu_v), _f64(k_self), _f64(v_self)
    B, H, d = q.shape
    n_max = zk.shape[2] if variant == "per_head" else zk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, H, d), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for b in range(B):
        n = n_max if seq_lens is None else int(min(max(int(seq_lens[b]), 0), n_max))
        for h in range(H):
            wk, wv, muk, muv = _loop_slices(variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
            lat_k = zk[b, h, :n] if variant == "per_head" else zk[b, :n]
            lat_v = zv[b, h, :n] if variant == "per_head" else zv[b, :n]
            K = reconstruct(lat_k, wk, muk)
            V = reconstruct(lat_v, wv, muv)
            if kv_round_bf16:
                K, V = round_bf16_via_f32(K), round_bf16_via_f32(V)
            if k_self is not None:
                K = np.concatenate([K, k_self[b, h][None, :]], axis=0)
                V = np.concatenate([V, v_self[b, h][None, :]], axis=0)
            o[b, h], lse[b, h] = softmax_attention(q[b, h], K, V, scale)
    return o, lse


def attend_decode_absorbed(q, zk, zv, Wk, Wv, t, seq_lens=None, mu_k=None, mu_v=None,
                           k_self=None, v_self=None, scale=None, variant="per_head"):
    """The same decode attention computed in the absorbed form of Section 7.

    Scores use q~ = W^K_t^T q against the latents (plus q . mu^K_t, which the bilinear identity
    leaves as a per-query constant), the softmax weights are applied to the latents, and W^V_t is
    applied once to the weighted latent sum (mu^V_t enters with the total latent weight).
    Kept beside the explicit form so the identity can be checked on the CPU; same signature and
    return as attend_decode.
    """
    _check_variant(variant)
    q = _f64(q)
    zk, zv, Wk, Wv = _f64(zk), _f64(zv), _f64(Wk), _f64(Wv)
    mu_k, mu_v, k_self, v_self = _f64(mu_k), _f64(mu_v), _f64(k_self), _f64(v_self)
    B, H, d = q.shape
    n_max = zk.shape[2] if variant == "per_head" else zk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, H, d), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for b in range(B):
        n = n_max if seq_lens is None else int(min(max(int(seq_lens[b]), 0), n_max))
        for h in range(H):
            wk, wv, muk, muv = _loop_slices(variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
            lat_k = zk[b, h, :n] if variant == "per_head" else zk[b, :n]
            lat_v = zv[b, h, :n] if variant == "per_head" else zv[b, :n]
            q_lat = wk.T @ q[b, h]
            beta = 0.0 if muk is None else float(q[b, h] @ muk)
            s = scale * (lat_k @ q_lat + beta)
            if k_self is not None:
                s = np.concatenate([s, [scale * float(q[b, h] @ k_self[b, h])]])
            if s.shape[0] == 0:
                o[b, h] = 0.0
                lse[b, h] = -math.inf
                continue
            m = np.max(s)
            e = np.exp(s - m)
            e_lat = e[:n]
            a = e_lat @ lat_v
            num = wv @ a
            if muv is not None:
                num = num + np.sum(e_lat) * muv
            if k_self is not None:
                num = num + e[n] * v_self[b, h]
            den = np.sum(e)
            o[b, h] = num / den
            lse[b, h] = m + math.log(den)
    return o, lse


def attend_prefill(q, zk, zv, Wk, Wv, t, ctx_lens, mu_k=None, mu_v=None, scale=None,
                   variant="per_head"):
    """Chunked-prefill attention at loop t over the latent cache, by explicit reconstruction.

    The chunk's own C tokens have already been encoded into slots ctx_len .. ctx_len + C - 1
    (the two-pass decoder of Appendix A, "Decoding and caching": encode, then attend). Query row
    j sits at position ctx_len + j and attends latents 0 .. ctx_len + j inclusive (causal).

    q [B,C,H,d]; caches and factors as attend_decode. Returns o [B,C,H,d] (float64).
    """
    _check_variant(variant)
    q = _f64(q)
    zk, zv, Wk, Wv = _f64(zk), _f64(zv), _f64(Wk), _f64(Wv)
    mu_k, mu_v = _f64(mu_k), _f64(mu_v)
    B, C, H, d = q.shape
    n_max = zk.shape[2] if variant == "per_head" else zk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, C, H, d), dtype=np.float64)
    for b in range(B):
        base = int(ctx_lens[b])
        for h in range(H):
            wk, wv, muk, muv = _loop_slices(variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
            lat_k = zk[b, h] if variant == "per_head" else zk[b]
            lat_v = zv[b, h] if variant == "per_head" else zv[b]
            # rebuild once for every position this head's chunk can see
            last = min(base + C, n_max)
            K = reconstruct(lat_k[:last], wk, muk)
            V = reconstruct(lat_v[:last], wv, muv)
            for j in range(C):
                n = min(base + j + 1, n_max)
                o[b, j, h], _ = softmax_attention(q[b, j, h], K[:n], V[:n], scale)
    return o


def streaming_kept_slots(n, sink, window):
    """Slots that a StreamingLLM-style eviction policy keeps out of n cached tokens.

    The first `sink` tokens (attention sinks) and the `window` most recent ones, each slot once, in
    increasing order. The paper composes LLA with this sequence-axis eviction (Section 7,
    "Memory, capacity and latency": a 1024-token budget on top of the 21.3x codec; Appendix C,
    Table 9: sink 4 + window 256).
    """
    n = max(int(n), 0)
    keep = set(range(min(int(sink), n))) | set(range(max(n - int(window), 0), n))
    return sorted(keep)


def attend_decode_gather(q, zk, zv, Wk, Wv, t, slots, counts=None, mu_k=None, mu_v=None,
                         k_self=None, v_self=None, scale=None, variant="per_head"):
    """Decode attention at loop t over a listed subset of the cached latents (token eviction
    composed with LLA: Section 7, "Memory, capacity and latency", and Appendix C).

    Row b attends the cached tokens at slots[b, 0 .. counts[b]-1] (counts clamped to [0, budget],
    None meaning the whole budget), in any order, plus the optional self token. A slot outside
    [0, n_max) is skipped; a slot listed twice is two keys. Each listed key is rebuilt explicitly
    (Eq. 3) and attended with textbook softmax.

    slots [B, budget] int; counts [B] int or None; the rest as attend_decode.
    Returns (o [B,H,d], lse [B,H]) in float64.
    """
    _check_variant(variant)
    q = _f64(q)
    zk, zv, Wk, Wv = _f64(zk), _f64(zv), _f64(Wk), _f64(Wv)
    mu_k, mu_v, k_self, v_self = _f64(mu_k), _f64(mu_v), _f64(k_self), _f64(v_self)
    slots = np.asarray(slots)
    B, H, d = q.shape
    budget = slots.shape[1]
    n_max = zk.shape[2] if variant == "per_head" else zk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, H, d), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for b in range(B):
        cnt = budget if counts is None else int(min(max(int(counts[b]), 0), budget))
        listed = [int(s) for s in slots[b, :cnt] if 0 <= int(s) < n_max]
        for h in range(H):
            wk, wv, muk, muv = _loop_slices(variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
            lat_k = zk[b, h] if variant == "per_head" else zk[b]
            lat_v = zv[b, h] if variant == "per_head" else zv[b]
            K = reconstruct(lat_k[listed], wk, muk)
            V = reconstruct(lat_v[listed], wv, muv)
            if k_self is not None:
                K = np.concatenate([K, k_self[b, h][None, :]], axis=0)
                V = np.concatenate([V, v_self[b, h][None, :]], axis=0)
            o[b, h], lse[b, h] = softmax_attention(q[b, h], K, V, scale)
    return o, lse


# --------------------------------------------------------------------------------------------
# Low-bit latent storage: the precision axis stacked on the loop axis (Section 8,
# "Compositionality": quantisation changes a different tensor dimension and can be stacked;
# Appendix C evaluates an 8-bit codec)
# --------------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(v):
    """Round to the nearest OCP FP8 E4M3 value (4 exponent bits with bias 7, 3 mantissa bits,
    subnormals, largest finite 448, no infinities), ties to even.

    Inside a binade [2^e, 2^(e+1)) with e >= -6 the spacing is 2^(e-3); below 2^-6 it is the
    subnormal spacing 2^-9. A value whose rounding would exceed 448 has no E4M3 encoding and
    becomes NaN. Returns float64 values.
    """
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = 2.0 ** (e - 3)
    r = np.round(a / step) * step  # numpy rounds halves to even; a / step is exact
    r = np.where(r > E4M3_MAX, np.nan, r)
    return np.copysign(r, v)


def quantize_latent_rows(z):
    """Low-bit latent rows: each row of r latent values (the last axis) is stored as r E4M3 codes
    and one float32 scale s = max|z| / 448, code_j = e4m3(z_j / s), both divisions in float32
    (a row of zeros has s = 0 and zero codes). Returns (codes as float64 values, scales as float64
    holding float32 values)."""
    z32 = np.asarray(z, np.float32)
    amax = np.max(np.abs(z32), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    v = (z32 / safe[..., None]).astype(np.float32)
    codes = e4m3_round(v.astype(np.float64))
    codes = np.where((s > 0)[..., None], codes, 0.0)
    return codes, s.astype(np.float64)


def dequantize_latent_rows(codes, scales):
    """The latent values a low-bit row stands for: code_j * s (exact in float64)."""
    return np.asarray(codes, np.float64) * np.asarray(scales, np.float64)[..., None]


INT8_MAX = 127.0


def quantize_latent_rows_int8(z):
    """Low-bit latent rows, integer form: each row of r latent values (the last axis) is stored as r
    signed 8-bit codes and one float32 scale s = max|z| / 127, code_j = round(z_j / s) with halves
    to even, both divisions in float32 (a row of zeros has s = 0 and zero codes). Symmetric: the
    codes lie in [-127, 127]. Returns (codes as float64 values, scales as float64 holding float32
    values)."""
    z32 = np.asarray(z, np.float32)
    amax = np.max(np.abs(z32), axis=-1)
    s = (amax / np.float32(INT8_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    v = (z32 / safe[..., None]).astype(np.float32)
    codes = np.clip(np.rint(v.astype(np.float64)), -INT8_MAX, INT8_MAX)  # rint: halves to even
    codes = np.where((s > 0)[..., None], codes, 0.0)
    return codes, s.astype(np.float64)


# --------------------------------------------------------------------------------------------
# Decoupled RoPE branch (Section 7, "Per-head LLA versus LLA-2D at inference": an MLA-style split
# into the NoPE latent content path and a small explicit rotary branch, shared across recurrence
# steps for a token; Section 3, "RoPE and reconstruction")
# --------------------------------------------------------------------------------------------

def rope_rotate(x, pos, base=10000.0):
    """Rotary position embedding (Su et al., 2021, RoFormer): channel pairs (2i, 2i+1) of a d-wide
    vector at position p are rotated by the angle p * base^(-2i/d).

    x [..., d] with d even; pos broadcastable to x.shape[:-1]. Returns float64.
    """
    x = _f64(x)
    d = x.shape[-1]
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    ang = np.asarray(pos, np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def attend_decode_rope(q, q_rope, zk, zv, k_rope, Wk, Wv, t, seq_lens=None, mu_k=None, mu_v=None,
                       k_self=None, v_self=None, k_rope_self=None, base=10000.0, scale=None,
                       variant="per_head"):
    """Decode attention with the decoupled rotary branch, by explicit reconstruction.

    Key i < N_b is the concatenation of its rebuilt content key k_i = W^K_t z^K_i + mu^K_t (Eq. 3)
    and its cached rotary key k_rope[b, i], which is stored already rotated at position i. The
    query is [q ; rope(q_rope, N_b)] (the decoding token sits at position N_b); the optional self
    key is [k_self ; rope(k_rope_self, N_b)]. Values are the rebuilt content values only. Scale
    defaults to 1/sqrt(d_head + d_rope) (the concatenated key width, as in MLA).

    q_rope [B,H,d_r]; k_rope [B,n_max,d_r] (one rotary key per token, shared by heads and loops);
    k_rope_self [B,d_r]; the rest as attend_decode. Returns (o [B,H,d], lse [B,H]).
    """
    _check_variant(variant)
    q, q_rope = _f64(q), _f64(q_rope)
    zk, zv, Wk, Wv, k_rope = _f64(zk), _f64(zv), _f64(Wk), _f64(Wv), _f64(k_rope)
    mu_k, mu_v, k_self, v_self = _f64(mu_k), _f64(mu_v), _f64(k_self), _f64(v_self)
    k_rope_self = _f64(k_rope_self)
    B, H, d = q.shape
    dr = q_rope.shape[-1]
    n_max = zk.shape[2] if variant == "per_head" else zk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d + dr)
    o = np.zeros((B, H, d), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for b in range(B):
        n = n_max if seq_lens is None else int(min(max(int(seq_lens[b]), 0), n_max))
        qr = rope_rotate(q_rope[b], n, base)  # [H, d_r]
        krs = None if k_rope_self is None else rope_rotate(k_rope_self[b], n, base)
        for h in range(H):
            wk, wv, muk, muv = _loop_slices(variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
            lat_k = zk[b, h, :n] if variant == "per_head" else zk[b, :n]
            lat_v = zv[b, h, :n] if variant == "per_head" else zv[b, :n]
            K = np.concatenate([reconstruct(lat_k, wk, muk), k_rope[b, :n]], axis=1)
            V = reconstruct(lat_v, wv, muv)
            if k_self is not None:
                K = np.concatenate([K, np.concatenate([k_self[b, h], krs])[None, :]], axis=0)
                V = np.concatenate([V, v_self[b, h][None, :]], axis=0)
            o[b, h], lse[b, h] = softmax_attention(np.concatenate([q[b, h], qr[h]]), K, V, scale)
    return o, lse


def attend_prefill_rope(q, q_rope, zk, zv, k_rope, Wk, Wv, t, ctx_lens, mu_k=None, mu_v=None,
                        base=10000.0, scale=None, variant="per_head"):
    """Chunked-prefill attention with the decoupled rotary branch, by explicit reconstruction.

    Row j of sequence b sits at position ctx_lens[b] + j and attends latents 0 .. ctx_lens[b] + j
    (the chunk's own latents and rotary keys are already cached, as in attend_prefill). Key i is
    [rebuilt content key ; k_rope[b, i]] (rotary keys stored rotated at their slot), the row's
    query is [q ; rope(q_rope, its position)], values are the content values. Scale defaults to
    1/sqrt(d_head + d_rope).

    q [B,C,H,d]; q_rope [B,C,H,d_r]; k_rope [B,n_max,d_r]; the rest as attend_prefill.
    Returns o [B,C,H,d].
    """
    _check_variant(variant)
    q, q_rope = _f64(q), _f64(q_rope)
    zk, zv, Wk, Wv, k_rope = _f64(zk), _f64(zv), _f64(Wk), _f64(Wv), _f64(k_rope)
    mu_k, mu_v = _f64(mu_k), _f64(mu_v)
    B, C, H, d = q.shape
    dr = q_rope.shape[-1]
    n_max = zk.shape[2] if variant == "per_head" else zk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d + dr)
    o = np.zeros((B, C, H, d), dtype=np.float64)
    for b in range(B):
        base_pos = int(ctx_lens[b])
        last = min(base_pos + C, n_max)
        for h in range(H):
            wk, wv, muk, muv = _loop_slices(variant, Wk, Wv, mu_k, mu_v, t, h, H, d)
            lat_k = zk[b, h] if variant == "per_head" else zk[b]
            lat_v = zv[b, h] if variant == "per_head" else zv[b]
            K = np.concatenate([reconstruct(lat_k[:last], wk, muk), k_rope[b, :last]], axis=1)
            V = reconstruct(lat_v[:last], wv, muv)
            for j in range(C):
                pos = base_pos + j
                n = min(pos + 1, n_max)
                qq = np.concatenate([q[b, j, h], rope_rotate(q_rope[b, j, h], pos, base)])
                o[b, j, h], _ = softmax_attention(qq, K[:n], V[:n], scale)
    return o
