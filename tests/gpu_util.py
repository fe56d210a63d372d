"""Helpers for the GPU parity tests: device transfer, comparison and the tolerances.

Tolerances (norm-wise per call output, max|gpu - ref| / max|ref|):
  fp32 storage: 1e-5 (fp32 accumulation of exact fp32 inputs);
  bf16 storage: 1e-2 (bf16 inputs are exact on both sides; the GPU rounds its result to bf16 once,
                a relative change of at most 2^-9, plus fp32 accumulation).
lse is always float32: |gpu - ref| <= 2e-5 * max(1, |ref|).
"""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla

TOL = {"f32": 1e-5, "bf16": 1e-2}
LSE_TOL = 2e-5

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
LLA_DT = {"f32": lla.LLA_F32, "bf16": lla.LLA_BF16}
LLA_VAR = {"per_head": lla.LLA_PER_HEAD, "2d": lla.LLA_2D}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import os
    if not os.path.exists(lla.LIB_PATH):
        pytest.fail("liblla.so is not built; the GPU tests need the HIP library")


def dev(a, dtype="f32"):
    """numpy (float32 holding storage values) -> device tensor of the storage dtype (exact)."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype in (torch.int32, torch.int64):
        return t.to(torch.int32).cuda()
    return t.to(TORCH_DT[dtype]).cuda().contiguous()


def host(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


def assert_close(got, ref, dtype, what=""):
    e = rel_err(got, ref)
    assert e <= TOL[dtype], f"{what}: relative error {e:.3e} > {TOL[dtype]:.0e}"
    return e


def assert_lse(got, ref, what="", slack=None):
    """lse within LSE_TOL * max(1, |lse|), plus an optional per-element absolute slack (the score
    error bound of a path that rounds its query, mfma_lse_slack)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf pattern differs"
    sl = np.zeros_like(ref) if slack is None else np.broadcast_to(np.asarray(slack, np.float64), ref.shape)
    g, r, sl = got[~inf_ref], ref[~inf_ref], sl[~inf_ref]
    if g.size:
        err = np.max((np.abs(g - r) - sl) / np.maximum(1.0, np.abs(r)))
        assert err <= LSE_TOL, f"{what}: lse error {err:.3e}"


def mfma_lse_slack(q, zk, Wk, t, lens, scale=None, q_rope=None, k_rope=None):
    """Absolute lse slack per (b, h) for the LLA-2D MFMA read. Its scores take q~ = W^K_t[h]^T q as
    a bf16 pair (hi + lo: each entry within 2^-18 of q~_j, relative) times bf16 latents, summed in
    fp32, so |ds_i| <= 2^-16 * scale * sum_j |q~_j z_ij| <= 2^-16 * scale * |q~| * |z_i| (Cauchy-
    Schwarz), and the lse moves by at most max_i |ds_i|. With a few keys and a sharpened query
    sum_j |q~_j z_ij| can exceed |lse| many times over, which a bound relative to |lse| misses.
    With the fused rotary branch the rotated rotary query is split the same way, adding
    |q_R| * |k_R,i| per key (rotation keeps norms), and the default scale is 1/sqrt(d + d_rope).
    q [B][H][d], zk [B][n][r], Wk [T][H*d][r], q_rope [B][H][d_rope], k_rope [B][n][d_rope]
    (float64 copies of the device values)."""
    B, H, d = q.shape
    qt = np.einsum("bhd,hdr->bhr", np.asarray(q, np.float64), np.asarray(Wk[t], np.float64).reshape(H, d, -1))
    qn = np.linalg.norm(qt, axis=-1)
    zn = np.linalg.norm(np.asarray(zk, np.float64), axis=-1)
    rope = q_rope is not None
    if rope:
        qrn = np.linalg.norm(np.asarray(q_rope, np.float64), axis=-1)
        krn = np.linalg.norm(np.asarray(k_rope, np.float64), axis=-1)
    out = np.zeros((B, H))
    for b in range(B):
        n = min(max(int(lens[b]), 0), zk.shape[1])
        if n:
            per_key = qn[b][:, None] * zn[b, :n][None, :]
            if rope:
                per_key = per_key + qrn[b][:, None] * krn[b, :n][None, :]
            out[b] = per_key.max(axis=1)
    d_all = d + (np.asarray(q_rope).shape[-1] if rope else 0)
    return 2.0 ** -16 * (scale if scale else 1.0 / np.sqrt(d_all)) * out


def desc_for(s, n_max=None, scale=0.0):
    return lla.make_desc(LLA_VAR[s.variant], LLA_DT[s.dtype], s.H, s.d, s.T, s.r_k, s.r_v,
                         s.n_max if n_max is None else n_max, scale)


def _bf16_rne(x):
    """float64 -> float32 -> bf16 (round to nearest even), returned as float64."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def rebuild_flip_lse_slack(q, zk, Wk, t, lens, mu_k=None, scale=None):
    """Absolute lse slack per (b, h) for reconstruct-then-attend. The comparator rounds each rebuilt
    K entry k = W^K_t z + mu to bf16 from an fp32 MFMA sum; the oracle rounds the exact value. The
    two can land one bf16 step apart only where k lies within the fp32 sum's error bound
    (r * 2^-24 * sum_l |W_jl z_l|, plus 2^-24 |k| for adding mu) of a rounding midpoint. Such
    entries may move score i by scale * sum_j |q_j| * step(k_ij), and the lse by at most the largest
    such move. q [B][H][d], zk [B][H][n][r], Wk [T][H][d][r], mu_k [H][T*d] or None (float64)."""
    q = np.asarray(q, np.float64)
    B, H, d = q.shape
    W = np.asarray(Wk[t], np.float64)                     # [H][d][r]
    r = W.shape[-1]
    out = np.zeros((B, H))
    for b in range(B):
        n = min(max(int(lens[b]), 0), zk.shape[2])
        if n == 0:
            continue
        z = np.asarray(zk[b, :, :n], np.float64)          # [H][n][r]
        k = np.einsum("hdr,hnr->hnd", W, z)
        mag = np.einsum("hdr,hnr->hnd", np.abs(W), np.abs(z))
        if mu_k is not None:
            k = k + np.asarray(mu_k, np.float64)[:, t * d:(t + 1) * d][:, None, :]
        kb = _bf16_rne(k)
        e = np.floor(np.log2(np.maximum(np.abs(kb), np.finfo(np.float32).tiny)))
        step = 2.0 ** (e - 7)                              # one bf16 step at kb's binade
        dist = np.minimum(np.abs(k - (kb - step / 2)), np.abs(k - (kb + step / 2)))
        flip = dist <= r * 2.0 ** -24 * mag + 2.0 ** -24 * np.abs(k)
        per_key = np.einsum("hd,hnd->hn", np.abs(q[b]), np.where(flip, 2 * step, 0.0))
        out[b] = per_key.max(axis=1)
    return (scale if scale else 1.0 / np.sqrt(d)) * out
