"""GPU parity: the HIP library (through the C ABI) against the CPU oracle, element by element.

Small shapes span several tiles, several token splits and a ragged tail; the five synthetic
workloads run at full size with outputs sampled where the oracle would be too slow. Tolerances
are in tests/gpu_util.py.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import (LLA_DT, LLA_VAR, assert_close, assert_lse, dev, host, mfma_lse_slack, rel_err,
                            require_gpu)

pytestmark = pytest.mark.gpu

PAIRS = [(8, 8), (16, 16), (24, 24), (32, 32), (64, 64), (96, 96), (128, 128), (96, 160),
         (256, 256)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def mk_desc(variant, dtype, H, d, T, rk, rv, n_max, scale=0.0):
    return lla.make_desc(LLA_VAR[variant], LLA_DT[dtype], H, d, T, rk, rv, n_max, scale)


def gpu_decode(desc, B, t, c, dtype, lens, self_token=True, mu=True, want_lse=True):
    """Run lla_attend_decode on device copies of case c at loop t; returns (o, lse) on host."""
    H, d = desc.H, desc.d_head
    q = dev(c["q"][t], dtype)
    out = torch.empty_like(q)
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda") if want_lse else None
    ws = lla.workspace(desc, B, 1)
    ks = dev(c["k_self"][t], dtype) if self_token else None
    vs = dev(c["v_self"][t], dtype) if self_token else None
    lla.lla_attend_decode(desc, B, t, q, c["_zk"], c["_zv"], dev(lens), c["_Wk"], c["_Wv"],
                          c["_muk"] if mu else None, c["_muv"] if mu else None, ks, vs, out, lse, ws)
    torch.cuda.synchronize()
    return host(out), (host(lse) if want_lse else None)


def upload(c, dtype):
    for k in ("zk", "zv", "Wk", "Wv"):
        c["_" + k] = dev(c[k], dtype)
    c["_muk"] = dev(c["mu_k"], dtype)
    c["_muv"] = dev(c["mu_v"], dtype)
    return c


def oracle_decode(c, t, lens, variant, self_token=True, mu=True, b_sel=None, absorbed=False):
    fn = O.attend_decode_absorbed if absorbed else O.attend_decode
    sl = slice(None) if b_sel is None else b_sel
    return fn(c["q"][t][sl], c["zk"][sl], c["zv"][sl], c["Wk"], c["Wv"], t, np.asarray(lens)[sl],
              c["mu_k"] if mu else None, c["mu_v"] if mu else None,
              c["k_self"][t][sl] if self_token else None, c["v_self"][t][sl] if self_token else None,
              variant=variant)


# --------------------------------------------------------------------------------------------
# shape sweep: every compiled rank pair, both storage types, ragged lengths, split-K
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rk,rv", PAIRS)
def test_decode_sweep_per_head(dtype, rk, rv):
    B, H, d, T, n_max = 3, 2, 64, 3, 3001
    lens = [3001, 517, 0]
    for gain, mu, self_token in ((1.0, True, True), (8.0, False, True), (1.0, True, False)):
        c = upload(synth.random_case("per_head", dtype, B, H, d, T, rk, rv, n_max,
                                     7000 + rk + rv, with_mu=mu, q_gain=gain), dtype)
        desc = mk_desc("per_head", dtype, H, d, T, rk, rv, n_max)
        assert lla.lla_workspace_bytes(desc, B) > 0  # 8-wave workgroups, split-K and the combine
        for t in range(T):
            o, lse = gpu_decode(desc, B, t, c, dtype, lens, self_token, mu)
            ro, rl = oracle_decode(c, t, lens, "per_head", self_token, mu)
            what = f"{dtype} r=({rk},{rv}) gain={gain} mu={mu} self={self_token} t={t}"
            assert_close(o, ro, dtype, what)
            assert_lse(lse, rl, what)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rk,rv", [(8, 8), (32, 32), (256, 256)])
def test_decode_sweep_2d(dtype, rk, rv):
    B, H, d, T, n_max = 2, 3, 32, 2, 777
    lens = [777, 130]
    c = upload(synth.random_case("2d", dtype, B, H, d, T, rk, rv, n_max, 7100 + rk), dtype)
    desc = mk_desc("2d", dtype, H, d, T, rk, rv, n_max)
    for t in range(T):
        o, lse = gpu_decode(desc, B, t, c, dtype, lens)
        ro, rl = oracle_decode(c, t, lens, "2d")
        assert_close(o, ro, dtype, f"2d {dtype} t={t}")
        assert_lse(lse, rl, f"2d {dtype} t={t}")


@pytest.mark.parametrize("dtype,rk,rv", [("bf16", 32, 32), ("f32", 8, 8), ("bf16", 96, 160)])
def test_decode_2d_streaming_xcd_grouped(dtype, rk, rv):
    """LLA-2D on the streaming read with B a multiple of 8: every head of a sequence is launched
    onto one XCD (they all stream the same latents); ragged lengths, mu, self token."""
    B, H, d, T, n_max = 16, 5, 32, 2, 1500
    lens = [1500, 1499, 0, 1, 700, 256, 257, 1024, 33, 1200, 64, 65, 900, 5, 511, 512]
    c = upload(synth.random_case("2d", dtype, B, H, d, T, rk, rv, n_max, 7150 + rk + rv, q_gain=4.0), dtype)
    desc = mk_desc("2d", dtype, H, d, T, rk, rv, n_max)
    o, lse = gpu_decode(desc, B, 1, c, dtype, lens)
    ro, rl = oracle_decode(c, 1, lens, "2d")
    assert_close(o, ro, dtype, f"2d streaming xcd {dtype} r=({rk},{rv})")
    assert_lse(lse, rl, f"2d streaming xcd {dtype} r=({rk},{rv})")


@pytest.mark.parametrize("dtype,rk,rv", [("bf16", 24, 24), ("bf16", 8, 8), ("bf16", 256, 256),
                                          ("f32", 24, 24), ("bf16", 96, 96), ("f32", 8, 8)])
def test_decode_batch_and_split_boundaries(dtype, rk, rv):
    """Sequence lengths just below, at and above multiples of the streaming kernel's batch
    (64/lanes-per-token tokens per tile, several tiles per batch, two batches in flight) and of
    the per-wave token range (two waves of 384 tokens at n_max = 700, merged in LDS), so every
    partly and wholly empty batch, and a wave's range that ends inside one, is exercised."""
    H, d, T, n_max = 2, 64, 2, 700
    lens = [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384, 385, 511, 512,
            513, 640, 699, 700]
    B = len(lens)
    c = upload(synth.random_case("per_head", dtype, B, H, d, T, rk, rv, n_max, 7050 + rk,
                                 q_gain=4.0), dtype)
    desc = mk_desc("per_head", dtype, H, d, T, rk, rv, n_max)
    for t in range(T):
        o, lse = gpu_decode(desc, B, t, c, dtype, lens, self_token=(t == 0))
        ro, rl = oracle_decode(c, t, lens, "per_head", self_token=(t == 0))
        assert_close(o, ro, dtype, f"boundaries {dtype} r=({rk},{rv}) t={t}")
        assert_lse(lse, rl, f"boundaries {dtype} r=({rk},{rv}) t={t}")


def test_decode_empty_and_clamped_lengths():
    dtype = "f32"
    B, H, d, T, n_max = 4, 2, 16, 2, 40
    c = upload(synth.random_case("per_head", dtype, B, H, d, T, 8, 8, n_max, 7200), dtype)
    desc = mk_desc("per_head", dtype, H, d, T, 8, 8, n_max)
    lens = [0, 99, -5, 40]
    o, lse = gpu_decode(desc, B, 1, c, dtype, lens, self_token=True)
    ro, rl = oracle_decode(c, 1, lens, "per_head", True)
    assert_close(o, ro, dtype)
    assert_lse(lse, rl)
    np.testing.assert_allclose(o[0], c["v_self"][1][0], rtol=0, atol=1e-6)
    o, lse = gpu_decode(desc, B, 1, c, dtype, lens, self_token=False)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    ro, rl = oracle_decode(c, 1, lens, "per_head", False)
    assert_close(o, ro, dtype)
    assert_lse(lse, rl)


def test_decode_null_seq_lens_means_n_max_and_is_deterministic():
    dtype = "bf16"
    B, H, d, T, n_max = 2, 4, 128, 2, 2000
    c = upload(synth.random_case("per_head", dtype, B, H, d, T, 32, 32, n_max, 7300), dtype)
    desc = mk_desc("per_head", dtype, H, d, T, 32, 32, n_max)
    q = dev(c["q"][0], dtype)
    outs = []
    for _ in range(2):
        out = torch.empty_like(q)
        lla.lla_attend_decode(desc, B, 0, q, c["_zk"], c["_zv"], None, c["_Wk"], c["_Wv"],
                              c["_muk"], c["_muv"], None, None, out, None, lla.workspace(desc, B))
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    ro, _ = oracle_decode(c, 0, [n_max] * B, "per_head", False)
    assert_close(host(outs[0]), ro, dtype)


# --------------------------------------------------------------------------------------------
# encode
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant,H,d,T,r", [("per_head", 3, 32, 4, 24), ("per_head", 2, 96, 32, 96),
                                             ("2d", 2, 16, 3, 32), ("per_head", 2, 64, 2, 160)])
def test_encode(dtype, variant, H, d, T, r):
    B, C, n_max = 3, 5, 12
    pos = np.array([0, 7, 10], np.int32)  # sequence 2 runs past the end: slots 12.. are skipped
    g = np.random.default_rng(r + T)
    xk = synth.normal((B, C, T, H, d), 900 + r, dtype)
    xv = synth.normal((B, C, T, H, d), 901 + r, dtype)
    K = T * d if variant == "per_head" else T * H * d
    es = (H, r, K) if variant == "per_head" else (r, K)
    ms = (H, K) if variant == "per_head" else (K,)
    zs = (B, H, n_max, r) if variant == "per_head" else (B, n_max, r)
    Ek = synth.normal(es, 902 + r, dtype, 1 / math.sqrt(K))
    Ev = synth.normal(es, 903 + r, dtype, 1 / math.sqrt(K))
    mk = synth.normal(ms, 904 + r, dtype, 0.5)
    mv = synth.normal(ms, 905 + r, dtype, 0.5)
    z0 = synth.normal(zs, 906 + r, dtype)  # pre-existing cache contents must survive
    desc = mk_desc(variant, dtype, H, d, T, r, r, n_max)
    for mu in (True, False):
        zk, zv = dev(z0, dtype), dev(z0, dtype)
        lla.lla_encode(desc, B, C, dev(xk, dtype), dev(xv, dtype), dev(Ek, dtype), dev(Ev, dtype),
                       dev(mk, dtype) if mu else None, dev(mv, dtype) if mu else None, dev(pos),
                       zk, zv)
        torch.cuda.synchronize()
        # oracle writes only the in-range slots, like the kernel
        keep = np.array([min(C, n_max - p) for p in pos])
        rk_, rv_ = z0.copy(), z0.copy()
        for b in range(B):
            sub = slice(b, b + 1)
            a, bb = O.encode_into_cache(z0[sub], z0[sub], xk[sub, :keep[b]], xv[sub, :keep[b]], Ek, Ev,
                                        pos[sub], mk if mu else None, mv if mu else None, variant)
            rk_[sub], rv_[sub] = a, bb
        assert_close(host(zk), rk_, dtype, f"encode zk {variant} mu={mu}")
        assert_close(host(zv), rv_, dtype, f"encode zv {variant} mu={mu}")
        # untouched slots are bit-identical
        mask = np.ones(zs[:-1], bool)
        for b in range(B):
            for cc in range(keep[b]):
                if variant == "per_head":
                    mask[b, :, pos[b] + cc] = False
                else:
                    mask[b, pos[b] + cc] = False
        assert np.array_equal(host(zk)[mask], z0.astype(np.float64)[mask])


# --------------------------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant,rk,rv", [("per_head", 24, 24), ("per_head", 96, 160), ("2d", 32, 32)])
def test_prefill(dtype, variant, rk, rv):
    B, C, H, d, T, n_max = 2, 37, 3, 32, 2, 400
    ctx = np.array([300, 0], np.int32)
    c = upload(synth.random_case(variant, dtype, B, H, d, T, rk, rv, n_max, 7400 + rk), dtype)
    q = synth.normal((B, C, H, d), 7401, dtype)
    desc = mk_desc(variant, dtype, H, d, T, rk, rv, n_max)
    for t in range(T):
        out = torch.empty(B, C, H, d, dtype=dev(q, dtype).dtype, device="cuda")
        lla.lla_attend_prefill(desc, B, C, t, dev(q, dtype), c["_zk"], c["_zv"], dev(ctx), c["_Wk"],
                               c["_Wv"], c["_muk"], c["_muv"], out, lla.workspace(desc, B, C))
        torch.cuda.synchronize()
        ref = O.attend_prefill(q, c["zk"], c["zv"], c["Wk"], c["Wv"], t, ctx, c["mu_k"], c["mu_v"],
                               variant=variant)
        assert_close(host(out), ref, dtype, f"prefill {variant} t={t}")


# --------------------------------------------------------------------------------------------
# the tiny fp32 workload: encode the 64-token context, decode with the self token, encode it
# --------------------------------------------------------------------------------------------

def test_tiny_fp32_pipeline():
    s = synth.CASES["tiny_fp32"]
    c = synth.tiny_fp32_case(s)
    B, H, d, T, N, r = s.B, s.H, s.d, s.T, s.N, s.r_k
    n_max = N + 1
    desc = mk_desc("per_head", "f32", H, d, T, r, r, n_max)
    dt = "f32"
    zk = torch.zeros(B, H, n_max, r, device="cuda")
    zv = torch.zeros_like(zk)
    # context: 64 tokens encoded from their per-loop trajectories
    lla.lla_encode(desc, B, N, dev(c["xk"][:, :N]), dev(c["xv"][:, :N]), dev(c["Ek"]), dev(c["Ev"]),
                   None, None, dev(np.zeros(B, np.int32)), zk, zv)
    z0 = np.zeros((B, H, n_max, r))
    rzk, rzv = O.encode_into_cache(z0, z0, c["xk"][:, :N], c["xv"][:, :N], c["Ek"], c["Ev"], [0])
    assert_close(host(zk), rzk, dt, "context encode")
    assert_close(host(zv), rzv, dt, "context encode")
    lens = np.full(B, N, np.int32)
    for t in range(T):
        q = dev(c["q"][t])
        ks = dev(c["xk"][:, N, t])  # the new token's own loop-t K/V, uncompressed
        vs = dev(c["xv"][:, N, t])
        out = torch.empty_like(q)
        lse = torch.empty(B, H, device="cuda")
        lla.lla_attend_decode(desc, B, t, q, zk, zv, dev(lens), dev(c["Wk"]), dev(c["Wv"]), None,
                              None, ks, vs, out, lse, lla.workspace(desc, B))
        torch.cuda.synchronize()
        ro, rl = O.attend_decode(c["q"][t], rzk, rzv, c["Wk"], c["Wv"], t, lens, None, None,
                                 c["xk"][:, N, t], c["xv"][:, N, t])
        assert_close(host(out), ro, dt, f"tiny decode t={t}")
        assert_lse(host(lse), rl, f"tiny decode t={t}")
    # after loop T the new token's 4 K/V vectors are folded into slot 64
    lla.lla_encode(desc, B, 1, dev(c["xk"][:, N:N + 1]), dev(c["xv"][:, N:N + 1]), dev(c["Ek"]),
                   dev(c["Ev"]), None, None, dev(lens), zk, zv)
    rzk, rzv = O.encode_into_cache(rzk, rzv, c["xk"][:, N:N + 1], c["xv"][:, N:N + 1], c["Ek"], c["Ev"], lens)
    assert_close(host(zk), rzk, dt, "new-token encode")
    assert_close(host(zv), rzv, dt, "new-token encode")
    # a second step reads all 65 latents
    q2 = synth.normal((B, H, d), 5555)
    out = torch.empty(B, H, d, device="cuda")
    lla.lla_attend_decode(desc, B, 2, dev(q2), zk, zv, dev(lens + 1), dev(c["Wk"]), dev(c["Wv"]),
                          None, None, None, None, out, None, lla.workspace(desc, B))
    torch.cuda.synchronize()
    ro, _ = O.attend_decode(q2, rzk, rzv, c["Wk"], c["Wv"], 2, lens + 1)
    assert_close(host(out), ro, dt, "second step")


# --------------------------------------------------------------------------------------------
# full-size workloads (sampled rows where the oracle is slow)
# --------------------------------------------------------------------------------------------

@pytest.mark.timeout(600)
@pytest.mark.parametrize("mu", [False, True])
def test_ouro_layer_full_size(mu):
    """One Ouro-1.4B-shaped layer at full size (B=32, N=4096, r=32): every row of the batch and
    every loop against the explicit-reconstruction oracle, without and with the calibration mean,
    then the encode of the new token into slot N."""
    s = synth.CASES["ouro_layer"]
    c = upload(synth.host_case(s, with_mu=mu), s.dtype)
    desc = mk_desc("per_head", s.dtype, s.H, s.d, s.T, s.r_k, s.r_v, s.n_max)
    lens = c["seq_lens"]
    for t in range(s.T):
        o, lse = gpu_decode(desc, s.B, t, c, s.dtype, lens, True, mu)
        ro, rl = oracle_decode(c, t, lens, "per_head", True, mu)
        assert_close(o, ro, s.dtype, f"ouro mu={mu} t={t}")
        assert_lse(lse, rl, f"ouro mu={mu} t={t}")
    # encode of the new token into slot N for every sequence
    zk, zv = c["_zk"], c["_zv"]
    lla.lla_encode(desc, s.B, 1, dev(c["xk"], s.dtype), dev(c["xv"], s.dtype), dev(c["Ek"], s.dtype),
                   dev(c["Ev"], s.dtype), c["_muk"] if mu else None, c["_muv"] if mu else None,
                   dev(lens), zk, zv)
    torch.cuda.synchronize()
    for ax, x, E, m, z in (("k", c["xk"], c["Ek"], c["mu_k"], zk), ("v", c["xv"], c["Ev"], c["mu_v"], zv)):
        got = host(z[:, :, s.N])
        ref = np.stack([[O.encode_stack(x[b, 0, :, h, :].reshape(-1), E[h], None if m is None else m[h])
                         for h in range(s.H)] for b in range(s.B)])
        assert_close(got, ref, s.dtype, f"ouro encode {ax} mu={mu}")


def _fill_device_case(s, layer=0, mu=False):
    """Device-resident inputs of a large workload (latents from a seeded device generator)."""
    dt = torch.bfloat16
    g = {}
    zshape_k = (s.B, s.H, s.n_max, s.r_k) if s.variant == "per_head" else (s.B, s.n_max, s.r_k)
    zshape_v = (s.B, s.H, s.n_max, s.r_v) if s.variant == "per_head" else (s.B, s.n_max, s.r_v)
    g["zk"] = synth.device_normal_(torch.empty(zshape_k, dtype=dt, device="cuda"), synth.seed(s.case, synth.SEED_ZK, layer))
    g["zv"] = synth.device_normal_(torch.empty(zshape_v, dtype=dt, device="cuda"), synth.seed(s.case, synth.SEED_ZV, layer))
    if s.variant == "per_head":
        Wk = synth.orthonormal_W(s.T, s.H, s.d, s.r_k, synth.seed(s.case, synth.SEED_WK, layer), "bf16")
        Wv = synth.orthonormal_W(s.T, s.H, s.d, s.r_v, synth.seed(s.case, synth.SEED_WV, layer), "bf16")
        mu_shape = (s.H, s.T * s.d)
    else:
        Wk = synth.orthonormal_W_2d(s.T, s.H, s.d, s.r_k, synth.seed(s.case, synth.SEED_WK, layer), "bf16")
        Wv = synth.orthonormal_W_2d(s.T, s.H, s.d, s.r_v, synth.seed(s.case, synth.SEED_WV, layer), "bf16")
        mu_shape = (s.T * s.H * s.d,)
    g["Wk"], g["Wv"] = Wk, Wv
    g["q"] = synth.normal((s.T, s.B, s.H, s.d), synth.seed(s.case, synth.SEED_Q, layer), "bf16")
    kv = synth.normal((2, s.T, s.B, s.H, s.d), synth.seed(s.case, synth.SEED_SELF, layer), "bf16")
    g["k_self"], g["v_self"] = kv[0], kv[1]
    if mu:
        m = synth.normal((2,) + mu_shape, synth.seed(s.case, synth.SEED_MU, layer), "bf16", std=0.5)
        g["mu_k"], g["mu_v"] = m[0], m[1]
    else:
        g["mu_k"] = g["mu_v"] = None
    return g


def _check_sampled(s, rows, loops, what, layer=0, mu=False):
    """One decode read per loop at the workload's full launch shape; the sampled rows (all heads)
    are compared with the explicit-reconstruction oracle (Eq. 3 rebuild, then softmax)."""
    g = _fill_device_case(s, layer, mu)
    desc = mk_desc(s.variant, s.dtype, s.H, s.d, s.T, s.r_k, s.r_v, s.n_max)
    lens = np.full(s.B, s.N, np.int32)
    Wk, Wv = dev(g["Wk"], "bf16"), dev(g["Wv"], "bf16")
    muk, muv = dev(g["mu_k"], "bf16"), dev(g["mu_v"], "bf16")
    ws = lla.workspace(desc, s.B, 1)
    zk_rows = host(g["zk"][rows])
    zv_rows = host(g["zv"][rows])
    for t in loops:
        q = dev(g["q"][t], "bf16")
        out = torch.empty_like(q)
        lse = torch.empty(s.B, s.H, device="cuda")
        lla.lla_attend_decode(desc, s.B, t, q, g["zk"], g["zv"], dev(lens), Wk, Wv, muk, muv,
                              dev(g["k_self"][t], "bf16"), dev(g["v_self"][t], "bf16"), out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode(g["q"][t][rows], zk_rows, zv_rows, g["Wk"], g["Wv"], t,
                                 lens[rows], g["mu_k"], g["mu_v"], g["k_self"][t][rows],
                                 g["v_self"][t][rows], variant=s.variant)
        assert_close(host(out)[rows], ro, s.dtype, f"{what} layer={layer} mu={mu} t={t}")
        slack = None
        if s.variant == "2d":
            slack = mfma_lse_slack(g["q"][t][rows], zk_rows, g["Wk"], t, lens[rows])
        assert_lse(host(lse)[rows], rl, f"{what} layer={layer} mu={mu} t={t}", slack)
    del g
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layer,mu", [(0, False), (23, True)])
def test_capacity_layer_full_size_sampled(layer, mu):
    """Capacity shape at the benchmark's launch shape (B=768, N=4096, r=24): the first layer's
    factors and inputs without the calibration mean, the last layer's with it; rows 0, 383, 767
    and five seeded ones, all heads, all loops."""
    s = synth.CASES["capacity"]
    rows = sorted({0, 383, 767, *np.random.default_rng(synth.seed(s.case, synth.SEED_SAMPLE)).choice(768, 5, replace=False).tolist()})
    _check_sampled(s, rows, range(s.T), "capacity", layer, mu)


@pytest.mark.timeout(900)
def test_deep_loop_full_size_sampled():
    """Deep-recurrence shape (H=40, d=96, T=32, r=96, B=64, N=4096): rows 0, 63 and two seeded
    ones, all heads, every one of the 32 loops."""
    s = synth.CASES["deep_loop"]
    rows = sorted({0, 63, *np.random.default_rng(synth.seed(s.case, synth.SEED_SAMPLE)).choice(64, 2, replace=False).tolist()})
    _check_sampled(s, rows, range(s.T), "deep_loop")


@pytest.mark.timeout(600)
def test_lla2d_decode_full_size_sampled():
    """LLA-2D decode (r=256+256, B=128, N=8192): rows 0 and 127, all heads, all loops."""
    s = synth.CASES["lla2d"].with_(C=1)
    _check_sampled(s, [0, 127], range(s.T), "lla2d")


@pytest.mark.parametrize("rk,rv", [(32, 32), (64, 64), (128, 128), (96, 160), (256, 256)])
def test_decode_2d_mfma(rk, rv):
    """LLA-2D bf16 decode on the MFMA path: two head groups (H=20), ragged lengths, mu, self token,
    plain and 8x sharpened queries."""
    dtype = "bf16"
    B, H, d, T, n_max = 5, 20, 64, 2, 1000
    lens = [1000, 999, 17, 0, 640]
    for gain, mu, self_token in ((1.0, True, True), (8.0, False, True), (1.0, True, False)):
        c = upload(synth.random_case("2d", dtype, B, H, d, T, rk, rv, n_max, 7600 + rk + rv,
                                     with_mu=mu, q_gain=gain), dtype)
        desc = mk_desc("2d", dtype, H, d, T, rk, rv, n_max)
        for t in range(T):
            o, lse = gpu_decode(desc, B, t, c, dtype, lens, self_token, mu)
            ro, rl = oracle_decode(c, t, lens, "2d", self_token, mu)
            what = f"2d mfma r=({rk},{rv}) gain={gain} mu={mu} self={self_token} t={t}"
            assert_close(o, ro, dtype, what)
            assert_lse(lse, rl, what)


@pytest.mark.parametrize("variant,H,d,T,r,B,C", [
    ("per_head", 16, 128, 4, 32, 8, 160),     # 1280 tokens: K split over the 4 waves
    ("per_head", 16, 128, 4, 32, 16, 512),    # 8192 tokens: whole-K waves
    ("2d", 16, 128, 4, 256, 2, 512),          # a 2D prefill chunk's encode (tiled GEMM)
    ("per_head", 16, 128, 4, 128, 3, 300),    # tiled GEMM, 128-row latent tiles, ragged tokens
    ("per_head", 8, 64, 4, 256, 2, 257),      # tiled GEMM, one token past a 256-token tile
    ("2d", 8, 64, 4, 512, 1, 700),            # tiled GEMM, two 256-row latent tiles
])
def test_encode_large_token_counts(variant, H, d, T, r, B, C):
    dtype = "bf16"
    n_max = C + 7
    # the last sequence starts 5 slots later: its last 5 tokens fall past n_max and are not written
    pos = np.array([7] * (B - 1) + [12], np.int32)
    K = T * d if variant == "per_head" else T * H * d
    es = (H, r, K) if variant == "per_head" else (r, K)
    ms = (H, K) if variant == "per_head" else (K,)
    zs = (B, H, n_max, r) if variant == "per_head" else (B, n_max, r)
    xk = synth.normal((B, C, T, H, d), 950 + r, dtype)
    xv = synth.normal((B, C, T, H, d), 951 + r, dtype)
    Ek = synth.normal(es, 952 + r, dtype, 1 / math.sqrt(K))
    Ev = synth.normal(es, 953 + r, dtype, 1 / math.sqrt(K))
    mk = synth.normal(ms, 954 + r, dtype, 0.5)
    desc = mk_desc(variant, dtype, H, d, T, r, r, n_max)
    zk = torch.zeros(zs, dtype=torch.bfloat16, device="cuda")
    zv = torch.zeros_like(zk)
    lla.lla_encode(desc, B, C, dev(xk, dtype), dev(xv, dtype), dev(Ek, dtype), dev(Ev, dtype),
                   dev(mk, dtype), None, dev(pos), zk, zv)
    torch.cuda.synchronize()
    z0 = np.zeros(zs)
    # the oracle writes only the in-range slots, like the kernel
    rk_, rv_ = z0.copy(), z0.copy()
    for b in range(B):
        keep = min(C, n_max - int(pos[b]))
        sub = slice(b, b + 1)
        rk_[sub], rv_[sub] = O.encode_into_cache(z0[sub], z0[sub], xk[sub, :keep], xv[sub, :keep], Ek, Ev,
                                                 pos[sub], mk, None, variant)
    assert_close(host(zk), rk_, dtype, f"encode zk {variant} B={B} C={C}")
    assert_close(host(zv), rv_, dtype, f"encode zv {variant} B={B} C={C}")


@pytest.mark.parametrize("variant", ["per_head", "2d"])
@pytest.mark.parametrize("rk,rv", [(64, 64), (128, 128), (256, 256), (64, 128), (128, 256)])
def test_prefill_mfma(variant, rk, rv):
    """MFMA chunked prefill: two row blocks with a ragged tail (C=150), eight sequences (the
    workgroup order that groups a sequence on one XCD) with different context lengths including
    none, mu on/off, plain and 8x sharpened queries."""
    dtype = "bf16"
    B, C, H, d, T = 8, 150, 3, 64, 2
    ctx = np.array([300, 0, 17, 299, 1, 64, 128, 250], np.int32)
    n_max = 460
    for gain, mu in ((1.0, True), (8.0, False)):
        c = upload(synth.random_case(variant, dtype, B, H, d, T, rk, rv, n_max, 7800 + rk + rv, with_mu=mu), dtype)
        q = synth.to_storage(gain * synth.normal((B, C, H, d), 7801), dtype)
        desc = mk_desc(variant, dtype, H, d, T, rk, rv, n_max)
        for t in range(T):
            out = torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda")
            lla.lla_attend_prefill(desc, B, C, t, dev(q, dtype), c["_zk"], c["_zv"], dev(ctx), c["_Wk"],
                                   c["_Wv"], c["_muk"] if mu else None, c["_muv"] if mu else None, out,
                                   lla.workspace(desc, B, C))
            torch.cuda.synchronize()
            ref = O.attend_prefill(q, c["zk"], c["zv"], c["Wk"], c["Wv"], t, ctx,
                                   c["mu_k"] if mu else None, c["mu_v"] if mu else None, variant=variant)
            assert_close(host(out), ref, dtype, f"prefill mfma {variant} r=({rk},{rv}) gain={gain} t={t}")


def test_lla2d_prefill_full_size_sampled():
    """LLA-2D chunked prefill at full size (B=128, C=512, N_ctx=8192, r=256): the chunk is encoded
    into slots 8192..8703, then loop 0 attends causally; rows {0, 255, 511} of sequence 0 (all
    heads) are checked against the oracle (a row j at position ctx + j is a one-row prefill)."""
    s = synth.CASES["lla2d"]
    B, C, H, d, T, r, N = s.B, s.C, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + C
    desc = mk_desc("2d", "bf16", H, d, T, r, r, n_max)
    g = {}
    g["zk"] = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    g["zv"] = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    Wk = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")
    Wv = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")
    Ek, Ev = synth.pinv_E_from_W_2d(Wk, "bf16"), synth.pinv_E_from_W_2d(Wv, "bf16")
    xk = synth.device_normal_(torch.empty(B, C, T, H, d, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_XK))
    xv = synth.device_normal_(torch.empty(B, C, T, H, d, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_XV))
    q = synth.device_normal_(torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    lla.lla_encode(desc, B, C, xk, xv, dev(Ek, "bf16"), dev(Ev, "bf16"), None, None, ctx, g["zk"], g["zv"])
    out = torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda")
    lla.lla_attend_prefill(desc, B, C, 0, q, g["zk"], g["zv"], ctx, dev(Wk, "bf16"), dev(Wv, "bf16"),
                           None, None, out, lla.workspace(desc, B, C))
    torch.cuda.synchronize()
    zk0, zv0 = host(g["zk"][:1]), host(g["zv"][:1])
    # the encoded chunk slots match the oracle's encode of the same per-loop K/V
    ek, _ = O.encode_into_cache(np.zeros((1, n_max, r)), np.zeros((1, n_max, r)), host(xk[:1]), host(xv[:1]),
                                Ek, Ev, [N], variant="2d")
    assert_close(zk0[:, N:], ek[:, N:], "bf16", "2d chunk encode")
    q0 = host(q[:1])
    o0 = host(out[:1])
    for j in (0, 255, 511):
        ref = O.attend_prefill(q0[:, j:j + 1], zk0, zv0, Wk, Wv, 0, [N + j], variant="2d")
        assert_close(o0[:, j:j + 1], ref, "bf16", f"2d prefill row {j}")
    del g, xk, xv, q, out
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------------------------
# randomized configurations: combinations the sweeps above do not enumerate
# --------------------------------------------------------------------------------------------

MFMA_2D_PAIRS = [(64, 64), (128, 128), (256, 256)]


def _random_configs(n, seed=7777):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = "2d" if rng.random() < 0.35 else "per_head"
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        pool = PAIRS + (MFMA_2D_PAIRS if variant == "2d" and dtype == "bf16" else [])
        rk, rv = pool[rng.integers(len(pool))]
        H = int(rng.choice([1, 3, 16, 17] if variant == "2d" else [1, 2, 5]))
        d = int(rng.choice([16, 64, 128]))
        T = int(rng.integers(1, 4))
        B = int(rng.integers(1, 6))
        n_max = int(rng.choice([1, 7, 255, 256, 257, 1000, 2500]))
        lens = [int(x) for x in rng.integers(0, n_max + 2, B)]
        out.append(dict(i=i, variant=variant, dtype=dtype, rk=int(rk), rv=int(rv), H=H, d=d, T=T,
                        B=B, n_max=n_max, lens=lens, mu=bool(rng.random() < 0.5),
                        self_token=bool(rng.random() < 0.7), gain=float(rng.choice([1.0, 8.0])),
                        t=int(rng.integers(0, T))))
    return out


@pytest.mark.parametrize("cfg", _random_configs(24), ids=lambda c: f"cfg{c['i']}")
def test_decode_random_configurations(cfg):
    """Seeded random draws over variant, storage, rank pair, heads (incl. a partial 16-head group),
    head width, loop, batch, cache size (1 .. 2500 slots), ragged and out-of-range lengths, mu, the
    self token and sharpened queries, each against the oracle. A row with no key and no self token
    is skipped (the entry point fills it but the oracle has no defined value)."""
    c = cfg
    desc = mk_desc(c["variant"], c["dtype"], c["H"], c["d"], c["T"], c["rk"], c["rv"], c["n_max"])
    case = upload(synth.random_case(c["variant"], c["dtype"], c["B"], c["H"], c["d"], c["T"], c["rk"],
                                    c["rv"], c["n_max"], 12000 + c["i"], with_mu=c["mu"],
                                    q_gain=c["gain"]), c["dtype"])
    o, lse = gpu_decode(desc, c["B"], c["t"], case, c["dtype"], c["lens"], c["self_token"], c["mu"])
    ro, rl = oracle_decode(case, c["t"], c["lens"], c["variant"], c["self_token"], c["mu"])
    live = [b for b in range(c["B"]) if c["self_token"] or min(max(c["lens"][b], 0), c["n_max"]) > 0]
    if live:
        assert_close(o[live], ro[live], c["dtype"], str(c))
        mfma = (c["variant"] == "2d" and c["dtype"] == "bf16" and (c["rk"], c["rv"]) in MFMA_2D_PAIRS
                and c["d"] <= 128)
        slack = mfma_lse_slack(case["q"][c["t"]], case["zk"], case["Wk"], c["t"], c["lens"])[live] if mfma else None
        assert_lse(lse[live], rl[live], str(c), slack)


PREFILL_MFMA_PAIRS = [(64, 64), (128, 128), (256, 256), (64, 128), (128, 256)]


def _random_prefill_configs(n, seed=8888):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = "2d" if rng.random() < 0.4 else "per_head"
        dtype = "bf16" if rng.random() < 0.8 else "f32"
        mfma = dtype == "bf16" and rng.random() < 0.6
        pool = PREFILL_MFMA_PAIRS if mfma else [p for p in PAIRS if p[0] <= 128]
        rk, rv = pool[rng.integers(len(pool))]
        d = int(rng.choice([32, 64, 128] if mfma else [16, 32, 64]))
        H = int(rng.choice([1, 2, 3]))
        B = int(rng.choice([1, 3, 8]))
        C = int(rng.choice([1, 15, 16, 17, 128, 129, 200]))
        ctx = [int(x) for x in rng.integers(0, 400, B)]
        ctx[0] = 0
        n_max = max(ctx) + C + int(rng.integers(0, 50))
        out.append(dict(i=i, variant=variant, dtype=dtype, rk=int(rk), rv=int(rv), H=H, d=d, T=2,
                        B=B, C=C, ctx=ctx, n_max=n_max, mu=bool(rng.random() < 0.5),
                        gain=float(rng.choice([1.0, 8.0])), t=int(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("cfg", _random_prefill_configs(16), ids=lambda c: f"cfg{c['i']}")
def test_prefill_random_configurations(cfg):
    """Seeded random chunked-prefill draws over variant, storage, MFMA and streaming rank pairs,
    head width, heads, batch (8 takes the XCD-grouped workgroup order), chunk length around the
    16- and 128-row block edges, context lengths (one empty), mu and sharpened queries."""
    c = cfg
    desc = mk_desc(c["variant"], c["dtype"], c["H"], c["d"], c["T"], c["rk"], c["rv"], c["n_max"])
    case = upload(synth.random_case(c["variant"], c["dtype"], c["B"], c["H"], c["d"], c["T"], c["rk"],
                                    c["rv"], c["n_max"], 13000 + c["i"], with_mu=c["mu"]), c["dtype"])
    q = synth.to_storage(c["gain"] * synth.normal((c["B"], c["C"], c["H"], c["d"]), 13500 + c["i"]), c["dtype"])
    ctx = np.array(c["ctx"], np.int32)
    out = torch.empty(c["B"], c["C"], c["H"], c["d"], dtype=dev(q, c["dtype"]).dtype, device="cuda")
    lla.lla_attend_prefill(desc, c["B"], c["C"], c["t"], dev(q, c["dtype"]), case["_zk"], case["_zv"],
                           dev(ctx), case["_Wk"], case["_Wv"], case["_muk"] if c["mu"] else None,
                           case["_muv"] if c["mu"] else None, out, lla.workspace(desc, c["B"], c["C"]))
    torch.cuda.synchronize()
    ref = O.attend_prefill(q, case["zk"], case["zv"], case["Wk"], case["Wv"], c["t"], ctx,
                           case["mu_k"] if c["mu"] else None, case["mu_v"] if c["mu"] else None,
                           variant=c["variant"])
    assert_close(host(out), ref, c["dtype"], str(c))
