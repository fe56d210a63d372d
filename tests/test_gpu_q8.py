"""GPU parity of low-bit latent rows (LLA_BF16_Q8: E4M3 codes; LLA_BF16_I8: int8 codes) against
the oracle.

The quantiser must be bit-exact: the codes and the float32 scale of every row equal the oracle's
quantize_latent_rows / quantize_latent_rows_int8 of the same bf16 rows (both sides divide in
float32 and round to nearest even). The reads (decode, gather decode, prefill on the streaming
kernels) are compared with the oracle's attention over the dequantised rows, to the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import assert_close, assert_lse, dev, host, mfma_lse_slack, require_gpu
from tests.test_gpu_parity import _fill_device_case, mk_desc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# low-bit format -> (descriptor dtype, oracle quantiser, code bytes -> values)
FORMATS = {
    "e4m3": (lla.LLA_BF16_Q8, O.quantize_latent_rows,
             lambda b: torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()),
    "int8": (lla.LLA_BF16_I8, O.quantize_latent_rows_int8,
             lambda b: b.view(np.int8).astype(np.float64)),
}


def q8_desc(variant, H, d, T, rk, rv, n_max, fmt="e4m3"):
    return lla.make_desc(lla.LLA_PER_HEAD if variant == "per_head" else lla.LLA_2D,
                         FORMATS[fmt][0], H, d, T, rk, rv, n_max)


def unpack_rows(raw, r, fmt="e4m3"):
    """uint8 rows [..., row_bytes] -> (code values [..., r] float64, scales [...] float64, padding)."""
    raw = np.ascontiguousarray(raw)
    codes = FORMATS[fmt][2](raw[..., :r].copy())
    scales = raw[..., -4:].copy().view(np.float32)[..., 0].astype(np.float64)
    return codes, scales, raw[..., r:-4]


def cache_rows(shape_src, n_max, rng, variant):
    """Seeded bf16 latent rows with per-row magnitudes from 1e-3 to 1e3 and one zero row."""
    z = rng.standard_normal(shape_src) * 10.0 ** rng.uniform(-3, 3, shape_src[:-1] + (1,))
    z = synth.to_storage(z.astype(np.float32), "bf16")
    z.reshape(-1, shape_src[-1])[1] = 0.0
    return z


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("variant", ["per_head", "2d"])
@pytest.mark.parametrize("r", [8, 13, 24, 32, 96, 256])
def test_quantize_bit_exact(variant, r, fmt):
    rng = np.random.default_rng(9400 + r)
    B, H, C, n_max = 3, 2, 5, 9
    desc = q8_desc(variant, H, 16, 2, r, r, n_max, fmt)
    src = (B, H, C, r) if variant == "per_head" else (B, C, r)
    zk = cache_rows(src, n_max, rng, variant)
    zv = cache_rows(src, n_max, rng, variant)
    rb = lla.lla_latent_row_bytes(lla.LLA_BF16_Q8, r)
    cshape = (B, H, n_max, rb) if variant == "per_head" else (B, n_max, rb)
    ck = torch.full(cshape, 0xAB, dtype=torch.uint8, device="cuda")
    cv = torch.full(cshape, 0xAB, dtype=torch.uint8, device="cuda")
    pos = np.array([0, 4, 7], np.int32)  # sequence 2: slots 7, 8 written, 9.. skipped
    lla.lla_quantize_latents(desc, B, C, dev(zk, "bf16"), dev(zv, "bf16"), dev(pos), ck, cv)
    torch.cuda.synchronize()
    for z, cache in ((zk, ck), (zv, cv)):
        raw = cache.cpu().numpy()
        want_codes, want_s = FORMATS[fmt][1](z)
        for b in range(B):
            for c in range(C):
                slot = pos[b] + c
                sel_src = (b, slice(None), c) if variant == "per_head" else (b, c)
                if slot >= n_max:
                    continue
                sel = (b, slice(None), slot) if variant == "per_head" else (b, slot)
                codes, s, pad = unpack_rows(raw[sel], r, fmt)
                np.testing.assert_array_equal(codes, want_codes[sel_src])
                np.testing.assert_array_equal(s, want_s[sel_src])
                assert np.all(pad == 0)
        # slots that no row maps to keep their bytes
        written = np.zeros((B, n_max), bool)
        for b in range(B):
            for c in range(C):
                if pos[b] + c < n_max:
                    written[b, pos[b] + c] = True
        for b in range(B):
            for slot in range(n_max):
                if not written[b, slot]:
                    sel = (b, slice(None), slot) if variant == "per_head" else (b, slot)
                    assert np.all(raw[sel] == 0xAB)


def _q8_case(variant, B, H, d, T, r, n_max, sd, gain=1.0, fmt="e4m3"):
    """bf16 case, its low-bit cache built on the device, and the oracle's dequantised rows."""
    c = synth.random_case(variant, "bf16", B, H, d, T, r, r, n_max, sd, q_gain=gain)
    desc = q8_desc(variant, H, d, T, r, r, n_max, fmt)
    rb = lla.lla_latent_row_bytes(lla.LLA_BF16_Q8, r)
    cshape = (B, H, n_max, rb) if variant == "per_head" else (B, n_max, rb)
    ck = torch.empty(cshape, dtype=torch.uint8, device="cuda")
    cv = torch.empty(cshape, dtype=torch.uint8, device="cuda")
    # the cache holds n_max slots: quantise them as one chunk per sequence at slot 0
    lla.lla_quantize_latents(desc, B, n_max, dev(c["zk"], "bf16"), dev(c["zv"], "bf16"),
                             dev(np.zeros(B, np.int32)), ck, cv)
    c["_ck"], c["_cv"] = ck, cv
    c["zk_dq"] = O.dequantize_latent_rows(*FORMATS[fmt][1](c["zk"]))
    c["zv_dq"] = O.dequantize_latent_rows(*FORMATS[fmt][1](c["zv"]))
    for k in ("Wk", "Wv", "mu_k", "mu_v"):
        c["_" + k] = dev(c[k], "bf16")
    return c, desc


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("variant,r", [("per_head", 8), ("per_head", 16), ("per_head", 24),
                                       ("per_head", 32), ("2d", 24), ("2d", 32), ("per_head", 96),
                                       ("2d", 96)])
def test_decode_q8(variant, r, fmt):
    B, H, d, T, n_max = 3, 2, 64, 2, 3001
    lens = np.array([3001, 517, 0], np.int32)
    for gain, mu, self_token in ((1.0, True, True), (8.0, False, True), (1.0, True, False)):
        c, desc = _q8_case(variant, B, H, d, T, r, n_max, 9500 + r, gain, fmt)
        assert lla.lla_workspace_bytes(desc, B) > 0  # 8-wave workgroups, split-K and the combine
        for t in range(T):
            q = dev(c["q"][t], "bf16")
            out = torch.empty_like(q)
            lse = torch.empty(B, H, device="cuda")
            lla.lla_attend_decode(desc, B, t, q, c["_ck"], c["_cv"], dev(lens), c["_Wk"], c["_Wv"],
                                  c["_mu_k"] if mu else None, c["_mu_v"] if mu else None,
                                  dev(c["k_self"][t], "bf16") if self_token else None,
                                  dev(c["v_self"][t], "bf16") if self_token else None, out, lse,
                                  lla.workspace(desc, B))
            torch.cuda.synchronize()
            ro, rl = O.attend_decode(c["q"][t], c["zk_dq"], c["zv_dq"], c["Wk"], c["Wv"], t, lens,
                                     c["mu_k"] if mu else None, c["mu_v"] if mu else None,
                                     c["k_self"][t] if self_token else None,
                                     c["v_self"][t] if self_token else None, variant=variant)
            what = f"{fmt} {variant} r={r} gain={gain} mu={mu} self={self_token} t={t}"
            assert_close(host(out), ro, "bf16", what)
            assert_lse(host(lse), rl, what)


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("r", [8, 16, 24, 32, 96])
def test_gather_and_prefill_q8(fmt, r):
    B, H, d, T, n_max = 2, 2, 64, 2, 700
    c, desc = _q8_case("per_head", B, H, d, T, r, n_max, 9600 + r, fmt=fmt)
    slots = synth.random_slots(B, 400, n_max, 9601, p_skip=0.05, p_repeat=0.05)
    counts = np.array([400, 211], np.int32)
    q = dev(c["q"][1], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode_gather(desc, B, 1, q, c["_ck"], c["_cv"], dev(slots), dev(counts),
                                 c["_Wk"], c["_Wv"], c["_mu_k"], c["_mu_v"], None, None, out, lse,
                                 lla.gather_workspace(desc, B, 400))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_gather(c["q"][1], c["zk_dq"], c["zv_dq"], c["Wk"], c["Wv"], 1, slots,
                                    counts, c["mu_k"], c["mu_v"])
    assert_close(host(out), ro, "bf16", f"{fmt} r={r} gather")
    assert_lse(host(lse), rl, f"{fmt} r={r} gather")
    # chunked prefill on the streaming path: 37 rows per sequence after contexts 600 and 0
    C = 37
    ctx = np.array([600, 0], np.int32)
    rng = np.random.default_rng(9602)
    qp = synth.to_storage(rng.standard_normal((B, C, H, d)).astype(np.float32), "bf16")
    outp = torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda")
    lla.lla_attend_prefill(desc, B, C, 0, dev(qp, "bf16"), c["_ck"], c["_cv"], dev(ctx), c["_Wk"],
                           c["_Wv"], c["_mu_k"], c["_mu_v"], outp, lla.workspace(desc, B, C))
    torch.cuda.synchronize()
    rp = O.attend_prefill(qp, c["zk_dq"], c["zv_dq"], c["Wk"], c["Wv"], 0, ctx, c["mu_k"], c["mu_v"])
    assert_close(host(outp), rp, "bf16", f"{fmt} r={r} prefill")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_capacity_q8_full_size_sampled(fmt):
    """Capacity shape (B=768, H=16, d=128, T=4, r=24, N=4096) with low-bit rows quantised on the
    device from the bf16 cache, at the benchmark's launch shape; sampled rows, all loops."""
    s = synth.CASES["capacity"]
    g = _fill_device_case(s)
    desc = q8_desc("per_head", s.H, s.d, s.T, s.r_k, s.r_v, s.n_max, fmt)
    rb = lla.lla_latent_row_bytes(lla.LLA_BF16_Q8, s.r_k)
    ck = torch.empty(s.B, s.H, s.n_max, rb, dtype=torch.uint8, device="cuda")
    cv = torch.empty_like(ck)
    lla.lla_quantize_latents(desc, s.B, s.n_max, g["zk"], g["zv"],
                             torch.zeros(s.B, dtype=torch.int32, device="cuda"), ck, cv)
    rows = sorted({0, 383, 767, *np.random.default_rng(synth.seed(s.case, synth.SEED_SAMPLE)).choice(768, 3, replace=False).tolist()})
    zk_dq = O.dequantize_latent_rows(*FORMATS[fmt][1](host(g["zk"][rows]).astype(np.float32)))
    zv_dq = O.dequantize_latent_rows(*FORMATS[fmt][1](host(g["zv"][rows]).astype(np.float32)))
    del g["zk"], g["zv"]
    torch.cuda.empty_cache()
    lens = np.full(s.B, s.N, np.int32)
    Wk, Wv = dev(g["Wk"], "bf16"), dev(g["Wv"], "bf16")
    ws = lla.workspace(desc, s.B, 1)
    for t in range(s.T):
        q = dev(g["q"][t], "bf16")
        out = torch.empty_like(q)
        lse = torch.empty(s.B, s.H, device="cuda")
        lla.lla_attend_decode(desc, s.B, t, q, ck, cv, dev(lens), Wk, Wv, None, None,
                              dev(g["k_self"][t], "bf16"), dev(g["v_self"][t], "bf16"), out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode_absorbed(g["q"][t][rows], zk_dq, zv_dq, g["Wk"], g["Wv"], t,
                                          lens[rows], None, None, g["k_self"][t][rows],
                                          g["v_self"][t][rows])
        assert_close(host(out)[rows], ro, "bf16", f"capacity {fmt} t={t}")
        assert_lse(host(lse)[rows], rl, f"capacity {fmt} t={t}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_deep_loop_q8_full_size_sampled(fmt):
    """Deep-recurrence shape (B=64, H=40, d=96, T=32, r=96, N=4096) with 112-byte low-bit rows
    (4 lanes x 28 bytes per row, two loads per lane) quantised on the device, at the benchmark's
    launch shape; sampled rows (all heads), loops 0, 17 and 31, against the explicit oracle on the
    dequantised rows."""
    s = synth.CASES["deep_loop"]
    g = _fill_device_case(s)
    desc = q8_desc("per_head", s.H, s.d, s.T, s.r_k, s.r_v, s.n_max, fmt)
    rb = lla.lla_latent_row_bytes(lla.LLA_BF16_Q8, s.r_k)
    assert rb == 112
    ck = torch.empty(s.B, s.H, s.n_max, rb, dtype=torch.uint8, device="cuda")
    cv = torch.empty_like(ck)
    lla.lla_quantize_latents(desc, s.B, s.n_max, g["zk"], g["zv"],
                             torch.zeros(s.B, dtype=torch.int32, device="cuda"), ck, cv)
    rows = sorted({0, 63, *np.random.default_rng(synth.seed(s.case, synth.SEED_SAMPLE)).choice(64, 2, replace=False).tolist()})
    zk_dq = O.dequantize_latent_rows(*FORMATS[fmt][1](host(g["zk"][rows]).astype(np.float32)))
    zv_dq = O.dequantize_latent_rows(*FORMATS[fmt][1](host(g["zv"][rows]).astype(np.float32)))
    del g["zk"], g["zv"]
    torch.cuda.empty_cache()
    lens = np.full(s.B, s.N, np.int32)
    Wk, Wv = dev(g["Wk"], "bf16"), dev(g["Wv"], "bf16")
    ws = lla.workspace(desc, s.B, 1)
    for t in (0, 17, 31):
        q = dev(g["q"][t], "bf16")
        out = torch.empty_like(q)
        lse = torch.empty(s.B, s.H, device="cuda")
        print(f"deep loop {fmt} t={t}", flush=True)
        lla.lla_attend_decode(desc, s.B, t, q, ck, cv, dev(lens), Wk, Wv, None, None,
                              dev(g["k_self"][t], "bf16"), dev(g["v_self"][t], "bf16"), out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode(g["q"][t][rows], zk_dq, zv_dq, g["Wk"], g["Wv"], t, lens[rows],
                                 None, None, g["k_self"][t][rows], g["v_self"][t][rows])
        assert_close(host(out)[rows], ro, "bf16", f"deep loop {fmt} t={t}")
        assert_lse(host(lse)[rows], rl, f"deep loop {fmt} t={t}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("r", [64, 128, 256])
def test_decode_q8_lla2d_mfma(r, fmt):
    """LLA-2D decode over low-bit rows on the MFMA read (codes converted to bf16, the K scale on each
    score, the V scale on each weight): 20 heads (two 16-head groups, the second ragged), split-K,
    ragged and empty sequences, sharpened queries, mu and the self token; lse within the MFMA
    read's q~-rounding slack on the dequantised rows."""
    B, H, d, T, n_max = 3, 20, 64, 2, 1500
    lens = np.array([1500, 517, 0], np.int32)
    for gain, mu, self_token in ((1.0, True, True), (8.0, False, True)):
        c, desc = _q8_case("2d", B, H, d, T, r, n_max, 9700 + r, gain, fmt)
        assert lla.lla_workspace_bytes(desc, B) > 0
        for t in range(T):
            q = dev(c["q"][t], "bf16")
            out = torch.full_like(q, float("nan"))
            lse = torch.full((B, H), float("nan"), device="cuda")
            print(f"2d mfma {fmt} r={r} gain={gain} t={t}", flush=True)
            lla.lla_attend_decode(desc, B, t, q, c["_ck"], c["_cv"], dev(lens), c["_Wk"], c["_Wv"],
                                  c["_mu_k"] if mu else None, c["_mu_v"] if mu else None,
                                  dev(c["k_self"][t], "bf16") if self_token else None,
                                  dev(c["v_self"][t], "bf16") if self_token else None, out, lse,
                                  lla.workspace(desc, B))
            torch.cuda.synchronize()
            ro, rl = O.attend_decode(c["q"][t], c["zk_dq"], c["zv_dq"], c["Wk"], c["Wv"], t, lens,
                                     c["mu_k"] if mu else None, c["mu_v"] if mu else None,
                                     c["k_self"][t] if self_token else None,
                                     c["v_self"][t] if self_token else None, variant="2d")
            what = f"2d mfma {fmt} r={r} gain={gain} mu={mu} t={t}"
            assert_close(host(out), ro, "bf16", what)
            assert_lse(host(lse), rl, what, mfma_lse_slack(c["q"][t], c["zk_dq"], c["Wk"], t, lens))


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_lla2d_q8_full_size_sampled(fmt):
    """The LLA-2D decode benchmark shape (B=128, H=16, d=128, T=4, r=256/256, N=8192) with low-bit
    rows quantised on the device, at the benchmark's launch shape; sequences 0 and 127 (all heads),
    loop 1, against the explicit oracle on the dequantised rows."""
    s = synth.CASES["lla2d"]
    g = _fill_device_case(s)
    desc = q8_desc("2d", s.H, s.d, s.T, s.r_k, s.r_v, s.n_max, fmt)
    rb = lla.lla_latent_row_bytes(lla.LLA_BF16_Q8, s.r_k)
    ck = torch.empty(s.B, s.n_max, rb, dtype=torch.uint8, device="cuda")
    cv = torch.empty_like(ck)
    lla.lla_quantize_latents(desc, s.B, s.n_max, g["zk"], g["zv"],
                             torch.zeros(s.B, dtype=torch.int32, device="cuda"), ck, cv)
    rows = [0, 127]
    zk_dq = O.dequantize_latent_rows(*FORMATS[fmt][1](host(g["zk"][rows]).astype(np.float32)))
    zv_dq = O.dequantize_latent_rows(*FORMATS[fmt][1](host(g["zv"][rows]).astype(np.float32)))
    del g["zk"], g["zv"]
    torch.cuda.empty_cache()
    lens = np.full(s.B, s.N, np.int32)
    Wk, Wv = dev(g["Wk"], "bf16"), dev(g["Wv"], "bf16")
    ws = lla.workspace(desc, s.B, 1)
    t = 1
    q = dev(g["q"][t], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(s.B, s.H, device="cuda")
    print(f"lla2d full size {fmt}", flush=True)
    lla.lla_attend_decode(desc, s.B, t, q, ck, cv, dev(lens), Wk, Wv, None, None,
                          dev(g["k_self"][t], "bf16"), dev(g["v_self"][t], "bf16"), out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = O.attend_decode(g["q"][t][rows], zk_dq, zv_dq, g["Wk"], g["Wv"], t, lens[rows],
                             None, None, g["k_self"][t][rows], g["v_self"][t][rows], variant="2d")
    assert_close(host(out)[rows], ro, "bf16", f"lla2d {fmt}")
    assert_lse(host(lse)[rows], rl, f"lla2d {fmt}",
               mfma_lse_slack(g["q"][t][rows], zk_dq, g["Wk"], t, lens[rows]))
