"""GPU parity of the decoupled rotary branch (lla_rope_write, lla_attend_decode_rope).

The rotary key write is compared with the oracle's RoFormer rotation rounded to bf16; the decode
with the rotary branch is compared with the oracle's explicit attention over concatenated
(content, rotary) keys, element by element, for both variants, three rotary widths, split-K, the
self token, long positions, and the capacity shape at full size on sampled rows.
"""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import assert_close, assert_lse, dev, host, mfma_lse_slack, require_gpu
from tests.test_gpu_parity import _fill_device_case, mk_desc, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d_rope,base", [(64, 0.0), (32, 500.0), (128, 10000.0)])
def test_rope_write(d_rope, base):
    rng = np.random.default_rng(9900 + d_rope)
    B, C, n_max = 3, 6, 262150
    desc = mk_desc("per_head", "bf16", 2, 64, 2, 24, 24, n_max)
    k_in = synth.to_storage(rng.standard_normal((B, C, d_rope)).astype(np.float32), "bf16")
    pos = np.array([0, 1000, 262146], np.int32)  # sequence 2: slots 262146..262149 written, then skipped
    kr = torch.full((B, n_max, d_rope), 7.0, dtype=torch.bfloat16, device="cuda")
    lla.lla_rope_write(desc, B, C, d_rope, base, dev(k_in, "bf16"), dev(pos), kr)
    torch.cuda.synchronize()
    b_eff = base if base > 0 else 10000.0
    for b in range(B):
        for c in range(C):
            slot = int(pos[b]) + c
            if slot >= n_max:
                continue
            want = O.round_bf16_via_f32(O.rope_rotate(k_in[b, c], slot, b_eff))
            got = host(kr[b, slot])
            # float64 trigonometry on both sides: equal up to a last-place difference in sin/cos,
            # which can move a bf16 rounding by one step
            ulp = np.maximum(np.abs(want), 1e-30) * 2.0 ** -7
            assert np.all(np.abs(got - want) <= ulp), (b, c)
            assert np.mean(got == want) >= 0.95, (b, c)
    untouched = host(kr[0, 6:1000])
    assert np.all(untouched == 7.0)


def _rope_inputs(rng, B, H, n_max, d_rope):
    q_rope = synth.to_storage(rng.standard_normal((B, H, d_rope)).astype(np.float32), "bf16")
    k_rope = synth.to_storage(rng.standard_normal((B, n_max, d_rope)).astype(np.float32), "bf16")
    krs = synth.to_storage(rng.standard_normal((B, d_rope)).astype(np.float32), "bf16")
    return q_rope, k_rope, krs


@pytest.mark.parametrize("variant,rk,rv,d_rope", [("per_head", 24, 24, 64), ("per_head", 96, 160, 32),
                                                  ("per_head", 128, 128, 128), ("2d", 32, 32, 64),
                                                  ("2d", 256, 256, 64), ("2d", 128, 128, 32),
                                                  ("2d", 64, 64, 128), ("per_head", 16, 16, 64),
                                                  ("per_head", 8, 8, 32)])
def test_decode_rope(variant, rk, rv, d_rope):
    B, H, d, T, n_max = 3, 2, 64, 2, 1301
    lens = np.array([1301, 517, 0], np.int32)
    desc = mk_desc(variant, "bf16", H, d, T, rk, rv, n_max)
    ws = lla.rope_workspace(desc, B)
    rng = np.random.default_rng(9950 + rk + d_rope)
    q_rope, k_rope, krs = _rope_inputs(rng, B, H, n_max, d_rope)
    d_qr, d_kr, d_krs = dev(q_rope, "bf16"), dev(k_rope, "bf16"), dev(krs, "bf16")
    for gain, mu, self_token in ((1.0, True, True), (8.0, False, True), (1.0, True, False)):
        c = upload(synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, 9960 + rk,
                                     with_mu=mu, q_gain=gain), "bf16")
        for t in range(T):
            q = dev(c["q"][t], "bf16")
            out = torch.empty_like(q)
            lse = torch.empty(B, H, device="cuda")
            lla.lla_attend_decode_rope(desc, B, t, q, d_qr, c["_zk"], c["_zv"], d_kr, d_rope, 0.0,
                                       dev(lens), c["_Wk"], c["_Wv"], c["_muk"] if mu else None,
                                       c["_muv"] if mu else None,
                                       dev(c["k_self"][t], "bf16") if self_token else None,
                                       dev(c["v_self"][t], "bf16") if self_token else None,
                                       d_krs if self_token else None, out, lse, ws)
            torch.cuda.synchronize()
            ro, rl = O.attend_decode_rope(c["q"][t], q_rope, c["zk"], c["zv"], k_rope, c["Wk"],
                                          c["Wv"], t, lens, c["mu_k"] if mu else None,
                                          c["mu_v"] if mu else None,
                                          c["k_self"][t] if self_token else None,
                                          c["v_self"][t] if self_token else None,
                                          krs if self_token else None, variant=variant)
            what = f"rope {variant} r=({rk},{rv}) d_rope={d_rope} gain={gain} mu={mu} self={self_token} t={t}"
            assert_close(host(out), ro, "bf16", what)
            assert_lse(host(lse), rl, what)


def test_lla2d_decode_rope_many_heads():
    """LLA-2D on MFMA with many heads and a wide branch (H = 144, d_rope = 128; nine 16-head
    groups), ragged lengths, self token, mu."""
    B, H, d, T, n_max, r, d_rope = 3, 144, 32, 2, 700, 64, 128
    lens = np.array([700, 333, 1], np.int32)
    desc = mk_desc("2d", "bf16", H, d, T, r, r, n_max)
    ws = lla.rope_workspace(desc, B)
    rng = np.random.default_rng(9990)
    q_rope, k_rope, krs = _rope_inputs(rng, B, H, n_max, d_rope)
    c = upload(synth.random_case("2d", "bf16", B, H, d, T, r, r, n_max, 9991), "bf16")
    t = 1
    q = dev(c["q"][t], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode_rope(desc, B, t, q, dev(q_rope, "bf16"), c["_zk"], c["_zv"],
                               dev(k_rope, "bf16"), d_rope, 0.0, dev(lens), c["_Wk"], c["_Wv"],
                               c["_muk"], c["_muv"], dev(c["k_self"][t], "bf16"),
                               dev(c["v_self"][t], "bf16"), dev(krs, "bf16"), out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(c["q"][t], q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], t,
                                  lens, c["mu_k"], c["mu_v"], c["k_self"][t], c["v_self"][t], krs,
                                  variant="2d")
    assert_close(host(out), ro, "bf16", "2d rope H=144")
    slack = mfma_lse_slack(c["q"][t], c["zk"], c["Wk"], t, lens, q_rope=q_rope, k_rope=k_rope)
    assert_lse(host(lse), rl, "2d rope H=144", slack)


@pytest.mark.parametrize("variant,rk,rv,d_rope,H", [("per_head", 24, 24, 128, 130), ("2d", 32, 32, 64, 40),
                                                      ("per_head", 96, 160, 64, 9)])
def test_decode_rope_xcd_grouped(variant, rk, rv, d_rope, H):
    """B a multiple of 8: every head (and split) of a sequence is launched onto one XCD, where they
    share the sequence's rotary keys (LLA-2D on the streaming read: its latents too). Many heads
    with a wide branch (H * d_rope = 16640), ragged lengths around the per-wave token parts,
    sharpened queries, self token."""
    B, d, T, n_max = 16, 32, 2, 2600
    lens = np.array([2600, 2599, 1, 0, 1300, 257, 1024, 1025, 31, 2048, 640, 641, 2000, 7, 99, 1555],
                    np.int32)
    desc = mk_desc(variant, "bf16", H, d, T, rk, rv, n_max)
    ws = lla.rope_workspace(desc, B)
    rng = np.random.default_rng(9970 + H)
    q_rope, k_rope, krs = _rope_inputs(rng, B, H, n_max, d_rope)
    c = upload(synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, 9971 + H, q_gain=4.0), "bf16")
    t = 1
    q = dev(c["q"][t], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode_rope(desc, B, t, q, dev(q_rope, "bf16"), c["_zk"], c["_zv"], dev(k_rope, "bf16"),
                               d_rope, 0.0, dev(lens), c["_Wk"], c["_Wv"], c["_muk"], c["_muv"],
                               dev(c["k_self"][t], "bf16"), dev(c["v_self"][t], "bf16"), dev(krs, "bf16"),
                               out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(c["q"][t], q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], t, lens,
                                  c["mu_k"], c["mu_v"], c["k_self"][t], c["v_self"][t], krs, variant=variant)
    what = f"rope xcd-grouped {variant} r=({rk},{rv}) d_rope={d_rope} H={H}"
    assert_close(host(out), ro, "bf16", what)
    assert_lse(host(lse), rl, what)


@pytest.mark.parametrize("variant,rk,rv,d_rope,H,lens", [
    ("per_head", 96, 160, 128, 8, [3001, 0]),                # one group, token splits, partial shares
    ("per_head", 24, 24, 64, 20, [2000, 777, 1]),            # 3 groups, 4 placeholder waves
    ("2d", 32, 32, 32, 8, [1500, 100]),                      # LLA-2D on the streaming read
    ("per_head", 8, 8, 128, 16, [1000, 999, 1, 0, 513, 512, 64, 65]),  # B = 8: XCD-grouped
])
def test_decode_rope_head_groups(variant, rk, rv, d_rope, H, lens):
    """The rotary read with workgroups of 8 heads of one sequence sharing each batch's rotary rows
    through LDS: with token splits, with placeholder waves past H, for both variants and the three
    rotary widths, ragged lengths, sharpened queries, self token and mu."""
    B, d, T = len(lens), 32, 2
    n_max = max(lens)
    lens = np.array(lens, np.int32)
    desc = mk_desc(variant, "bf16", H, d, T, rk, rv, n_max)
    ws = lla.rope_workspace(desc, B)
    rng = np.random.default_rng(9960 + H + d_rope)
    q_rope, k_rope, krs = _rope_inputs(rng, B, H, n_max, d_rope)
    c = upload(synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, 9961 + H + rk, q_gain=4.0), "bf16")
    t = 1
    q = dev(c["q"][t], "bf16")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H), float("nan"), device="cuda")
    print(f"head groups {variant} r=({rk},{rv}) d_rope={d_rope} H={H} B={B}", flush=True)
    lla.lla_attend_decode_rope(desc, B, t, q, dev(q_rope, "bf16"), c["_zk"], c["_zv"], dev(k_rope, "bf16"),
                               d_rope, 0.0, dev(lens), c["_Wk"], c["_Wv"], c["_muk"], c["_muv"],
                               dev(c["k_self"][t], "bf16"), dev(c["v_self"][t], "bf16"), dev(krs, "bf16"),
                               out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(c["q"][t], q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], t, lens,
                                  c["mu_k"], c["mu_v"], c["k_self"][t], c["v_self"][t], krs, variant=variant)
    what = f"rope head groups {variant} r=({rk},{rv}) d_rope={d_rope} H={H}"
    assert_close(host(out), ro, "bf16", what)
    assert_lse(host(lse), rl, what)


def test_decode_rope_many_units_ragged():
    """4096 (row, head) units over 5000 cached tokens, one split per row, with ragged lengths
    around multiples of 1024 and of the kernel's batch."""
    B, H, d, T, n_max, r, d_rope = 64, 64, 16, 1, 5000, 8, 32
    desc = mk_desc("per_head", "bf16", H, d, T, r, r, n_max)
    rng = np.random.default_rng(9975)
    q_rope, k_rope, krs = _rope_inputs(rng, B, H, n_max, d_rope)
    c = upload(synth.random_case("per_head", "bf16", B, H, d, T, r, r, n_max, 9976, q_gain=4.0), "bf16")
    lens = np.full(B, n_max, np.int32)
    lens[::7] = [4096, 4097, 1, 0, 4999, 2048, 1023, 1025, 17, 4095][: len(lens[::7])]
    q = dev(c["q"][0], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode_rope(desc, B, 0, q, dev(q_rope, "bf16"), c["_zk"], c["_zv"],
                               dev(k_rope, "bf16"), d_rope, 0.0, dev(lens), c["_Wk"], c["_Wv"],
                               c["_muk"], c["_muv"], dev(c["k_self"][0], "bf16"),
                               dev(c["v_self"][0], "bf16"), dev(krs, "bf16"), out, lse,
                               lla.rope_workspace(desc, B))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(c["q"][0], q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], 0,
                                  lens, c["mu_k"], c["mu_v"], c["k_self"][0], c["v_self"][0], krs)
    assert_close(host(out), ro, "bf16", "rope long split")
    assert_lse(host(lse), rl, "rope long split")


def test_decode_rope_very_long_context():
    """One sequence, 2 heads, 1.2M cached tokens: 254 splits of 4736 tokens."""
    B, H, d, T, r, d_rope, N = 1, 2, 16, 1, 8, 32, 1200000
    n_max = N + 3
    desc = mk_desc("per_head", "bf16", H, d, T, r, r, n_max)
    rng = np.random.default_rng(9977)
    q_rope, k_rope, krs = _rope_inputs(rng, B, H, n_max, d_rope)
    c = upload(synth.random_case("per_head", "bf16", B, H, d, T, r, r, n_max, 9978, q_gain=4.0), "bf16")
    lens = np.array([N], np.int32)
    q = dev(c["q"][0], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode_rope(desc, B, 0, q, dev(q_rope, "bf16"), c["_zk"], c["_zv"],
                               dev(k_rope, "bf16"), d_rope, 0.0, dev(lens), c["_Wk"], c["_Wv"],
                               None, None, None, None, None, out, lse, lla.rope_workspace(desc, B))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(c["q"][0], q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], 0,
                                  lens)
    assert_close(host(out), ro, "bf16", "rope 1.2M")
    assert_lse(host(lse), rl, "rope 1.2M")


def test_decode_rope_long_positions_and_explicit_scale():
    """One sequence at 70000 cached tokens (large rotation angles for the query) and a scale given
    by the descriptor."""
    B, H, d, T, n_max, r, d_rope = 1, 2, 64, 1, 70001, 24, 64
    desc = mk_desc("per_head", "bf16", H, d, T, r, r, n_max, scale=0.07)
    rng = np.random.default_rng(9970)
    q_rope, k_rope, krs = _rope_inputs(rng, B, H, n_max, d_rope)
    c = upload(synth.random_case("per_head", "bf16", B, H, d, T, r, r, n_max, 9971), "bf16")
    lens = np.array([70000], np.int32)
    q = dev(c["q"][0], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode_rope(desc, B, 0, q, dev(q_rope, "bf16"), c["_zk"], c["_zv"],
                               dev(k_rope, "bf16"), d_rope, 0.0, dev(lens), c["_Wk"], c["_Wv"], None,
                               None, None, None, None, out, lse, lla.rope_workspace(desc, B))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(c["q"][0], q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], 0,
                                  lens, scale=0.07)
    assert_close(host(out), ro, "bf16", "rope 70k")
    assert_lse(host(lse), rl, "rope 70k")


def test_capacity_rope_full_size_sampled():
    """Capacity shape (B=768, H=16, d=128, T=4, r=24, N=4096) with a 64-wide rotary branch, at the
    benchmark's launch shape; sampled rows, all loops."""
    s = synth.CASES["capacity"]
    d_rope = 64
    g = _fill_device_case(s)
    desc = mk_desc(s.variant, s.dtype, s.H, s.d, s.T, s.r_k, s.r_v, s.n_max)
    kr = synth.device_normal_(torch.empty(s.B, s.n_max, d_rope, dtype=torch.bfloat16, device="cuda"), 9980)
    qr = synth.device_normal_(torch.empty(s.T, s.B, s.H, d_rope, dtype=torch.bfloat16, device="cuda"), 9981)
    krs = synth.device_normal_(torch.empty(s.B, d_rope, dtype=torch.bfloat16, device="cuda"), 9982)
    rows = sorted({0, 383, 767, *np.random.default_rng(synth.seed(s.case, synth.SEED_SAMPLE)).choice(768, 3, replace=False).tolist()})
    zk_rows, zv_rows = host(g["zk"][rows]), host(g["zv"][rows])
    kr_rows, krs_rows = host(kr[rows]), host(krs[rows])
    lens = np.full(s.B, s.N, np.int32)
    Wk, Wv = dev(g["Wk"], "bf16"), dev(g["Wv"], "bf16")
    ws = lla.rope_workspace(desc, s.B)
    for t in range(s.T):
        q = dev(g["q"][t], "bf16")
        out = torch.empty_like(q)
        lse = torch.empty(s.B, s.H, device="cuda")
        lla.lla_attend_decode_rope(desc, s.B, t, q, qr[t], g["zk"], g["zv"], kr, d_rope, 0.0,
                                   dev(lens), Wk, Wv, None, None, dev(g["k_self"][t], "bf16"),
                                   dev(g["v_self"][t], "bf16"), krs, out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode_rope(g["q"][t][rows], host(qr[t][rows]), zk_rows, zv_rows, kr_rows,
                                      g["Wk"], g["Wv"], t, lens[rows], None, None,
                                      g["k_self"][t][rows], g["v_self"][t][rows], krs_rows)
        assert_close(host(out)[rows], ro, s.dtype, f"capacity rope t={t}")
        assert_lse(host(lse)[rows], rl, f"capacity rope t={t}")
    del g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant,rk,rv,d_rope", [("per_head", 128, 128, 64), ("2d", 256, 256, 64),
                                                  ("2d", 256, 256, 128), ("per_head", 64, 128, 128),
                                                  ("2d", 128, 256, 64)])
def test_prefill_rope(variant, rk, rv, d_rope):
    """Chunked prefill with the rotary branch on the MFMA path: 150 rows (two row blocks, ragged),
    three contexts (one empty), mu on, against the oracle."""
    B, C, H, d, T, n_max = 3, 150, 2, 64, 2, 1200
    desc = mk_desc(variant, "bf16", H, d, T, rk, rv, n_max)
    rng = np.random.default_rng(9990 + rk + d_rope)
    c = upload(synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, 9991 + rk), "bf16")
    q = synth.to_storage(rng.standard_normal((B, C, H, d)).astype(np.float32), "bf16")
    q_rope = synth.to_storage(rng.standard_normal((B, C, H, d_rope)).astype(np.float32), "bf16")
    k_rope = synth.to_storage(rng.standard_normal((B, n_max, d_rope)).astype(np.float32), "bf16")
    ctx = np.array([300, 0, 1000], np.int32)
    out = torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        lla.lla_attend_prefill_rope(desc, B, C, t, dev(q, "bf16"), dev(q_rope, "bf16"), c["_zk"],
                                    c["_zv"], dev(k_rope, "bf16"), d_rope, 0.0, dev(ctx), c["_Wk"],
                                    c["_Wv"], c["_muk"], c["_muv"], out, lla.workspace(desc, B, C))
        torch.cuda.synchronize()
        ref = O.attend_prefill_rope(q, q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], t, ctx,
                                    c["mu_k"], c["mu_v"], variant=variant)
        assert_close(host(out), ref, "bf16", f"prefill rope {variant} ({rk},{rv}) d_rope={d_rope} t={t}")


@pytest.mark.parametrize("variant,rk,rv,d_rope,d", [("per_head", 24, 24, 64, 64), ("per_head", 96, 160, 32, 64),
                                                    ("2d", 32, 32, 128, 64), ("per_head", 8, 8, 32, 64),
                                                    ("per_head", 64, 64, 64, 48), ("2d", 256, 256, 32, 48)])
def test_prefill_rope_streaming(variant, rk, rv, d_rope, d):
    """Chunked prefill with the rotary branch on the streaming path (pairs and head widths without
    the MFMA prefill): each chunk row is a query at position ctx + j over latents 0 .. ctx + j,
    70 rows, three contexts (one empty), mu on, sharpened queries, against the oracle."""
    B, C, H, T, n_max = 3, 70, 2, 2, 1200
    desc = mk_desc(variant, "bf16", H, d, T, rk, rv, n_max)
    rng = np.random.default_rng(9890 + rk + d_rope + d)
    c = upload(synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, 9891 + rk + d), "bf16")
    q = synth.to_storage(4.0 * rng.standard_normal((B, C, H, d)).astype(np.float32), "bf16")
    q_rope = synth.to_storage(2.0 * rng.standard_normal((B, C, H, d_rope)).astype(np.float32), "bf16")
    k_rope = synth.to_storage(rng.standard_normal((B, n_max, d_rope)).astype(np.float32), "bf16")
    ctx = np.array([300, 0, 1000], np.int32)
    out = torch.full((B, C, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"streaming prefill rope {variant} ({rk},{rv}) d_rope={d_rope} d={d}", flush=True)
    for t in range(T):
        lla.lla_attend_prefill_rope(desc, B, C, t, dev(q, "bf16"), dev(q_rope, "bf16"), c["_zk"],
                                    c["_zv"], dev(k_rope, "bf16"), d_rope, 0.0, dev(ctx), c["_Wk"],
                                    c["_Wv"], c["_muk"], c["_muv"], out, lla.workspace(desc, B, C))
        torch.cuda.synchronize()
        ref = O.attend_prefill_rope(q, q_rope, c["zk"], c["zv"], k_rope, c["Wk"], c["Wv"], t, ctx,
                                    c["mu_k"], c["mu_v"], variant=variant)
        what = f"streaming prefill rope {variant} ({rk},{rv}) d_rope={d_rope} d={d} t={t}"
        assert_close(host(out), ref, "bf16", what)
        # row by row as well: a position or mask slip on one row must not hide under the global max
        o = host(out).astype(np.float64)
        for b in range(B):
            for j in range(C):
                assert_close(o[b, j], ref[b, j], "bf16", f"{what} row ({b}, {j})")


def test_lla2d_decode_rope_full_size_sampled():
    """The LLA-2D decode benchmark shape (B=128, H=16, d=128, T=4, r=256, N=8192) on the MFMA
    path with a 64-wide rotary branch and the self token; sequences {0, 77, 127}, all heads, all
    loops."""
    s = synth.CASES["lla2d"]
    B, H, d, T, r, N = s.B, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + 1
    d_rope = 64
    desc = mk_desc("2d", "bf16", H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), 10010)
    zv = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), 10011)
    kr = synth.device_normal_(torch.empty(B, n_max, d_rope, dtype=torch.bfloat16, device="cuda"), 10012)
    krs = synth.device_normal_(torch.empty(B, d_rope, dtype=torch.bfloat16, device="cuda"), 10013)
    Wk = synth.orthonormal_W_2d(T, H, d, r, 10014, "bf16")
    Wv = synth.orthonormal_W_2d(T, H, d, r, 10015, "bf16")
    q = synth.device_normal_(torch.empty(T, B, H, d, dtype=torch.bfloat16, device="cuda"), 10016)
    qr = synth.device_normal_(torch.empty(T, B, H, d_rope, dtype=torch.bfloat16, device="cuda"), 10017)
    ks = synth.device_normal_(torch.empty(T, B, H, d, dtype=torch.bfloat16, device="cuda"), 10018)
    vs = synth.device_normal_(torch.empty(T, B, H, d, dtype=torch.bfloat16, device="cuda"), 10019)
    lens = np.full(B, N, np.int32)
    rows = [0, 77, 127]
    zk0, zv0, kr0, krs0 = host(zk[rows]), host(zv[rows]), host(kr[rows]), host(krs[rows])
    ws = lla.rope_workspace(desc, B)
    dWk, dWv = dev(Wk, "bf16"), dev(Wv, "bf16")
    for t in range(T):
        out = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, H, device="cuda")
        lla.lla_attend_decode_rope(desc, B, t, q[t], qr[t], zk, zv, kr, d_rope, 0.0, dev(lens), dWk,
                                   dWv, None, None, ks[t], vs[t], krs, out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode_rope(host(q[t][rows]), host(qr[t][rows]), zk0, zv0, kr0, Wk, Wv, t,
                                      lens[rows], None, None, host(ks[t][rows]), host(vs[t][rows]),
                                      krs0, variant="2d")
        assert_close(host(out)[rows], ro, "bf16", f"2d decode rope t={t}")
        assert_lse(host(lse)[rows], rl, f"2d decode rope t={t}")
    del zk, zv, kr, out
    torch.cuda.empty_cache()


def test_lla2d_prefill_rope_full_size_sampled():
    """The LLA-2D 512-token prefill benchmark shape (B=128, C=512, N_ctx=8192, r=256) with a
    64-wide rotary branch; rows {0, 255, 511} of sequence 0, all heads."""
    s = synth.CASES["lla2d"]
    B, C, H, d, T, r, N = s.B, s.C, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + C
    d_rope = 64
    desc = mk_desc("2d", "bf16", H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), 9995)
    zv = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), 9996)
    kr = synth.device_normal_(torch.empty(B, n_max, d_rope, dtype=torch.bfloat16, device="cuda"), 9997)
    Wk = synth.orthonormal_W_2d(T, H, d, r, 9998, "bf16")
    Wv = synth.orthonormal_W_2d(T, H, d, r, 9999, "bf16")
    q = synth.device_normal_(torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda"), 10000)
    qr = synth.device_normal_(torch.empty(B, C, H, d_rope, dtype=torch.bfloat16, device="cuda"), 10001)
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    out = torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda")
    lla.lla_attend_prefill_rope(desc, B, C, 1, q, qr, zk, zv, kr, d_rope, 0.0, ctx, dev(Wk, "bf16"),
                                dev(Wv, "bf16"), None, None, out, lla.workspace(desc, B, C))
    torch.cuda.synchronize()
    zk0, zv0, kr0 = host(zk[:1]), host(zv[:1]), host(kr[:1])
    q0, qr0, o0 = host(q[:1]), host(qr[:1]), host(out[:1])
    for j in (0, 255, 511):
        ref = O.attend_prefill_rope(q0[:, j:j + 1], qr0[:, j:j + 1], zk0, zv0, kr0, Wk, Wv, 1,
                                    [N + j], variant="2d")
        assert_close(o0[:, j:j + 1], ref, "bf16", f"2d prefill rope row {j}")
    del zk, zv, kr, q, qr, out
    torch.cuda.empty_cache()
