"""Seeded random configurations of the entry points beyond the plain decode and prefill (which
tests/test_gpu_parity.py draws): gather-indexed decode, decode and prefill with the decoupled
rotary branch, encode, and reads over low-bit latent rows. Each draw combines shape, storage,
lengths and options that the enumerated sweeps do not, and is checked against the oracle.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import (assert_close, assert_lse, dev, host, mfma_lse_slack, rebuild_flip_lse_slack,
                            require_gpu)
from tests.test_gpu_parity import PAIRS, mk_desc, upload

pytestmark = pytest.mark.gpu

MFMA_2D_PAIRS = [(64, 64), (128, 128), (256, 256)]
PREFILL_MFMA_PAIRS = [(64, 64), (128, 128), (256, 256), (64, 128), (128, 256)]
LOW_BIT = {"e4m3": (lla.LLA_BF16_Q8, O.quantize_latent_rows),
           "int8": (lla.LLA_BF16_I8, O.quantize_latent_rows_int8)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _live(lens, n, self_token):
    """Rows with at least one key (empty rows without a self token have no defined value)."""
    return [b for b, x in enumerate(lens) if self_token or min(max(int(x), 0), n) > 0]


# --------------------------------------------------------------------------------------------
# gather-indexed decode
# --------------------------------------------------------------------------------------------

def _gather_configs(n, seed=21000):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = "2d" if rng.random() < 0.3 else "per_head"
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        rk, rv = PAIRS[rng.integers(len(PAIRS))]
        n_max = int(rng.choice([5, 300, 1200, 3000]))
        budget = int(rng.choice([1, 64, 700, 2049, 2600]))
        B = int(rng.integers(1, 5))
        counts = [int(x) for x in rng.integers(-2, budget + 3, B)]
        out.append(dict(i=i, variant=variant, dtype=dtype, rk=int(rk), rv=int(rv),
                        H=int(rng.choice([1, 2, 3])), d=int(rng.choice([16, 64])), T=2, B=B,
                        n_max=n_max, budget=budget, counts=counts if rng.random() < 0.8 else None,
                        skip=float(rng.choice([0.0, 0.1])), rep=float(rng.choice([0.0, 0.2])),
                        self_token=bool(rng.random() < 0.6), mu=bool(rng.random() < 0.5),
                        gain=float(rng.choice([1.0, 8.0]))))
    return out


@pytest.mark.parametrize("cfg", _gather_configs(12), ids=lambda c: f"cfg{c['i']}")
def test_gather_random(cfg):
    c = cfg
    desc = mk_desc(c["variant"], c["dtype"], c["H"], c["d"], c["T"], c["rk"], c["rv"], c["n_max"])
    case = upload(synth.random_case(c["variant"], c["dtype"], c["B"], c["H"], c["d"], c["T"], c["rk"],
                                    c["rv"], c["n_max"], 21100 + c["i"], with_mu=c["mu"],
                                    q_gain=c["gain"]), c["dtype"])
    slots = synth.random_slots(c["B"], c["budget"], c["n_max"], 21200 + c["i"], p_skip=c["skip"],
                               p_repeat=c["rep"])
    t = 1
    q = dev(case["q"][t], c["dtype"])
    out = torch.empty_like(q)
    lse = torch.empty(c["B"], c["H"], device="cuda")
    counts = None if c["counts"] is None else dev(np.array(c["counts"], np.int32))
    lla.lla_attend_decode_gather(desc, c["B"], t, q, case["_zk"], case["_zv"], dev(slots), counts,
                                 case["_Wk"], case["_Wv"], case["_muk"] if c["mu"] else None,
                                 case["_muv"] if c["mu"] else None,
                                 dev(case["k_self"][t], c["dtype"]) if c["self_token"] else None,
                                 dev(case["v_self"][t], c["dtype"]) if c["self_token"] else None,
                                 out, lse, lla.gather_workspace(desc, c["B"], c["budget"]))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_gather(case["q"][t], case["zk"], case["zv"], case["Wk"], case["Wv"], t,
                                    slots, c["counts"], case["mu_k"] if c["mu"] else None,
                                    case["mu_v"] if c["mu"] else None,
                                    case["k_self"][t] if c["self_token"] else None,
                                    case["v_self"][t] if c["self_token"] else None,
                                    variant=c["variant"])
    # a row is live when a self token is given or one of its listed slots is in range
    cnt = [c["budget"] if c["counts"] is None else min(max(x, 0), c["budget"]) for x in
           (c["counts"] or [c["budget"]] * c["B"])]
    live = [b for b in range(c["B"]) if c["self_token"] or
            np.any((slots[b, :cnt[b]] >= 0) & (slots[b, :cnt[b]] < c["n_max"]))]
    if live:
        assert_close(host(out)[live], ro[live], c["dtype"], str(c))
        assert_lse(host(lse)[live], rl[live], str(c))


# --------------------------------------------------------------------------------------------
# decode and prefill with the decoupled rotary branch
# --------------------------------------------------------------------------------------------

def _rope_decode_configs(n, seed=22000):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = "2d" if rng.random() < 0.5 else "per_head"
        pool = PAIRS + (MFMA_2D_PAIRS if variant == "2d" else [])
        rk, rv = pool[rng.integers(len(pool))]
        # H >= 8 takes the head-group read (8 heads share each batch's rotary rows) where it pays
        H = int(rng.choice([1, 3, 8, 17] if variant == "2d" else [1, 2, 5, 8, 20]))
        n_max = int(rng.choice([3, 257, 1500, 4400]))
        B = int(rng.integers(1, 4))
        out.append(dict(i=i, variant=variant, rk=int(rk), rv=int(rv), H=H,
                        d=int(rng.choice([32, 64, 128])), T=2, B=B, n_max=n_max,
                        lens=[int(x) for x in rng.integers(0, n_max + 2, B)],
                        d_rope=int(rng.choice([32, 64, 128])),
                        base=float(rng.choice([0.0, 500.0])),
                        self_token=bool(rng.random() < 0.6), mu=bool(rng.random() < 0.5),
                        gain=float(rng.choice([1.0, 6.0])), t=int(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("cfg", _rope_decode_configs(12), ids=lambda c: f"cfg{c['i']}")
def test_rope_decode_random(cfg):
    c = cfg
    desc = mk_desc(c["variant"], "bf16", c["H"], c["d"], c["T"], c["rk"], c["rv"], c["n_max"])
    rng = np.random.default_rng(22100 + c["i"])
    case = upload(synth.random_case(c["variant"], "bf16", c["B"], c["H"], c["d"], c["T"], c["rk"],
                                    c["rv"], c["n_max"], 22200 + c["i"], with_mu=c["mu"],
                                    q_gain=c["gain"]), "bf16")
    qr = synth.to_storage(rng.standard_normal((c["B"], c["H"], c["d_rope"])).astype(np.float32), "bf16")
    kr = synth.to_storage(rng.standard_normal((c["B"], c["n_max"], c["d_rope"])).astype(np.float32), "bf16")
    krs = synth.to_storage(rng.standard_normal((c["B"], c["d_rope"])).astype(np.float32), "bf16")
    t = c["t"]
    q = dev(case["q"][t], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(c["B"], c["H"], device="cuda")
    st = c["self_token"]
    lla.lla_attend_decode_rope(desc, c["B"], t, q, dev(qr, "bf16"), case["_zk"], case["_zv"],
                               dev(kr, "bf16"), c["d_rope"], c["base"], dev(np.array(c["lens"], np.int32)),
                               case["_Wk"], case["_Wv"], case["_muk"] if c["mu"] else None,
                               case["_muv"] if c["mu"] else None,
                               dev(case["k_self"][t], "bf16") if st else None,
                               dev(case["v_self"][t], "bf16") if st else None,
                               dev(krs, "bf16") if st else None, out, lse, lla.rope_workspace(desc, c["B"]))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(case["q"][t], qr, case["zk"], case["zv"], kr, case["Wk"], case["Wv"],
                                  t, c["lens"], case["mu_k"] if c["mu"] else None,
                                  case["mu_v"] if c["mu"] else None,
                                  case["k_self"][t] if st else None, case["v_self"][t] if st else None,
                                  krs if st else None, base=c["base"] if c["base"] > 0 else 10000.0,
                                  variant=c["variant"])
    live = _live(c["lens"], c["n_max"], st)
    if live:
        assert_close(host(out)[live], ro[live], "bf16", str(c))
        mfma = c["variant"] == "2d" and (c["rk"], c["rv"]) in MFMA_2D_PAIRS and c["d"] <= 128
        slack = mfma_lse_slack(case["q"][t], case["zk"], case["Wk"], t, c["lens"], q_rope=qr,
                               k_rope=kr)[live] if mfma else None
        assert_lse(host(lse)[live], rl[live], str(c), slack)


def _rope_prefill_configs(n, seed=23000):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = "2d" if rng.random() < 0.5 else "per_head"
        # head widths that are a multiple of 32 with an MFMA pair take the MFMA path (d_rope 64,
        # 128); every other draw the streaming path (d_rope 32, 64, 128)
        d = int(rng.choice([32, 48, 64]))
        pool = (PREFILL_MFMA_PAIRS + PAIRS) if d % 32 == 0 else PAIRS
        rk, rv = pool[rng.integers(len(pool))]
        mfma = d % 32 == 0 and (rk, rv) in PREFILL_MFMA_PAIRS
        B = int(rng.choice([1, 2, 8]))
        C = int(rng.choice([1, 16, 33, 128, 150]))
        ctx = [int(x) for x in rng.integers(0, 300, B)]
        ctx[-1] = 0
        out.append(dict(i=i, variant=variant, rk=int(rk), rv=int(rv), H=int(rng.choice([1, 2, 3])),
                        d=d, T=2, B=B, C=C, ctx=ctx,
                        n_max=max(ctx) + C + int(rng.integers(0, 20)),
                        d_rope=int(rng.choice([64, 128] if mfma else [32, 64, 128])), mu=bool(rng.random() < 0.5),
                        gain=float(rng.choice([1.0, 6.0])), t=int(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("cfg", _rope_prefill_configs(10), ids=lambda c: f"cfg{c['i']}")
def test_rope_prefill_random(cfg):
    c = cfg
    desc = mk_desc(c["variant"], "bf16", c["H"], c["d"], c["T"], c["rk"], c["rv"], c["n_max"])
    rng = np.random.default_rng(23100 + c["i"])
    case = upload(synth.random_case(c["variant"], "bf16", c["B"], c["H"], c["d"], c["T"], c["rk"],
                                    c["rv"], c["n_max"], 23200 + c["i"], with_mu=c["mu"]), "bf16")
    q = synth.to_storage(c["gain"] * rng.standard_normal((c["B"], c["C"], c["H"], c["d"])).astype(np.float32), "bf16")
    qr = synth.to_storage(rng.standard_normal((c["B"], c["C"], c["H"], c["d_rope"])).astype(np.float32), "bf16")
    kr = synth.to_storage(rng.standard_normal((c["B"], c["n_max"], c["d_rope"])).astype(np.float32), "bf16")
    ctx = np.array(c["ctx"], np.int32)
    out = torch.empty(c["B"], c["C"], c["H"], c["d"], dtype=torch.bfloat16, device="cuda")
    lla.lla_attend_prefill_rope(desc, c["B"], c["C"], c["t"], dev(q, "bf16"), dev(qr, "bf16"),
                                case["_zk"], case["_zv"], dev(kr, "bf16"), c["d_rope"], 0.0, dev(ctx),
                                case["_Wk"], case["_Wv"], case["_muk"] if c["mu"] else None,
                                case["_muv"] if c["mu"] else None, out,
                                lla.workspace(desc, c["B"], c["C"]))
    torch.cuda.synchronize()
    ref = O.attend_prefill_rope(q, qr, case["zk"], case["zv"], kr, case["Wk"], case["Wv"], c["t"], ctx,
                                case["mu_k"] if c["mu"] else None, case["mu_v"] if c["mu"] else None,
                                variant=c["variant"])
    assert_close(host(out), ref, "bf16", str(c))


# --------------------------------------------------------------------------------------------
# encode
# --------------------------------------------------------------------------------------------

def _encode_configs(n, seed=24000):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = "2d" if rng.random() < 0.4 else "per_head"
        B = int(rng.integers(1, 5))
        C = int(rng.choice([1, 3, 64, 300]))
        n_max = C + int(rng.integers(0, 40))
        r = int(rng.choice([8, 24, 96, 128, 256]))
        # unequal ranks in some draws: the two axes then take separate launches instead of one
        rv = r if rng.random() < 0.7 else int(rng.choice([16, 32, 160]))
        out.append(dict(i=i, variant=variant, dtype="bf16" if rng.random() < 0.75 else "f32",
                        H=int(rng.choice([1, 2, 3])), d=int(rng.choice([16, 64, 128])),
                        T=int(rng.choice([1, 2, 4])), r=r, rv=rv,
                        B=B, C=C, n_max=n_max,
                        pos=[int(x) for x in rng.integers(-3, n_max + 3, B)],
                        mu_k=bool(rng.random() < 0.5), mu_v=bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("cfg", _encode_configs(16), ids=lambda c: f"cfg{c['i']}")
def test_encode_random(cfg):
    """Random encode shapes, including write positions before the cache and past its end (rows
    whose slot falls outside [0, n_max) are not written; untouched slots keep their contents)."""
    c = cfg
    dtype, variant, H, d, T, r, rv, B, C, n_max = (c[k] for k in ("dtype", "variant", "H", "d", "T", "r",
                                                               "rv", "B", "C", "n_max"))
    base = 24100 + 10 * c["i"]
    K = T * d if variant == "per_head" else T * H * d
    ms = (H, K) if variant == "per_head" else (K,)

    def zshape(rank):
        return (B, H, n_max, rank) if variant == "per_head" else (B, n_max, rank)

    def eshape(rank):
        return (H, rank, K) if variant == "per_head" else (rank, K)

    xk = synth.normal((B, C, T, H, d), base + 1, dtype)
    xv = synth.normal((B, C, T, H, d), base + 2, dtype)
    Ek = synth.normal(eshape(r), base + 3, dtype, 1 / math.sqrt(K))
    Ev = synth.normal(eshape(rv), base + 4, dtype, 1 / math.sqrt(K))
    mk = synth.normal(ms, base + 5, dtype, 0.5) if c["mu_k"] else None
    mv = synth.normal(ms, base + 6, dtype, 0.5) if c["mu_v"] else None
    zk0 = synth.normal(zshape(r), base + 7, dtype)
    zv0 = synth.normal(zshape(rv), base + 8, dtype)
    pos = np.array(c["pos"], np.int32)
    desc = mk_desc(variant, dtype, H, d, T, r, rv, n_max)
    zk, zv = dev(zk0, dtype), dev(zv0, dtype)
    lla.lla_encode(desc, B, C, dev(xk, dtype), dev(xv, dtype), dev(Ek, dtype), dev(Ev, dtype),
                   None if mk is None else dev(mk, dtype), None if mv is None else dev(mv, dtype), dev(pos),
                   zk, zv)
    torch.cuda.synchronize()
    want_k, want_v = zk0.astype(np.float64).copy(), zv0.astype(np.float64).copy()
    written = np.zeros(zshape(r)[:-1], bool)
    for b in range(B):
        c0, c1 = max(0, -int(pos[b])), min(C, n_max - int(pos[b]))  # chunk rows whose slot is in range
        if c0 >= c1:
            continue
        sub = slice(b, b + 1)
        ak, av = O.encode_into_cache(zk0[sub], zv0[sub], xk[sub, c0:c1], xv[sub, c0:c1], Ek, Ev,
                                     np.array([pos[b] + c0]), mk, mv, variant)
        want_k[sub], want_v[sub] = ak, av
        slots = slice(int(pos[b]) + c0, int(pos[b]) + c1)
        if variant == "per_head":
            written[b, :, slots] = True
        else:
            written[b, slots] = True
    gk, gv = host(zk), host(zv)
    if written.any():
        assert_close(gk[written], want_k[written], dtype, f"encode zk {c}")
        assert_close(gv[written], want_v[written], dtype, f"encode zv {c}")
    assert np.array_equal(gk[~written], zk0.astype(np.float64)[~written])
    assert np.array_equal(gv[~written], zv0.astype(np.float64)[~written])


# --------------------------------------------------------------------------------------------
# low-bit latent rows
# --------------------------------------------------------------------------------------------

def _low_bit_configs(n, seed=25000):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        n_max = int(rng.choice([2, 300, 2100]))
        variant = "2d" if rng.random() < 0.4 else "per_head"
        # the streaming ranks (r = 96: two loads per lane), and on LLA-2D the MFMA read's ranks
        ranks = [8, 16, 24, 32, 96] + ([64, 128, 256] if variant == "2d" else [])
        out.append(dict(i=i, fmt=str(rng.choice(sorted(LOW_BIT))), variant=variant,
                        r=int(rng.choice(ranks)), H=int(rng.choice([1, 2, 3, 17] if variant == "2d" else [1, 2, 3])),
                        d=int(rng.choice([16, 64])), T=2, B=B, n_max=n_max,
                        lens=[int(x) for x in rng.integers(0, n_max + 2, B)],
                        self_token=bool(rng.random() < 0.6), mu=bool(rng.random() < 0.5),
                        gain=float(rng.choice([1.0, 8.0])), t=int(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("cfg", _low_bit_configs(12), ids=lambda c: f"cfg{c['i']}")
def test_low_bit_decode_random(cfg):
    c = cfg
    dt, quant = LOW_BIT[c["fmt"]]
    variant, r, B, H, n_max = c["variant"], c["r"], c["B"], c["H"], c["n_max"]
    case = synth.random_case(variant, "bf16", B, H, c["d"], c["T"], r, r, n_max, 25100 + c["i"],
                             with_mu=c["mu"], q_gain=c["gain"])
    desc = lla.make_desc(lla.LLA_PER_HEAD if variant == "per_head" else lla.LLA_2D, dt, H, c["d"],
                         c["T"], r, r, n_max)
    rb = lla.lla_latent_row_bytes(dt, r)
    cshape = (B, H, n_max, rb) if variant == "per_head" else (B, n_max, rb)
    ck = torch.empty(cshape, dtype=torch.uint8, device="cuda")
    cv = torch.empty_like(ck)
    lla.lla_quantize_latents(desc, B, n_max, dev(case["zk"], "bf16"), dev(case["zv"], "bf16"),
                             dev(np.zeros(B, np.int32)), ck, cv)
    zk_dq = O.dequantize_latent_rows(*quant(case["zk"]))
    zv_dq = O.dequantize_latent_rows(*quant(case["zv"]))
    t, st = c["t"], c["self_token"]
    q = dev(case["q"][t], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode(desc, B, t, q, ck, cv, dev(np.array(c["lens"], np.int32)),
                          dev(case["Wk"], "bf16"), dev(case["Wv"], "bf16"),
                          dev(case["mu_k"], "bf16") if c["mu"] else None,
                          dev(case["mu_v"], "bf16") if c["mu"] else None,
                          dev(case["k_self"][t], "bf16") if st else None,
                          dev(case["v_self"][t], "bf16") if st else None, out, lse, lla.workspace(desc, B))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode(case["q"][t], zk_dq, zv_dq, case["Wk"], case["Wv"], t, c["lens"],
                             case["mu_k"] if c["mu"] else None, case["mu_v"] if c["mu"] else None,
                             case["k_self"][t] if st else None, case["v_self"][t] if st else None,
                             variant=variant)
    live = _live(c["lens"], n_max, st)
    if live:
        assert_close(host(out)[live], ro[live], "bf16", str(c))
        mfma = variant == "2d" and (r, r) in MFMA_2D_PAIRS and c["d"] <= 128
        slack = mfma_lse_slack(case["q"][t], zk_dq, case["Wk"], t, c["lens"])[live] if mfma else None
        assert_lse(host(lse)[live], rl[live], str(c), slack)


# --------------------------------------------------------------------------------------------
# reconstruct-then-attend comparator
# --------------------------------------------------------------------------------------------

def _reconstruct_configs(n, seed=26000):
    rng = np.random.default_rng(seed)
    ranks = [32 * k for k in range(1, 9)]  # every compiled rank of the rebuild kernel
    out = []
    for i in range(n):
        n_max = int(rng.choice([1, 100, 129, 700]))
        B = int(rng.integers(1, 5))
        out.append(dict(i=i, d=int(rng.choice([64, 128])), rk=int(rng.choice(ranks)),
                        rv=int(rng.choice(ranks)), H=int(rng.choice([1, 2, 3])), T=int(rng.integers(1, 3)),
                        B=B, n_max=n_max, lens=[int(x) for x in rng.integers(0, n_max + 2, B)],
                        mu=bool(rng.random() < 0.5), self_token=bool(rng.random() < 0.6),
                        gain=float(rng.choice([1.0, 8.0]))))
    return out


@pytest.mark.parametrize("cfg", _reconstruct_configs(16), ids=lambda c: f"cfg{c['i']}")
def test_reconstruct_random(cfg):
    """Seeded draws over head width, both ranks (32 .. 256, so every rebuild tile shape), heads,
    batch, cache size, ragged and out-of-range lengths, mu, the self token and sharpened queries:
    the comparator against the oracle's explicit decode with the rebuilt K/V rounded to bf16."""
    c = cfg
    desc = mk_desc("per_head", "bf16", c["H"], c["d"], c["T"], c["rk"], c["rv"], c["n_max"])
    case = upload(synth.random_case("per_head", "bf16", c["B"], c["H"], c["d"], c["T"], c["rk"], c["rv"],
                                    c["n_max"], 26100 + c["i"], with_mu=c["mu"], q_gain=c["gain"]), "bf16")
    t = c["T"] - 1
    st = c["self_token"]
    q = dev(case["q"][t], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(c["B"], c["H"], device="cuda")
    lla.lla_attend_decode_reconstruct(desc, c["B"], t, q, case["_zk"], case["_zv"],
                                      dev(np.array(c["lens"], np.int32)), case["_Wk"], case["_Wv"],
                                      case["_muk"] if c["mu"] else None, case["_muv"] if c["mu"] else None,
                                      dev(case["k_self"][t], "bf16") if st else None,
                                      dev(case["v_self"][t], "bf16") if st else None, out, lse,
                                      lla.reconstruct_workspace(desc, c["B"]))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode(case["q"][t], case["zk"], case["zv"], case["Wk"], case["Wv"], t, c["lens"],
                             case["mu_k"] if c["mu"] else None, case["mu_v"] if c["mu"] else None,
                             case["k_self"][t] if st else None, case["v_self"][t] if st else None,
                             kv_round_bf16=True)
    live = _live(c["lens"], c["n_max"], st)
    if live:
        assert_close(host(out)[live], ro[live], "bf16", str(c))
        slack = rebuild_flip_lse_slack(case["q"][t], case["zk"], case["Wk"], t, c["lens"],
                                       case["mu_k"] if c["mu"] else None)[live]
        assert_lse(host(lse)[live], rl[live], str(c), slack)
