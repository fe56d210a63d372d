"""GPU parity at the edges of the key range, where a one-key slip would otherwise hide.

With nearly uniform softmax weights over N keys, dropping or adding one key moves o by about 1/N of
its size, under the bf16 tolerance once N passes ~100. These tests plant latents so that the key at
an edge carries almost all of a row's weight and the first key past the row's end would carry more
still: a key dropped at the edge, or one taken past the end, then moves that row's o by about its
own size. Edges covered: the last visible key, token-split and tile boundaries of the decode read,
and the causal limit of every prefill row block (32-key tiles, 16- and 128-row blocks).

The planted inputs are built on the host from the bf16 inputs (a latent along the row's absorbed
query, sized for a chosen score); the expected outputs come from the explicit-reconstruction oracle
on exactly those inputs. Every check is made per row (max|gpu - oracle| <= 1e-2 * max|oracle| over
the row's d outputs) as well as over the whole call, and decode rows also check the log-sum-exp,
which sees a key counted twice.
"""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import (LLA_DT, LLA_VAR, TOL, assert_close, assert_lse, dev, host,
                            mfma_lse_slack, require_gpu)

pytestmark = pytest.mark.gpu

MARGIN = 12.0   # planted key's score above the row's other visible keys (weight ratio e^-12)
PAST = 24.0     # the key just past the row's end scores this far above them


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _w_head(W, t, h, d, variant):
    """W_t restricted to head h: [d][r] (LLA-2D: rows h*d .. (h+1)*d of the loop-t block)."""
    return W[t, h] if variant == "per_head" else W[t, h * d:(h + 1) * d]


def _plant(qt, score, scale):
    """A bf16 latent whose score scale * (q~ . z) against the absorbed query q~ is about `score`."""
    qt = np.asarray(qt, np.float64)
    return synth.round_bf16((score / scale) * qt / float(qt @ qt))


def _row_check(got, ref, what):
    """Per-row relative error over the last axis."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=-1)
    err = np.max(np.abs(got - ref), axis=-1) / np.where(den > 0, den, 1.0)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err[worst] <= TOL["bf16"], f"{what}: row {worst} relative error {err[worst]:.3e}"


# --------------------------------------------------------------------------------------------
# decode: the last visible key, split and tile edges, and the first key past the end
# --------------------------------------------------------------------------------------------

# Token ranges of the reads start at multiples of 32 (streaming read: splits of a multiple of 128
# tokens cut into up to 4 per-wave parts, tiles of 8 to 64 rows; LLA-2D MFMA read: splits of a
# multiple of 64 tokens, 16-token tiles), so lengths and marked keys sit at and beside every
# multiple of 32 up to the cache size.
N_MAX_DEC = 1100
DEC_LENS = sorted({1, 2, 15, 16, 17, N_MAX_DEC - 1, N_MAX_DEC} |
                  {32 * k + e for k in range(1, 35) for e in (0, 1)})
DEC_EDGES = sorted({0, 1, 15, 16} | {32 * k + e for k in range(1, 35) for e in (-1, 0)})


def _decode_case(variant, rk, rv, H, seed):
    d, T, t, n_max = 64, 2, 1, N_MAX_DEC
    B = len(DEC_LENS)
    c = synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, seed, with_mu=False,
                          with_self=False)
    scale = 1.0 / np.sqrt(d)
    zk, zv = c["zk"], c["zv"]
    g = np.random.default_rng(seed + 1)
    marks = {}
    turn = 0
    for b, n in enumerate(DEC_LENS):
        heads = range(H) if variant == "per_head" else [b % H]
        for h in heads:
            qt = _w_head(c["Wk"], t, h, d, variant).astype(np.float64).T @ c["q"][t][b, h].astype(np.float64)
            # the marked key: the row's last visible key (head 0 of a per-head row, even rows of
            # LLA-2D), else the next edge inside the row in turn
            inner = [e for e in DEC_EDGES if e < n - 1]
            last = (h == 0) if variant == "per_head" else (b % 2 == 0)
            if last or not inner:
                m = n - 1
            else:
                m = inner[turn % len(inner)]
                turn += 1
            kz = zk[b, h] if variant == "per_head" else zk[b]
            vz = zv[b, h] if variant == "per_head" else zv[b]
            others = np.delete(np.arange(n), m)
            bg = float(np.max(scale * (kz[others].astype(np.float64) @ qt))) if others.size else 0.0
            kz[m] = _plant(qt, bg + MARGIN, scale)
            vz[m] = synth.round_bf16(3.0 * g.standard_normal(vz.shape[-1]))
            if n < n_max:
                kz[n] = _plant(qt, bg + PAST, scale)
                vz[n] = synth.round_bf16(3.0 * g.standard_normal(vz.shape[-1]))
            marks[(b, h)] = m
    return c, dict(B=B, H=H, d=d, T=T, t=t, n_max=n_max, marks=marks)


@pytest.mark.parametrize("variant,rk,rv,H", [
    ("per_head", 8, 8, 4), ("per_head", 24, 24, 4), ("per_head", 32, 32, 4), ("per_head", 96, 96, 4),
    ("per_head", 96, 160, 4), ("per_head", 256, 256, 4),
    ("2d", 32, 32, 3),                                           # LLA-2D on the streaming read
    ("2d", 64, 64, 20), ("2d", 128, 128, 16), ("2d", 256, 256, 16),  # LLA-2D on MFMA
])
def test_decode_edge_key_dominant(variant, rk, rv, H):
    c, k = _decode_case(variant, rk, rv, H, 21000 + rk + rv + H)
    B, t = k["B"], k["t"]
    desc = lla.make_desc(LLA_VAR[variant], LLA_DT["bf16"], H, k["d"], k["T"], rk, rv, k["n_max"])
    q = dev(c["q"][t], "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    lens = np.array(DEC_LENS, np.int32)
    lla.lla_attend_decode(desc, B, t, q, dev(c["zk"], "bf16"), dev(c["zv"], "bf16"), dev(lens),
                          dev(c["Wk"], "bf16"), dev(c["Wv"], "bf16"), None, None, None, None, out,
                          lse, lla.workspace(desc, B))
    torch.cuda.synchronize()
    ro, rl = O.attend_decode(c["q"][t], c["zk"], c["zv"], c["Wk"], c["Wv"], t, lens, variant=variant)
    what = f"edge decode {variant} r=({rk},{rv})"
    o = host(out)
    assert_close(o, ro, "bf16", what)
    _row_check(o, ro, what)
    # the planted rows really are dominated by their marked key (the construction holds)
    for (b, h), m in k["marks"].items():
        kz = c["zk"][b, h] if variant == "per_head" else c["zk"][b]
        qt = _w_head(c["Wk"], t, h, k["d"], variant).astype(np.float64).T @ c["q"][t][b, h].astype(np.float64)
        s = kz[:DEC_LENS[b]].astype(np.float64) @ qt / np.sqrt(k["d"])
        assert int(np.argmax(s)) == m
    mfma = variant == "2d" and (rk, rv) in ((64, 64), (128, 128), (256, 256))
    slack = mfma_lse_slack(c["q"][t], c["zk"], c["Wk"], t, lens) if mfma else None
    assert_lse(host(lse), rl, what, slack)


# --------------------------------------------------------------------------------------------
# prefill: the causal limit of each row
# --------------------------------------------------------------------------------------------

# marked rows per head, at least two apart (the key past one marked row must not be another's own)
PRE_ROWS = [[0, 16, 32, 64, 128, 256, 298], [1, 15, 31, 63, 127, 129, 255], [2, 30, 95, 126, 200, 297]]


def _prefill_case(variant, rk, rv, seed, B, C, H, d, ctx, n_max):
    T, t = 2, 1
    c = synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, seed, with_mu=False,
                          with_self=False)
    q = synth.normal((B, C, H, d), seed + 2, "bf16")
    scale = 1.0 / np.sqrt(d)
    zk, zv = c["zk"], c["zv"]
    g = np.random.default_rng(seed + 1)
    marked = []
    for b in range(B):
        if variant == "per_head":
            plan = [(h, j) for h in range(H) for j in PRE_ROWS[h % len(PRE_ROWS)] if j < C]
        else:  # one latent per token for all heads: the marked rows of the sequence, spaced apart
            rows = sorted({j for hs in PRE_ROWS for j in hs if j < C})
            keep = []
            for j in rows:
                if not keep or j >= keep[-1] + 2:
                    keep.append(j)
            plan = [(i % H, j) for i, j in enumerate(keep)]
        for h, j in sorted(plan, key=lambda p: p[1]):
            pos = int(ctx[b]) + j
            qt = _w_head(c["Wk"], t, h, d, variant).astype(np.float64).T @ q[b, j, h].astype(np.float64)
            kz = zk[b, h] if variant == "per_head" else zk[b]
            vz = zv[b, h] if variant == "per_head" else zv[b]
            bg = float(np.max(scale * (kz[:pos].astype(np.float64) @ qt))) if pos else 0.0
            kz[pos] = _plant(qt, bg + MARGIN, scale)
            vz[pos] = synth.round_bf16(3.0 * g.standard_normal(vz.shape[-1]))
            if pos + 1 < n_max:
                kz[pos + 1] = _plant(qt, bg + PAST, scale)
                vz[pos + 1] = synth.round_bf16(3.0 * g.standard_normal(vz.shape[-1]))
            marked.append((b, j, h))
    return c, q, t, marked


@pytest.mark.parametrize("variant,rk,rv", [
    ("per_head", 64, 64), ("per_head", 128, 128), ("per_head", 256, 256), ("per_head", 64, 128),
    ("per_head", 128, 256), ("2d", 64, 64), ("2d", 128, 128), ("2d", 256, 256), ("2d", 64, 128),
    ("2d", 128, 256),                               # the MFMA prefill
    ("per_head", 24, 24), ("2d", 32, 32),           # streaming prefill
])
def test_prefill_edge_key_dominant(variant, rk, rv):
    """Rows at 32-key tile offsets, 16- and 128-row block edges and the chunk's last rows, with
    contexts 0, 31, 97 and 250 so the same rows meet the causal limit at different tile offsets."""
    B, C, H, d = 4, 300, 3, 64
    ctx = np.array([0, 31, 97, 250], np.int32)
    n_max = int(ctx.max()) + C + 2
    c, q, t, marked = _prefill_case(variant, rk, rv, 22000 + rk + rv, B, C, H, d, ctx, n_max)
    desc = lla.make_desc(LLA_VAR[variant], LLA_DT["bf16"], H, d, 2, rk, rv, n_max)
    out = torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda")
    lla.lla_attend_prefill(desc, B, C, t, dev(q, "bf16"), dev(c["zk"], "bf16"), dev(c["zv"], "bf16"),
                           dev(ctx), dev(c["Wk"], "bf16"), dev(c["Wv"], "bf16"), None, None, out,
                           lla.workspace(desc, B, C))
    torch.cuda.synchronize()
    ref = O.attend_prefill(q, c["zk"], c["zv"], c["Wk"], c["Wv"], t, ctx, variant=variant)
    o = host(out)
    what = f"edge prefill {variant} r=({rk},{rv})"
    assert_close(o, ref, "bf16", what)
    _row_check(o, ref, what)
    # each marked row's own key dominates and the next key would dominate it further
    scale = 1.0 / np.sqrt(d)
    for b, j, h in marked:
        pos = int(ctx[b]) + j
        kz = c["zk"][b, h] if variant == "per_head" else c["zk"][b]
        qt = _w_head(c["Wk"], t, h, d, variant).astype(np.float64).T @ q[b, j, h].astype(np.float64)
        s = scale * (kz[:pos + 2].astype(np.float64) @ qt)
        assert int(np.argmax(s[:pos + 1])) == pos and (pos + 1 >= n_max or s[pos + 1] > s[pos] + 6)


@pytest.mark.timeout(600)
def test_lla2d_prefill_full_size_edge_rows():
    """The LLA-2D 512-token prefill chunk at full size (B=128, N_ctx=8192, r=256): after the
    chunk's encode, rows 0, 255 and 510 of sequence 0 get a dominant own key (slots 8192, 8447,
    8702, planted along one head's absorbed query) and a larger key one slot past; rows 0, 255, 510
    and 511 (all heads) are checked against the oracle row by row."""
    s = synth.CASES["lla2d"]
    B, C, H, d, T, r, N = s.B, s.C, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + C
    desc = lla.make_desc(lla.LLA_2D, lla.LLA_BF16, H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    zv = synth.device_normal_(torch.empty(B, n_max, r, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    Wk = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")
    Wv = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")
    Ek, Ev = synth.pinv_E_from_W_2d(Wk, "bf16"), synth.pinv_E_from_W_2d(Wv, "bf16")
    xk = synth.device_normal_(torch.empty(B, C, T, H, d, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_XK))
    xv = synth.device_normal_(torch.empty(B, C, T, H, d, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_XV))
    q = synth.device_normal_(torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    lla.lla_encode(desc, B, C, xk, xv, dev(Ek, "bf16"), dev(Ev, "bf16"), None, None, ctx, zk, zv)
    torch.cuda.synchronize()
    t = 1
    zk0, zv0 = host(zk[0]), host(zv[0])
    q0 = host(q[0])
    scale = 1.0 / np.sqrt(d)
    g = np.random.default_rng(23001)
    for i, j in enumerate((0, 255, 510)):
        h = (5 * i) % H
        pos = N + j
        qt = Wk[t, h * d:(h + 1) * d].astype(np.float64).T @ q0[j, h]
        bg = float(np.max(scale * (zk0[:pos] @ qt)))
        zk0[pos] = _plant(qt, bg + MARGIN, scale)
        zk0[pos + 1] = _plant(qt, bg + PAST, scale)
        zv0[pos] = synth.round_bf16(3.0 * g.standard_normal(r))
        zv0[pos + 1] = synth.round_bf16(3.0 * g.standard_normal(r))
    zk[0].copy_(torch.from_numpy(zk0.astype(np.float32)).to(torch.bfloat16))
    zv[0].copy_(torch.from_numpy(zv0.astype(np.float32)).to(torch.bfloat16))
    out = torch.empty(B, C, H, d, dtype=torch.bfloat16, device="cuda")
    lla.lla_attend_prefill(desc, B, C, t, q, zk, zv, ctx, dev(Wk, "bf16"), dev(Wv, "bf16"), None, None,
                           out, lla.workspace(desc, B, C))
    torch.cuda.synchronize()
    o0 = host(out[0])
    for j in (0, 255, 510, 511):
        ref = O.attend_prefill(q0[None, j:j + 1], zk0[None], zv0[None], Wk, Wv, t, [N + j], variant="2d")
        what = f"2d full-size prefill edge row {j}"
        assert_close(o0[None, j:j + 1], ref, "bf16", what)
        _row_check(o0[None, j:j + 1], ref, what)
    del zk, zv, xk, xv, q, out
    torch.cuda.empty_cache()
