"""GPU parity at batch counts past 65535 in a launch dimension.

HIP caps the y and z grid dimensions at 65535 workgroups, so every launch keeps batch-dependent
counts in x. These cases put the batch-dependent count of each multi-dimensional launch past
that cap, with short ragged caches, and compare sampled sequences with the oracle:
the LLA-2D MFMA read (its query projection, split read and merge, with and without the fused
rotary branch) at B = 270000, the per-head rotary read at B = 70000, and the
reconstruct comparator at B * H = 67200.
"""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import assert_close, assert_lse, dev, host, require_gpu
from tests.test_gpu_parity import mk_desc

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rows(B, rng):
    return sorted({0, 1, B // 2, B - 1, *(int(x) for x in rng.integers(0, B, 4))})


def _lens(B, n_max, rng):
    lens = rng.integers(0, n_max + 1, B).astype(np.int32)
    lens[0], lens[-1] = n_max, 0
    return lens


@pytest.mark.parametrize("rope", [False, True])
def test_lla2d_decode_batch_past_grid_limit(rope):
    B, H, d, T, r, n_max, d_rope = 270000, 2, 64, 2, 64, 17, 32
    rng = np.random.default_rng(20001)
    desc = mk_desc("2d", "bf16", H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, n_max, r, dtype=BF, device="cuda"), 20002)
    zv = synth.device_normal_(torch.empty(B, n_max, r, dtype=BF, device="cuda"), 20003)
    Wk = synth.orthonormal_W_2d(T, H, d, r, 20004, "bf16")
    Wv = synth.orthonormal_W_2d(T, H, d, r, 20005, "bf16")
    q = synth.device_normal_(torch.empty(B, H, d, dtype=BF, device="cuda"), 20006)
    ks = synth.device_normal_(torch.empty(B, H, d, dtype=BF, device="cuda"), 20007)
    vs = synth.device_normal_(torch.empty(B, H, d, dtype=BF, device="cuda"), 20008)
    lens = _lens(B, n_max, rng)
    rows = _rows(B, rng)
    out = torch.empty(B, H, d, dtype=BF, device="cuda")
    lse = torch.empty(B, H, device="cuda")
    t = 1
    if rope:
        kr = synth.device_normal_(torch.empty(B, n_max, d_rope, dtype=BF, device="cuda"), 20009)
        krs = synth.device_normal_(torch.empty(B, d_rope, dtype=BF, device="cuda"), 20010)
        qr = synth.device_normal_(torch.empty(B, H, d_rope, dtype=BF, device="cuda"), 20011)
        ws = lla.rope_workspace(desc, B)
        lla.lla_attend_decode_rope(desc, B, t, q, qr, zk, zv, kr, d_rope, 0.0, dev(lens),
                                   dev(Wk, "bf16"), dev(Wv, "bf16"), None, None, ks, vs, krs, out,
                                   lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode_rope(host(q[rows]), host(qr[rows]), host(zk[rows]), host(zv[rows]),
                                      host(kr[rows]), Wk, Wv, t, lens[rows], None, None,
                                      host(ks[rows]), host(vs[rows]), host(krs[rows]), variant="2d")
    else:
        ws = lla.workspace(desc, B)
        lla.lla_attend_decode(desc, B, t, q, zk, zv, dev(lens), dev(Wk, "bf16"), dev(Wv, "bf16"),
                              None, None, ks, vs, out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode(host(q[rows]), host(zk[rows]), host(zv[rows]), Wk, Wv, t,
                                 lens[rows], None, None, host(ks[rows]), host(vs[rows]),
                                 variant="2d")
    what = f"2d decode B={B} rope={rope} rows={rows}"
    assert_close(host(out[rows]), ro, "bf16", what)
    assert_lse(host(lse[rows]), rl, what)


def test_per_head_rope_batch_past_grid_limit():
    B, H, d, T, r, n_max, d_rope = 70000, 1, 64, 1, 24, 17, 32
    rng = np.random.default_rng(20101)
    desc = mk_desc("per_head", "bf16", H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, H, n_max, r, dtype=BF, device="cuda"), 20102)
    zv = synth.device_normal_(torch.empty(B, H, n_max, r, dtype=BF, device="cuda"), 20103)
    Wk = synth.orthonormal_W(T, H, d, r, 20104, "bf16")
    Wv = synth.orthonormal_W(T, H, d, r, 20105, "bf16")
    q = synth.device_normal_(torch.empty(B, H, d, dtype=BF, device="cuda"), 20106)
    qr = synth.device_normal_(torch.empty(B, H, d_rope, dtype=BF, device="cuda"), 20107)
    kr = synth.device_normal_(torch.empty(B, n_max, d_rope, dtype=BF, device="cuda"), 20108)
    krs = synth.device_normal_(torch.empty(B, d_rope, dtype=BF, device="cuda"), 20109)
    ks = synth.device_normal_(torch.empty(B, H, d, dtype=BF, device="cuda"), 20110)
    vs = synth.device_normal_(torch.empty(B, H, d, dtype=BF, device="cuda"), 20111)
    lens = _lens(B, n_max, rng)
    rows = _rows(B, rng)
    out = torch.empty(B, H, d, dtype=BF, device="cuda")
    lse = torch.empty(B, H, device="cuda")
    ws = lla.rope_workspace(desc, B)
    lla.lla_attend_decode_rope(desc, B, 0, q, qr, zk, zv, kr, d_rope, 0.0, dev(lens), dev(Wk, "bf16"),
                               dev(Wv, "bf16"), None, None, ks, vs, krs, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = O.attend_decode_rope(host(q[rows]), host(qr[rows]), host(zk[rows]), host(zv[rows]),
                                  host(kr[rows]), Wk, Wv, 0, lens[rows], None, None, host(ks[rows]),
                                  host(vs[rows]), host(krs[rows]))
    what = f"per-head rope decode B={B} rows={rows}"
    assert_close(host(out[rows]), ro, "bf16", what)
    assert_lse(host(lse[rows]), rl, what)


def test_reconstruct_heads_times_batch_past_grid_limit():
    B, H, d, T, rk, rv, n_max = 4200, 16, 64, 1, 32, 64, 17
    rng = np.random.default_rng(20201)
    desc = mk_desc("per_head", "bf16", H, d, T, rk, rv, n_max)
    zk = synth.device_normal_(torch.empty(B, H, n_max, rk, dtype=BF, device="cuda"), 20202)
    zv = synth.device_normal_(torch.empty(B, H, n_max, rv, dtype=BF, device="cuda"), 20203)
    Wk = synth.orthonormal_W(T, H, d, rk, 20204, "bf16")
    Wv = synth.orthonormal_W(T, H, d, rv, 20205, "bf16")
    q = synth.device_normal_(torch.empty(B, H, d, dtype=BF, device="cuda"), 20206)
    lens = _lens(B, n_max, rng)
    rows = _rows(B, rng)
    out = torch.empty(B, H, d, dtype=BF, device="cuda")
    lse = torch.empty(B, H, device="cuda")
    ws = lla.reconstruct_workspace(desc, B)
    lla.lla_attend_decode_reconstruct(desc, B, 0, q, zk, zv, dev(lens), dev(Wk, "bf16"),
                                      dev(Wv, "bf16"), None, None, None, None, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = O.attend_decode(host(q[rows]), host(zk[rows]), host(zv[rows]), Wk, Wv, 0, lens[rows],
                             kv_round_bf16=True)
    what = f"reconstruct B*H={B * H} rows={rows}"
    assert_close(host(out[rows]), ro, "bf16", what)
    assert_lse(host(lse[rows]), rl, what)
