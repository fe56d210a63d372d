"""GPU parity of the reconstruct-then-attend comparator (lla_attend_decode_reconstruct).

The comparator rebuilds loop t's K and V (Eq. 3) into the workspace as bf16 rows and attends over
them; it is compared with the oracle's explicit decode with the rebuilt K/V rounded to bf16
(kv_round_bf16), element by element, and at the paper's long-context shape (262k tokens at the
4x geometry, Section 7) both it and the absorbed read are checked on all heads.
"""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import assert_close, assert_lse, dev, host, require_gpu
from tests.test_gpu_parity import mk_desc, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d,rk,rv", [(128, 96, 160), (128, 128, 128), (64, 32, 32), (64, 64, 256)])
def test_reconstruct_sweep(d, rk, rv):
    B, H, T, n_max = 3, 2, 2, 1301
    lens = np.array([1301, 517, 0], np.int32)
    desc = mk_desc("per_head", "bf16", H, d, T, rk, rv, n_max)
    ws = lla.reconstruct_workspace(desc, B)
    for gain, mu, self_token in ((1.0, True, True), (8.0, False, True), (1.0, True, False)):
        c = upload(synth.random_case("per_head", "bf16", B, H, d, T, rk, rv, n_max, 9700 + rk + rv,
                                     with_mu=mu, q_gain=gain), "bf16")
        for t in range(T):
            q = dev(c["q"][t], "bf16")
            out = torch.empty_like(q)
            lse = torch.empty(B, H, device="cuda")
            lla.lla_attend_decode_reconstruct(
                desc, B, t, q, c["_zk"], c["_zv"], dev(lens), c["_Wk"], c["_Wv"],
                c["_muk"] if mu else None, c["_muv"] if mu else None,
                dev(c["k_self"][t], "bf16") if self_token else None,
                dev(c["v_self"][t], "bf16") if self_token else None, out, lse, ws)
            torch.cuda.synchronize()
            ro, rl = O.attend_decode(c["q"][t], c["zk"], c["zv"], c["Wk"], c["Wv"], t, lens,
                                     c["mu_k"] if mu else None, c["mu_v"] if mu else None,
                                     c["k_self"][t] if self_token else None,
                                     c["v_self"][t] if self_token else None, kv_round_bf16=True)
            what = f"reconstruct d={d} r=({rk},{rv}) gain={gain} mu={mu} self={self_token} t={t}"
            assert_close(host(out), ro, "bf16", what)
            assert_lse(host(lse), rl, what)


def test_long_context_262k_both_paths():
    """B=1, H=16, d=128, T=4, r=96/160 (the 4x split), 262144 cached tokens: the absorbed read and
    the comparator against the oracle's absorbed form, every head, loops 0 and 3."""
    B, H, d, T, rk, rv, N = 1, 16, 128, 4, 96, 160, 262144
    n_max = N + 1
    desc = mk_desc("per_head", "bf16", H, d, T, rk, rv, n_max)
    sd = 9800
    zk = synth.device_normal_(torch.empty(B, H, n_max, rk, dtype=torch.bfloat16, device="cuda"), sd + 1)
    zv = synth.device_normal_(torch.empty(B, H, n_max, rv, dtype=torch.bfloat16, device="cuda"), sd + 2)
    # r_v = 160 > d: Gaussian factors with variance 1/r (rebuilt K/V of unit variance)
    wk = synth.normal((T, H, d, rk), sd + 3, "bf16", std=1 / np.sqrt(rk))
    wv = synth.normal((T, H, d, rv), sd + 4, "bf16", std=1 / np.sqrt(rv))
    q_all = synth.normal((T, B, H, d), sd + 5, "bf16")
    lens = np.array([N], np.int32)
    zk_h, zv_h = host(zk), host(zv)
    Wk, Wv = dev(wk, "bf16"), dev(wv, "bf16")
    ws_a = lla.workspace(desc, B)
    ws_r = lla.reconstruct_workspace(desc, B)
    for t in (0, 3):
        q = dev(q_all[t], "bf16")
        ro, rl = O.attend_decode_absorbed(q_all[t], zk_h, zv_h, wk, wv, t, lens)
        for name, fn, ws in (("absorbed", lla.lla_attend_decode, ws_a),
                             ("reconstruct", lla.lla_attend_decode_reconstruct, ws_r)):
            out = torch.empty_like(q)
            lse = torch.empty(B, H, device="cuda")
            fn(desc, B, t, q, zk, zv, dev(lens), Wk, Wv, None, None, None, None, out, lse, ws)
            torch.cuda.synchronize()
            assert_close(host(out), ro, "bf16", f"262k {name} t={t}")
            assert_lse(host(lse), rl, f"262k {name} t={t}")
