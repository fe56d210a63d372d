"""lla_attend_decode_noalloc (the decode entry point that allocates nothing) against
lla_attend_decode with a fresh workspace, through the C ABI: two calls in a row on each path, the
second with a smaller input, so the static scratch is reused with the last call's contents still in
it. The two entry points run the same kernels, so their outputs must be identical; the oracle check
keeps both honest."""
import ctypes

import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import LLA_DT, LLA_VAR, assert_close, assert_lse, dev, host, mfma_lse_slack, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _run(entry, desc, B, t, c, lens, mu, self_token):
    q = dev(c["q"][t], "bf16")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, desc.H), float("nan"), dtype=torch.float32, device="cuda")
    args = (desc, B, t, q, c["_zk"], c["_zv"], dev(np.asarray(lens, np.int32)), c["_Wk"], c["_Wv"],
            c["_muk"] if mu else None, c["_muv"] if mu else None,
            dev(c["k_self"][t], "bf16") if self_token else None,
            dev(c["v_self"][t], "bf16") if self_token else None, out, lse)
    if entry == "noalloc":
        lla.lla_attend_decode_noalloc(*args)
    else:
        lla.lla_attend_decode(*args, lla.workspace(desc, B, 1))
    torch.cuda.synchronize()
    return out, lse


# (variant, H, d, T, r_k, r_v, [(B, n_max, lens), (smaller B, n_max, lens)])
CASES = [
    ("per_head", 16, 128, 4, 32, 32, [(4, 8193, None), (3, 3000, [3000, 3, 777])]),
    ("per_head", 2, 64, 2, 96, 160, [(3, 3000, [3000, 2999, 129]), (2, 2400, [2400, 1])]),
    ("2d", 16, 128, 2, 256, 256, [(8, 2048, None), (3, 700, [700, 65, 1])]),
    ("2d", 20, 64, 2, 64, 64, [(6, 1000, [1000, 999, 17, 0, 640, 1]), (2, 300, [300, 299])]),
]


@pytest.mark.parametrize("variant,H,d,T,rk,rv,calls", CASES,
                         ids=[f"{c[0]}-r{c[4]}-{c[5]}" for c in CASES])
def test_noalloc_matches_workspace_entry(variant, H, d, T, rk, rv, calls):
    for i, (B, n_max, lens) in enumerate(calls):
        lens = [n_max] * B if lens is None else lens
        mu, self_token = (i == 0), (i == 1 or variant == "2d")
        c = synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, 31000 + 10 * i + rk + H,
                              with_mu=mu, q_gain=4.0 if i else 1.0)
        for k in ("zk", "zv", "Wk", "Wv"):
            c["_" + k] = dev(c[k], "bf16")
        c["_muk"], c["_muv"] = dev(c["mu_k"], "bf16"), dev(c["mu_v"], "bf16")
        desc = lla.make_desc(LLA_VAR[variant], LLA_DT["bf16"], H, d, T, rk, rv, n_max)
        assert 0 < lla.lla_workspace_bytes(desc, B, 1) <= lla.LLA_NOALLOC_SCRATCH_BYTES
        t = T - 1
        o_ref, l_ref = _run("workspace", desc, B, t, c, lens, mu, self_token)
        o, l = _run("noalloc", desc, B, t, c, lens, mu, self_token)
        what = f"{variant} r=({rk},{rv}) call {i} B={B} n_max={n_max}"
        assert torch.equal(o, o_ref), what
        assert torch.equal(l, l_ref), what
        ro, rl = O.attend_decode(c["q"][t], c["zk"], c["zv"], c["Wk"], c["Wv"], t, lens,
                                 c["mu_k"] if mu else None, c["mu_v"] if mu else None,
                                 c["k_self"][t] if self_token else None,
                                 c["v_self"][t] if self_token else None, variant=variant)
        live = [b for b in range(B) if self_token or min(max(lens[b], 0), n_max) > 0]
        assert_close(host(o)[live], ro[live], "bf16", what)
        mfma = variant == "2d" and (rk, rv) in ((64, 64), (128, 128), (256, 256))
        slack = mfma_lse_slack(c["q"][t], c["zk"], c["Wk"], t, lens)[live] if mfma else None
        assert_lse(host(l)[live], rl[live], what, slack)


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    # LLA-2D MFMA read at B = 4096: the absorbed queries alone take 4096 * 16 * 256 * 4 B = 64 MiB
    desc = lla.make_desc(lla.LLA_2D, lla.LLA_BF16, 16, 128, 4, 256, 256, 8193)
    B = 4096
    assert lla.lla_workspace_bytes(desc, B, 1) > lla.LLA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, 16, 128, dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lla.LLAError) as e:
        # the buffers below are never read: the call is refused on the host
        st = lla.library().lla_attend_decode_noalloc(
            ctypes.byref(desc), B, 0, q.data_ptr(), z.data_ptr(), z.data_ptr(), None,
            z.data_ptr(), z.data_ptr(), None, None, None, None, q.data_ptr(), None, None)
        lla._check(st, "lla_attend_decode_noalloc")
    assert e.value.status == lla.LLA_ERR_SCRATCH_LIMIT
