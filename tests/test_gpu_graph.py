"""A decode step captured in a HIP graph: T loop reads (through the workspace entry point or the
no-allocation one) and the encode of the new token, replayed several times. Before each replay the
queries are rewritten eagerly; every replay must reproduce, bit for bit, an eager run of the same
step on the same inputs. Per-head with token splits (partial + combine kernels) and LLA-2D on the
MFMA read (q~ projection, partial, combine)."""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from tests.gpu_util import dev, require_gpu
from tests.test_gpu_parity import mk_desc, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("variant,H,rk,rv,B,n_max", [("per_head", 4, 32, 32, 2, 5000),
                                                     ("2d", 20, 64, 64, 3, 700)])
def test_captured_decode_step_replays(variant, H, rk, rv, B, n_max, noalloc):
    d, T = 64, 2
    desc = mk_desc(variant, "bf16", H, d, T, rk, rv, n_max)
    c = upload(synth.random_case(variant, "bf16", B, H, d, T, rk, rv, n_max, 9700 + rk), "bf16")
    lens_h = np.array([n_max - 1 - 7 * b for b in range(B)], np.int32)  # the encode writes slot lens[b]
    lens = dev(lens_h)
    Ek, Ev = dev(c["Ek"], "bf16"), dev(c["Ev"], "bf16")
    ks, vs = dev(c["k_self"], "bf16"), dev(c["v_self"], "bf16")
    xk = dev(synth.normal((B, 1, T, H, d), 9701, "bf16"), "bf16")
    xv = dev(synth.normal((B, 1, T, H, d), 9702, "bf16"), "bf16")
    q = dev(c["q"], "bf16")
    out = torch.empty(T, B, H, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T, B, H, dtype=torch.float32, device="cuda")
    ws = None if noalloc else lla.workspace(desc, B, 1)
    if not noalloc and variant == "per_head":
        assert ws is not None  # the plan splits the tokens: partial and combine kernels

    def step(stream):
        for t in range(T):
            if noalloc:
                lla.lla_attend_decode_noalloc(desc, B, t, q[t], c["_zk"], c["_zv"], lens, c["_Wk"], c["_Wv"],
                                              c["_muk"], c["_muv"], ks[t], vs[t], out[t], lse[t], stream)
            else:
                lla.lla_attend_decode(desc, B, t, q[t], c["_zk"], c["_zv"], lens, c["_Wk"], c["_Wv"],
                                      c["_muk"], c["_muv"], ks[t], vs[t], out[t], lse[t], ws, stream)
        lla.lla_encode(desc, B, 1, xk, xv, Ek, Ev, None, None, lens, c["_zk"], c["_zv"], stream)

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    rng = np.random.default_rng(9703)
    for rep in range(3):
        q.copy_(torch.from_numpy(rng.standard_normal(tuple(q.shape)).astype(np.float32)).to(torch.bfloat16))
        torch.cuda.synchronize()
        step(torch.cuda.current_stream())  # eager reference
        torch.cuda.synchronize()
        want_o, want_l = out.clone(), lse.clone()
        zk_after = c["_zk"].clone()
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o), f"replay {rep}: outputs differ from the eager step"
        assert torch.equal(lse, want_l), f"replay {rep}: lse differs from the eager step"
        assert torch.equal(c["_zk"], zk_after), f"replay {rep}: encoded cache differs"
