"""GPU parity of the gather-indexed decode (token eviction composed with LLA) against the oracle.

Row b attends the cached latents at a listed set of slots (Section 7, "Memory, capacity and
latency"; Appendix C). Small shapes cover every streaming rank pair class, both variants and
storage types, split-K, duplicates, out-of-range slots and ragged counts; the capacity shape runs
at full size with the paper's sink + window policy and a 1024-token budget, checked on sampled
rows.
"""
import numpy as np
import pytest
import torch

from decode_attention_lla_amd import lla, synth
from oracle import lla_oracle as O
from tests.gpu_util import assert_close, assert_lse, dev, host, rel_err, require_gpu
from tests.test_gpu_parity import PAIRS, _fill_device_case, mk_desc, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def gpu_gather(desc, B, t, c, dtype, slots, counts, self_token=True, mu=True):
    q = dev(c["q"][t], dtype)
    out = torch.empty_like(q)
    lse = torch.empty(B, desc.H, dtype=torch.float32, device="cuda")
    budget = slots.shape[1]
    ws = lla.gather_workspace(desc, B, budget)
    ks = dev(c["k_self"][t], dtype) if self_token else None
    vs = dev(c["v_self"][t], dtype) if self_token else None
    lla.lla_attend_decode_gather(desc, B, t, q, c["_zk"], c["_zv"], dev(slots),
                                 None if counts is None else dev(np.asarray(counts, np.int32)),
                                 c["_Wk"], c["_Wv"], c["_muk"] if mu else None,
                                 c["_muv"] if mu else None, ks, vs, out, lse, ws)
    torch.cuda.synchronize()
    return host(out), host(lse)


def oracle_gather(c, t, slots, counts, variant, self_token=True, mu=True):
    return O.attend_decode_gather(c["q"][t], c["zk"], c["zv"], c["Wk"], c["Wv"], t, slots, counts,
                                  c["mu_k"] if mu else None, c["mu_v"] if mu else None,
                                  c["k_self"][t] if self_token else None,
                                  c["v_self"][t] if self_token else None, variant=variant)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant,rk,rv", [("per_head", rk, rv) for rk, rv in PAIRS] +
                         [("2d", 32, 32), ("2d", 128, 128)])
def test_gather_sweep(dtype, variant, rk, rv):
    B, H, d, T, n_max, budget = 3, 2, 64, 2, 1301, 700
    desc = mk_desc(variant, dtype, H, d, T, rk, rv, n_max)
    assert lla.lla_gather_workspace_bytes(desc, B, budget) > 0  # split-K plus the combine
    slots = synth.random_slots(B, budget, n_max, 9100 + rk + rv, p_skip=0.05, p_repeat=0.05)
    counts = [budget, 333, 0]
    for gain, mu, self_token in ((1.0, True, True), (8.0, False, True), (1.0, True, False)):
        c = upload(synth.random_case(variant, dtype, B, H, d, T, rk, rv, n_max, 9000 + rk + rv,
                                     with_mu=mu, q_gain=gain), dtype)
        for t in range(T):
            o, lse = gpu_gather(desc, B, t, c, dtype, slots, counts, self_token, mu)
            ro, rl = oracle_gather(c, t, slots, counts, variant, self_token, mu)
            what = f"{variant} {dtype} r=({rk},{rv}) gain={gain} mu={mu} self={self_token} t={t}"
            assert_close(o, ro, dtype, what)
            assert_lse(lse, rl, what)


def test_gather_short_lists_null_counts_and_empty_rows():
    dtype = "f32"
    B, H, d, T, n_max = 4, 2, 16, 2, 40
    desc = mk_desc("per_head", dtype, H, d, T, 8, 8, n_max)
    c = upload(synth.random_case("per_head", dtype, B, H, d, T, 8, 8, n_max, 9200), dtype)
    slots = np.array([[39, 0, 17, 17, 5], [-1, 40, 41, -7, 99], [1, 2, 3, 4, 5], [6, 6, 6, 6, 6]],
                     dtype=np.int32)
    for counts in (None, [5, 5, 0, 2], [9, -3, 5, 1]):
        for self_token in (True, False):
            o, lse = gpu_gather(desc, B, 1, c, dtype, slots, counts, self_token)
            ro, rl = oracle_gather(c, 1, slots, counts, "per_head", self_token)
            assert_close(o, ro, dtype, f"counts={counts} self={self_token}")
            assert_lse(lse, rl, f"counts={counts} self={self_token}")
    # row 1 lists only out-of-range slots: without a self token it is empty
    o, lse = gpu_gather(desc, B, 0, c, dtype, slots, None, self_token=False)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def test_gather_identity_list_matches_contiguous_read():
    """A list 0 .. n_max-1 with counts = lengths reads exactly the contiguous read's keys. The two
    entry points agree to rounding: the contiguous read may cut a row's tokens among the waves of
    one workgroup while the gather read keeps one wave per split, so the sums run in another order
    (o within one bf16 step, lse within 1e-6)."""
    dtype = "bf16"
    B, H, d, T, n_max = 3, 4, 128, 2, 2000
    desc = mk_desc("per_head", dtype, H, d, T, 24, 24, n_max)
    c = upload(synth.random_case("per_head", dtype, B, H, d, T, 24, 24, n_max, 9300), dtype)
    lens = np.array([2000, 1234, 7], np.int32)
    q = dev(c["q"][1], dtype)
    ks, vs = dev(c["k_self"][1], dtype), dev(c["v_self"][1], dtype)
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty(B, H, device="cuda")
    l2 = torch.empty(B, H, device="cuda")
    lla.lla_attend_decode(desc, B, 1, q, c["_zk"], c["_zv"], dev(lens), c["_Wk"], c["_Wv"],
                          c["_muk"], c["_muv"], ks, vs, o1, l1, lla.workspace(desc, B))
    slots = np.tile(np.arange(n_max, dtype=np.int32), (B, 1))
    lla.lla_attend_decode_gather(desc, B, 1, q, c["_zk"], c["_zv"], dev(slots), dev(lens),
                                 c["_Wk"], c["_Wv"], c["_muk"], c["_muv"], ks, vs, o2, l2,
                                 lla.gather_workspace(desc, B, n_max))
    torch.cuda.synchronize()
    assert rel_err(host(o1), host(o2)) <= 2.0 ** -8
    np.testing.assert_allclose(host(l1), host(l2), rtol=1e-6, atol=1e-6)
    ro, rl = oracle_gather(c, 1, slots, lens, "per_head")
    assert_close(host(o2), ro, dtype)
    assert_lse(host(l2), rl)


def test_gather_long_list_takes_the_unstaged_loop():
    """A 600000-entry list for one row (repeats and out-of-range slots): 247 splits of 2432
    positions, longer than the kernel stages in LDS, so the one-batch loop runs."""
    dtype = "bf16"
    B, H, d, T, n_max, budget = 1, 2, 16, 1, 5000, 600000
    desc = mk_desc("per_head", dtype, H, d, T, 8, 8, n_max)
    c = upload(synth.random_case("per_head", dtype, B, H, d, T, 8, 8, n_max, 9250), dtype)
    slots = synth.random_slots(B, budget, n_max, 9251, p_skip=0.02, p_repeat=0.3)
    o, lse = gpu_gather(desc, B, 0, c, dtype, slots, [budget - 17])
    ro, rl = oracle_gather(c, 0, slots, [budget - 17], "per_head")
    assert_close(o, ro, dtype, "600k list")
    assert_lse(lse, rl, "600k list")


def test_gather_plan_resplit_for_the_staged_list():
    """2048 (row, head) units and a 5000-entry list: the streaming plan's 2 splits of 2560
    positions are re-planned as 3 splits of at most 2048, which the kernel stages in LDS."""
    dtype = "bf16"
    B, H, d, T, n_max, budget = 32, 64, 16, 1, 5200, 5000
    desc = mk_desc("per_head", dtype, H, d, T, 24, 24, n_max)
    ws_bytes = lla.lla_gather_workspace_bytes(desc, B, budget)
    assert ws_bytes >= B * H * 3 * (2 + 24) * 4  # three splits' partials
    c = upload(synth.random_case("per_head", dtype, B, H, d, T, 24, 24, n_max, 9260, q_gain=4.0), dtype)
    slots = synth.random_slots(B, budget, n_max, 9261, p_skip=0.02, p_repeat=0.05)
    counts = np.full(B, budget, np.int32)
    counts[::5] = [4097, 2048, 2049, 1, 0, 3000, 5000][: len(counts[::5])]
    o, lse = gpu_gather(desc, B, 0, c, dtype, slots, counts)
    ro, rl = oracle_gather(c, 0, slots, counts, "per_head")
    assert_close(o, ro, dtype, "re-split list")
    assert_lse(lse, rl, "re-split list")


def test_capacity_eviction_full_size_sampled():
    """Capacity shape (B=768, H=16, d=128, T=4, r=24, N=4096 cached) read through a 1024-slot
    StreamingLLM list (4 sinks + the 1020 most recent tokens), at the benchmark's launch shape."""
    s = synth.CASES["capacity"]
    g = _fill_device_case(s)
    desc = mk_desc(s.variant, s.dtype, s.H, s.d, s.T, s.r_k, s.r_v, s.n_max)
    keep = np.asarray(O.streaming_kept_slots(s.N, 4, 1020), np.int32)
    slots = np.tile(keep, (s.B, 1))
    Wk, Wv = dev(g["Wk"], "bf16"), dev(g["Wv"], "bf16")
    ws = lla.gather_workspace(desc, s.B, keep.size)
    rows = sorted({0, 383, 767, *np.random.default_rng(synth.seed(s.case, synth.SEED_SAMPLE)).choice(768, 3, replace=False).tolist()})
    zk_rows, zv_rows = host(g["zk"][rows]), host(g["zv"][rows])
    d_slots = dev(slots)
    for t in range(s.T):
        q = dev(g["q"][t], "bf16")
        out = torch.empty_like(q)
        lse = torch.empty(s.B, s.H, device="cuda")
        lla.lla_attend_decode_gather(desc, s.B, t, q, g["zk"], g["zv"], d_slots, None, Wk, Wv,
                                     None, None, dev(g["k_self"][t], "bf16"),
                                     dev(g["v_self"][t], "bf16"), out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = O.attend_decode_gather(g["q"][t][rows], zk_rows, zv_rows, g["Wk"], g["Wv"], t,
                                        slots[rows], None, None, None, g["k_self"][t][rows],
                                        g["v_self"][t][rows])
        assert_close(host(out)[rows], ro, s.dtype, f"capacity eviction t={t}")
        assert_lse(host(lse)[rows], rl, f"capacity eviction t={t}")
    del g
    torch.cuda.empty_cache()
