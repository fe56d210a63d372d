"""The C ABI on the CPU: the library loads, exports what include/lla.h declares, and rejects bad
arguments on the host before launching anything (no GPU needed, no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

from decode_attention_lla_amd import lla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

if not os.path.exists(lla.LIB_PATH):
    pytest.skip("liblla.so not built (run python -m decode_attention_lla_amd.build)", allow_module_level=True)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "lla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lla_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"lla_encode", "lla_attend_decode", "lla_attend_prefill", "lla_workspace_bytes",
            "lla_status_string", "lla_abi_version"} <= set(names)
    lib = ctypes.CDLL(lla.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert lla.lla_abi_version() == 2
    assert lla.lla_status_string(lla.LLA_OK) == "ok"
    assert "workspace" in lla.lla_status_string(lla.LLA_ERR_WORKSPACE)
    assert lla.lla_status_string(99) == "unknown status"


# fake, aligned, never-dereferenced addresses: every call below fails validation first
A = ctypes.c_void_p(0x10000)
M = ctypes.c_void_p(0x10008)  # misaligned
N = None
S = ctypes.c_void_p(0)


def desc(**kw):
    base = dict(variant=lla.LLA_PER_HEAD, dtype=lla.LLA_BF16, H=16, d_head=128, T=4, r_k=32,
                r_v=32, n_max=4097, scale=0.0)
    base.update(kw)
    return lla.make_desc(**base)


def decode(d, B=2, t=0, q=A, zk=A, zv=A, lens=N, Wk=A, Wv=A, muk=N, muv=N, ks=N, vs=N, out=A,
           lse=N, ws=N, wsb=0):
    lib = lla.library()
    return lib.lla_attend_decode(ctypes.byref(d), B, t, q, zk, zv, lens, Wk, Wv, muk, muv, ks, vs,
                                 out, lse, ws, ctypes.c_size_t(wsb), S)


def encode(d, B=2, C=1, xk=A, xv=A, Ek=A, Ev=A, muk=N, muv=N, pos=A, zk=A, zv=A):
    lib = lla.library()
    return lib.lla_encode(ctypes.byref(d), B, C, xk, xv, Ek, Ev, muk, muv, pos, zk, zv, S)


def prefill(d, B=2, C=4, t=0, q=A, zk=A, zv=A, ctx=A, Wk=A, Wv=A, out=A, ws=N, wsb=0):
    lib = lla.library()
    return lib.lla_attend_prefill(ctypes.byref(d), B, C, t, q, zk, zv, ctx, Wk, Wv, N, N, out, ws,
                                  ctypes.c_size_t(wsb), S)


@pytest.mark.parametrize("kw", [
    dict(t=4), dict(t=-1), dict(B=0), dict(q=N), dict(zk=N), dict(Wv=N), dict(out=N),
    dict(q=M), dict(lse=M), dict(ks=A), dict(vs=A),
])
def test_decode_rejects_bad_arguments(kw):
    d = desc(n_max=100)  # small cache: no split, no workspace needed
    assert decode(d, **kw) == lla.LLA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(H=0), dict(d_head=12), dict(d_head=264), dict(T=0), dict(n_max=0), dict(variant=3),
    dict(dtype=7), dict(scale=-1.0), dict(scale=float("inf")),
])
def test_bad_descriptor(kw):
    d = desc(**kw)
    assert decode(d) == lla.LLA_ERR_INVALID_ARG
    assert encode(d) == lla.LLA_ERR_INVALID_ARG
    assert lla.lla_workspace_bytes(d, 2, 1) == 0


def test_unsupported_ranks():
    assert decode(desc(r_k=33, r_v=33, n_max=100)) == lla.LLA_ERR_UNSUPPORTED
    assert decode(desc(r_k=24, r_v=32, n_max=100)) == lla.LLA_ERR_UNSUPPORTED


def test_workspace_checked_before_launch():
    d = desc(n_max=16385)  # 2 x 16 units over 16385 slots: more parts than a workgroup's waves
    need = lla.lla_workspace_bytes(d, 2, 1)
    assert need > 0
    assert decode(d, B=2) == lla.LLA_ERR_WORKSPACE
    assert decode(d, B=2, ws=A, wsb=need - 4) == lla.LLA_ERR_WORKSPACE


def test_workspace_sizes():
    # no split when B*H alone fills the chip (capacity shape)
    assert lla.lla_workspace_bytes(desc(r_k=24, r_v=24), 768, 1) == 0
    # the Ouro-shaped layer (512 units) splits its tokens among the waves of one workgroup only
    assert lla.lla_workspace_bytes(desc(), 32, 1) == 0
    # split partials are (m, l, a[r_v]) floats per (b, h, split)
    n = lla.lla_workspace_bytes(desc(n_max=16385), 2, 1)
    assert n % (2 * 16 * (2 + 32) * 4) == 0
    splits = n // (2 * 16 * (2 + 32) * 4)
    assert 2 <= splits <= 64


def test_encode_rejects_bad_arguments():
    d = desc()
    assert encode(d, C=0) == lla.LLA_ERR_INVALID_ARG
    assert encode(d, C=5000) == lla.LLA_ERR_INVALID_ARG
    assert encode(d, pos=N) == lla.LLA_ERR_INVALID_ARG
    assert encode(d, xk=M) == lla.LLA_ERR_INVALID_ARG
    assert encode(d, muk=M) == lla.LLA_ERR_INVALID_ARG
    assert encode(d, zv=N) == lla.LLA_ERR_INVALID_ARG
    # B * C tokens are counted in 32-bit integers by the encode kernels: 2^31 of them are refused
    small = desc(H=1, d_head=8, T=1, r_k=8, r_v=8, n_max=1024)
    assert encode(small, B=2 ** 21, C=1024) == lla.LLA_ERR_INVALID_ARG


def test_prefill_rejects_bad_arguments():
    d = desc(n_max=64)
    assert prefill(d, t=4) == lla.LLA_ERR_INVALID_ARG
    assert prefill(d, C=0) == lla.LLA_ERR_INVALID_ARG
    assert prefill(d, C=65) == lla.LLA_ERR_INVALID_ARG
    assert prefill(d, ctx=N) == lla.LLA_ERR_INVALID_ARG
    assert prefill(desc(n_max=64, r_k=33, r_v=33)) == lla.LLA_ERR_UNSUPPORTED


def test_binding_checks_shapes_without_gpu():
    torch = pytest.importorskip("torch")
    d = desc(n_max=8)
    q = torch.zeros(2, 16, 128)  # CPU tensor: rejected before any library call
    with pytest.raises(ValueError):
        lla.lla_attend_decode(d, 2, 0, q, q, q, None, q, q, None, None, None, None, q)


def test_2d_mfma_workspace_matches_its_plan():
    """The LLA-2D MFMA decode needs q~, beta and split partials; the call refuses any smaller
    workspace before launching (the split plan is computed once, by the call that sizes it)."""
    d = desc(variant=lla.LLA_2D, r_k=256, r_v=256, n_max=8193)
    need = lla.lla_workspace_bytes(d, 128, 1)
    bh = 128 * 16
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    fixed = al(bh * 256 * 4) + al(bh * 4)
    assert (need - fixed) % (bh * 258 * 4) == 0
    splits = (need - fixed) // (bh * 258 * 4)
    assert 1 <= splits <= 64
    assert decode(d, B=128, ws=A, wsb=need - 1) == lla.LLA_ERR_WORKSPACE
    assert decode(d, B=128) == lla.LLA_ERR_WORKSPACE


def test_prefill_workspace_checked_before_launch():
    d = desc(n_max=4097, r_k=24, r_v=24)
    need = lla.lla_workspace_bytes(d, 2, 64)
    if need > 0:
        assert prefill(d, B=2, C=64, ws=A, wsb=need - 4) == lla.LLA_ERR_WORKSPACE


def gather(d, B=2, t=0, q=A, zk=A, zv=A, slots=A, budget=64, counts=N, Wk=A, Wv=A, ks=N, vs=N,
           out=A, lse=N, ws=N, wsb=0):
    lib = lla.library()
    return lib.lla_attend_decode_gather(ctypes.byref(d), B, t, q, zk, zv, slots, budget, counts,
                                        Wk, Wv, N, N, ks, vs, out, lse, ws, ctypes.c_size_t(wsb), S)


@pytest.mark.parametrize("kw", [
    dict(slots=N), dict(slots=M), dict(budget=0), dict(budget=-4), dict(counts=M), dict(t=4),
    dict(B=0), dict(q=N), dict(out=M), dict(ks=A), dict(B=1 << 20, budget=1 << 12),
])
def test_gather_rejects_bad_arguments(kw):
    assert gather(desc(n_max=100), **kw) == lla.LLA_ERR_INVALID_ARG


def test_gather_unsupported_and_workspace():
    # the LLA-2D MFMA-only pairs have no streaming kernel, so no gather path
    assert gather(desc(variant=lla.LLA_2D, r_k=64, r_v=128, n_max=100)) == lla.LLA_ERR_UNSUPPORTED
    assert gather(desc(r_k=24, r_v=32, n_max=100)) == lla.LLA_ERR_UNSUPPORTED
    d = desc()  # 2 x 16 units over a 4096-slot list: split-K, needs a workspace
    need = lla.lla_gather_workspace_bytes(d, 2, 4096)
    assert need > 0 and need % (2 * 16 * (2 + 32) * 4) == 0
    assert gather(d, budget=4096) == lla.LLA_ERR_WORKSPACE
    assert gather(d, budget=4096, ws=A, wsb=need - 4) == lla.LLA_ERR_WORKSPACE
    # the split plan follows the list length, not the cache size
    assert lla.lla_gather_workspace_bytes(d, 2, 64) == 0
    assert lla.lla_gather_workspace_bytes(desc(H=0), 2, 64) == 0
    assert lla.lla_gather_workspace_bytes(d, 2, 0) == 0


def _one_wave_splits(H, B, n_max):
    """Token splits of the streaming plan with one wave per (row, head, split): about 2048 waves,
    parts of at least 256 tokens, at most 256 splits, chunks a multiple of 128 tokens."""
    want = min(-(-2048 // (B * H)), max(n_max // 256, 1))
    s = min(max(want, 1), 256)
    c = -(-n_max // s)
    c = -(-c // 128) * 128
    return -(-n_max // c)


def test_rope_workspace_follows_the_rope_plan():
    """The rotary read forms its rotary scores inside the read, so its workspace holds only split
    partials: under the decode plan where heads are not grouped (H < 8, or groups of 8 that would
    leave more than a quarter of the waves as placeholders), else under the one-wave plan of the
    head-group read (none when that plan has one split per row and head)."""
    lib = lla.library()
    for d, B in ((desc(H=2, r_k=24, r_v=24, n_max=70000), 3), (desc(H=9, r_k=24, r_v=24, n_max=9000), 2),
                 (desc(H=5, r_k=96, r_v=160, n_max=70000), 1)):
        need = lib.lla_rope_workspace_bytes(ctypes.byref(d), B)
        assert need == lla.lla_workspace_bytes(d, B) > 0
    for H, r, n_max, B in ((16, 24, 4097, 768), (16, 24, 4097, 2), (64, 8, 5000, 64), (40, 32, 9000, 3),
                           (130, 24, 3000, 1)):
        d = desc(H=H, r_k=r, r_v=r, n_max=n_max)
        s = _one_wave_splits(H, B, n_max)
        want = 0 if s == 1 else B * H * s * (2 + r) * 4
        assert lib.lla_rope_workspace_bytes(ctypes.byref(d), B) == want, (H, r, n_max, B)
    assert lib.lla_rope_workspace_bytes(ctypes.byref(desc(H=16, r_k=24, r_v=24, n_max=4097)), 2) > 0


def test_gather_plan_keeps_splits_within_the_staged_list():
    """The gather plan prefers splits of at most 2048 list positions (the kernel stages such a
    split's slots in LDS) while 256 splits allow it; the workspace holds one partial per split."""
    per_split = lambda d, B: B * d.H * (2 + d.r_v) * 4  # noqa: E731
    d = desc(H=64, r_k=24, r_v=24, n_max=5200)
    # 32 x 64 units: the streaming plan would take 2 splits of 2560 positions; 3 of 1792 instead
    assert lla.lla_gather_workspace_bytes(d, 32, 5000) == 3 * per_split(d, 32)
    # a list of 2048 positions fits one staged split: no split-K
    assert lla.lla_gather_workspace_bytes(d, 64, 2048) == 0
    # 600000 positions on 2 units: at most 256 splits (the combine's limit); 2344 positions
    # rounded up to 2432 (whole 128-position tiles) give 247 splits, longer than the staged list
    d1 = desc(H=2, r_k=8, r_v=8, n_max=5000)
    assert lla.lla_gather_workspace_bytes(d1, 1, 600000) == 247 * per_split(d1, 1)


def test_latent_row_bytes():
    f = lla.lla_latent_row_bytes
    assert (f(lla.LLA_F32, 24), f(lla.LLA_BF16, 24), f(lla.LLA_BF16_Q8, 24)) == (96, 48, 32)
    assert [f(lla.LLA_BF16_Q8, r) for r in (1, 8, 12, 13, 16, 28, 32, 256)] == \
        [16, 16, 16, 32, 32, 32, 48, 272]
    assert f(7, 8) == 0 and f(lla.LLA_BF16_Q8, 0) == 0
    assert [f(lla.LLA_BF16_I8, r) for r in (1, 12, 13, 24, 32)] == [16, 16, 32, 32, 48]


def quantize(d, B=2, C=1, ks=A, vs=A, pos=A, zk=A, zv=A):
    return lla.library().lla_quantize_latents(ctypes.byref(d), B, C, ks, vs, pos, zk, zv, S)


@pytest.mark.parametrize("kw,dkw", [
    (dict(), dict(dtype=lla.LLA_BF16)), (dict(B=0), {}), (dict(C=0), {}), (dict(C=101), {}),
    (dict(ks=N), {}), (dict(vs=M), {}), (dict(pos=N), {}), (dict(zk=M), {}), (dict(zv=N), {}),
    (dict(), dict(r_k=513)),
])
@pytest.mark.parametrize("low", ["LLA_BF16_Q8", "LLA_BF16_I8"])
def test_quantize_rejects_bad_arguments(kw, dkw, low):
    base = dict(dtype=getattr(lla, low), n_max=100, r_k=24, r_v=24)
    base.update(dkw)
    assert quantize(desc(**base), **kw) == lla.LLA_ERR_INVALID_ARG


@pytest.mark.parametrize("low", ["LLA_BF16_Q8", "LLA_BF16_I8"])
def test_low_bit_support_matrix(low):
    q8 = dict(dtype=getattr(lla, low), n_max=100)
    assert encode(desc(r_k=24, r_v=24, **q8)) == lla.LLA_ERR_UNSUPPORTED
    assert decode(desc(r_k=64, r_v=64, **q8)) == lla.LLA_ERR_UNSUPPORTED
    assert gather(desc(r_k=96, r_v=160, **q8)) == lla.LLA_ERR_UNSUPPORTED
    assert prefill(desc(r_k=128, r_v=128, **q8)) == lla.LLA_ERR_UNSUPPORTED
    # LLA-2D low-bit rows on the MFMA read (d_head <= 128): supported, it needs its workspace
    assert decode(desc(variant=lla.LLA_2D, r_k=256, r_v=256, **q8)) == lla.LLA_ERR_WORKSPACE
    # the absorbed queries, beta and one split's partials: 2*16*256*4 + 256 + 2*16*(2+256)*4 bytes
    assert lla.lla_workspace_bytes(desc(variant=lla.LLA_2D, r_k=256, r_v=256, **q8), 2, 1) == \
        2 * 16 * 256 * 4 + 256 + 2 * 16 * 258 * 4
    assert decode(desc(variant=lla.LLA_2D, r_k=256, r_v=256, d_head=160, **q8)) == lla.LLA_ERR_UNSUPPORTED
    # same split plan and workspace as bf16 storage on the streaming path
    assert lla.lla_workspace_bytes(desc(r_k=32, r_v=32, dtype=q8["dtype"]), 32, 1) == \
        lla.lla_workspace_bytes(desc(r_k=32, r_v=32), 32, 1)
    assert lla.lla_workspace_bytes(desc(r_k=24, r_v=24, dtype=q8["dtype"]), 2, 1) > 0  # compiled
    assert lla.lla_workspace_bytes(desc(r_k=96, r_v=96, dtype=q8["dtype"]), 2, 1) > 0  # 112-byte rows
    assert decode(desc(r_k=96, r_v=96, dtype=q8["dtype"], n_max=70000)) == lla.LLA_ERR_WORKSPACE  # supported
    # an unknown dtype is an invalid descriptor
    assert decode(desc(r_k=24, r_v=24, dtype=4, n_max=100)) == lla.LLA_ERR_INVALID_ARG


def reconstruct(d, B=2, t=0, ws=N, wsb=0, **kw):
    args = dict(q=A, zk=A, zv=A, lens=N, Wk=A, Wv=A, muk=N, muv=N, ks=N, vs=N, out=A, lse=N)
    args.update(kw)
    return lla.library().lla_attend_decode_reconstruct(
        ctypes.byref(d), B, t, args["q"], args["zk"], args["zv"], args["lens"], args["Wk"],
        args["Wv"], args["muk"], args["muv"], args["ks"], args["vs"], args["out"], args["lse"], ws,
        ctypes.c_size_t(wsb), S)


def test_reconstruct_support_and_workspace():
    ok = dict(r_k=96, r_v=160, n_max=100)
    assert reconstruct(desc(**ok), q=N) == lla.LLA_ERR_INVALID_ARG
    assert reconstruct(desc(**ok), t=4) == lla.LLA_ERR_INVALID_ARG
    for bad in (dict(d_head=96), dict(dtype=lla.LLA_F32), dict(variant=lla.LLA_2D),
                dict(r_k=24, r_v=24), dict(r_k=512, r_v=32)):
        base = dict(ok)
        base.update(bad)
        assert reconstruct(desc(**base)) == lla.LLA_ERR_UNSUPPORTED, bad
    d = desc(**ok)
    need = lla.lla_reconstruct_workspace_bytes(d, 2)
    kv = 2 * 16 * 100 * 128 * 2
    assert need >= 2 * kv + 16 * 128 * 128 * 2  # rebuilt K and V plus the identity factors
    assert reconstruct(d) == lla.LLA_ERR_WORKSPACE
    assert reconstruct(d, ws=A, wsb=need - 1) == lla.LLA_ERR_WORKSPACE
    assert lla.lla_reconstruct_workspace_bytes(desc(H=0), 2) == 0


def rope_decode(d, B=2, t=0, d_rope=64, base=0.0, ws=N, wsb=0, **kw):
    a = dict(q=A, qr=A, zk=A, zv=A, kr=A, lens=N, Wk=A, Wv=A, ks=N, vs=N, krs=N, out=A, lse=N)
    a.update(kw)
    return lla.library().lla_attend_decode_rope(
        ctypes.byref(d), B, t, a["q"], a["qr"], a["zk"], a["zv"], a["kr"], d_rope,
        ctypes.c_float(base), a["lens"], a["Wk"], a["Wv"], N, N, a["ks"], a["vs"], a["krs"],
        a["out"], a["lse"], ws, ctypes.c_size_t(wsb), S)


def test_rope_arguments_support_and_workspace():
    d = desc(r_k=24, r_v=24, n_max=100)
    for kw in (dict(qr=N), dict(kr=M), dict(ks=A, vs=A), dict(krs=A), dict(base=-1.0),
               dict(base=float("inf")), dict(t=4)):
        assert rope_decode(d, **kw) == lla.LLA_ERR_INVALID_ARG, kw
    assert rope_decode(d, d_rope=48) == lla.LLA_ERR_UNSUPPORTED
    assert rope_decode(desc(r_k=24, r_v=24, n_max=100, dtype=lla.LLA_F32)) == lla.LLA_ERR_UNSUPPORTED
    assert rope_decode(desc(r_k=64, r_v=128, n_max=100)) == lla.LLA_ERR_UNSUPPORTED
    # no per-head LDS cap on the streaming read any more: a long cache with many heads stops at the
    # workspace check
    assert rope_decode(desc(r_k=24, r_v=24, n_max=70000, H=200), B=1, d_rope=128) == lla.LLA_ERR_WORKSPACE
    # the LLA-2D MFMA read fuses the branch and has no per-head LDS cap: H * d_rope > 16384 is
    # accepted (the call then stops at the workspace check)
    big2d = desc(variant=lla.LLA_2D, r_k=64, r_v=64, d_head=32, n_max=100, H=200)
    assert rope_decode(big2d, d_rope=128) == lla.LLA_ERR_WORKSPACE
    # the rotary scores are formed inside the read: the workspace holds only split partials, and
    # a long cache at small B * H needs them
    dl = desc(r_k=24, r_v=24, n_max=5000)
    need = lla.lla_rope_workspace_bytes(dl, 2)
    assert need == 2 * 16 * _one_wave_splits(16, 2, 5000) * (2 + 24) * 4 > 0  # head groups of 8
    assert need % (2 * 16 * (2 + 24) * 4) == 0
    assert rope_decode(dl) == lla.LLA_ERR_WORKSPACE
    assert rope_decode(dl, ws=A, wsb=need - 1) == lla.LLA_ERR_WORKSPACE
    lib = lla.library()
    w = lambda dd, **k: lib.lla_rope_write(ctypes.byref(dd), k.get("B", 2), k.get("C", 1),
                                           k.get("dr", 64), ctypes.c_float(k.get("base", 0.0)),
                                           k.get("x", A), k.get("pos", A), k.get("kr", A), S)
    assert w(d, dr=63) == lla.LLA_ERR_INVALID_ARG
    assert w(d, C=101) == lla.LLA_ERR_INVALID_ARG
    assert w(d, pos=N) == lla.LLA_ERR_INVALID_ARG
    assert w(desc(dtype=lla.LLA_F32, n_max=100)) == lla.LLA_ERR_INVALID_ARG


def test_prefill_rope_arguments_and_support():
    lib = lla.library()

    def call(d, B=2, C=4, t=0, d_rope=64, base=0.0, **kw):
        a = dict(q=A, qr=A, zk=A, zv=A, kr=A, ctx=A, Wk=A, Wv=A, out=A, ws=N, wsb=0)
        a.update(kw)
        return lib.lla_attend_prefill_rope(ctypes.byref(d), B, C, t, a["q"], a["qr"], a["zk"],
                                           a["zv"], a["kr"], d_rope, ctypes.c_float(base),
                                           a["ctx"], a["Wk"], a["Wv"], N, N, a["out"], a["ws"],
                                           ctypes.c_size_t(a["wsb"]), S)
    d = desc(variant=lla.LLA_2D, r_k=256, r_v=256, n_max=100)
    for kw in (dict(qr=N), dict(kr=M), dict(ctx=N), dict(base=-2.0), dict(C=101), dict(t=4)):
        assert call(d, **kw) == lla.LLA_ERR_INVALID_ARG, kw
    assert call(d, d_rope=32) == lla.LLA_ERR_UNSUPPORTED  # MFMA path: 64 or 128
    assert call(d) == lla.LLA_ERR_WORKSPACE
    # pairs without the MFMA prefill take the streaming path: d_rope 32, 64 or 128, bf16 only
    dl = desc(r_k=24, r_v=24, n_max=70000)
    for dr in (32, 64, 128):
        assert call(dl, B=1, C=2, d_rope=dr) == lla.LLA_ERR_WORKSPACE  # supported; needs split partials
    assert call(dl, B=1, C=2, d_rope=48) == lla.LLA_ERR_UNSUPPORTED
    assert call(desc(r_k=24, r_v=24, n_max=70000, dtype=lla.LLA_F32), B=1, C=2) == lla.LLA_ERR_UNSUPPORTED
    assert call(desc(variant=lla.LLA_2D, r_k=32, r_v=32, n_max=70000), B=1, C=2, d_rope=32) == \
        lla.LLA_ERR_WORKSPACE


def test_noalloc_decode_refusals_on_the_host():
    """lla_attend_decode_noalloc validates like lla_attend_decode and refuses a plan larger than
    its static scratch before touching the GPU."""
    lib = lla.library()

    def call(d, B=2, t=0, q=A, out=A):
        return lib.lla_attend_decode_noalloc(ctypes.byref(d), B, t, q, A, A, N, A, A, N, N, N, N,
                                             out, N, S)
    assert call(desc(n_max=100), t=4) == lla.LLA_ERR_INVALID_ARG
    assert call(desc(n_max=100), q=M) == lla.LLA_ERR_INVALID_ARG
    assert call(desc(n_max=100, r_k=40, r_v=40)) == lla.LLA_ERR_UNSUPPORTED
    # LLA-2D MFMA read at B = 4096: 64 MiB of absorbed queries alone
    big = desc(variant=lla.LLA_2D, r_k=256, r_v=256, n_max=8193)
    assert lla.lla_workspace_bytes(big, 4096) > lla.LLA_NOALLOC_SCRATCH_BYTES
    assert call(big, B=4096) == lla.LLA_ERR_SCRATCH_LIMIT
    assert "scratch" in lla.lla_status_string(lla.LLA_ERR_SCRATCH_LIMIT)


def test_noalloc_cases_use_the_scratch():
    """Every call of the no-alloc GPU test plans token splits (so the static scratch is written and
    then reused by the smaller second call) within the scratch limit."""
    from tests.test_zz_no_alloc import CASES
    for variant, H, d, T, rk, rv, calls in CASES:
        for B, n_max, _ in calls:
            v = lla.LLA_PER_HEAD if variant == "per_head" else lla.LLA_2D
            d_ = lla.make_desc(v, lla.LLA_BF16, H, d, T, rk, rv, n_max)
            assert 0 < lla.lla_workspace_bytes(d_, B, 1) <= lla.LLA_NOALLOC_SCRATCH_BYTES, \
                (variant, rk, rv, B, n_max)
