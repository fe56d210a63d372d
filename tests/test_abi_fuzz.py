"""Seeded fuzz of the C ABI's host-side validation (CPU only, no GPU, no launch).

Every call built here carries at least one argument the library must refuse (a null required
pointer or a misaligned one), drawn together with extreme sizes: descriptors and batch or chunk
counts up to the int32 limit, ranks and head widths past what is compiled. The calls must return
LLA_ERR_INVALID_ARG (never crash, never reach a launch), and the workspace queries must return 0 or
a size that a 64-bit count holds without wrapping.
"""
import ctypes

import numpy as np
import pytest

from decode_attention_lla_amd import lla
from tests.test_abi_cpu import A, M, N, S, decode, encode, gather, prefill, quantize

BIG = 2**31 - 1


def _desc(rng):
    pick = lambda xs: int(xs[rng.integers(len(xs))])  # noqa: E731
    return lla.make_desc(pick([lla.LLA_PER_HEAD, lla.LLA_2D, 2, -1]),
                         pick([lla.LLA_F32, lla.LLA_BF16, lla.LLA_BF16_Q8, lla.LLA_BF16_I8, 7]),
                         pick([0, 1, 16, 2**16, BIG]), pick([8, 128, 256, 264, 7, BIG]),
                         pick([0, 1, 4, 2**20]), pick([8, 24, 256, 512, 513, BIG]),
                         pick([8, 24, 256, 512, 513, BIG]), pick([1, 4097, 2**24, BIG]),
                         float(rng.choice([0.0, 0.1, -1.0, np.inf, np.nan])))


def _sizes(rng):
    return [int(x) for x in rng.choice([0, 1, 2, 2**16, BIG, -1], 2)]


@pytest.mark.parametrize("seed", range(8))
def test_refused_calls_never_crash(seed):
    rng = np.random.default_rng(40000 + seed)
    for _ in range(150):
        d = _desc(rng)
        B, C = _sizes(rng)
        bad = [N, M][rng.integers(2)]  # a null or a misaligned pointer for a required argument
        which = int(rng.integers(3))
        args = [A, A, A]
        args[which] = bad
        assert decode(d, B=B, t=int(rng.integers(-1, 5)), q=args[0], zk=args[1], out=args[2]) == \
            lla.LLA_ERR_INVALID_ARG
        assert encode(d, B=B, C=C, xk=args[0], Ek=args[1], zk=args[2]) == lla.LLA_ERR_INVALID_ARG
        assert prefill(d, B=B, C=C, q=args[0], zv=args[1], ctx=args[2]) == lla.LLA_ERR_INVALID_ARG
        assert gather(d, B=B, budget=C, q=args[0], slots=args[1], Wv=args[2]) == \
            lla.LLA_ERR_INVALID_ARG
        assert quantize(d, B=B, C=C, ks=args[0], pos=args[1], zv=args[2]) == lla.LLA_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", range(4))
def test_workspace_queries_are_total(seed):
    rng = np.random.default_rng(41000 + seed)
    lib = lla.library()
    for _ in range(300):
        d = _desc(rng)
        B, C = _sizes(rng)
        for n in (lla.lla_workspace_bytes(d, B, C), lla.lla_gather_workspace_bytes(d, B, C),
                  lib.lla_reconstruct_workspace_bytes(ctypes.byref(d), B),
                  lib.lla_rope_workspace_bytes(ctypes.byref(d), B)):
            assert 0 <= n < 2**62
        if B <= 0 or C <= 0:
            assert lla.lla_workspace_bytes(d, B, C) == 0


def test_workspace_queries_refuse_what_the_calls_refuse():
    """Row counts past the calls' limit (B·C·H, and B·budget for the gather read) give 0, not a
    wrapped product."""
    lib = lla.library()
    d = lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, 16, 128, 4, 24, 24, 4097)
    assert lla.lla_workspace_bytes(d, 2**20, 2**11) == 0        # B·C·H = 2^35
    assert lla.lla_workspace_bytes(d, 2**21, 1) == 0            # B·H = 2^25 >= 2^31 / 64
    assert lla.lla_gather_workspace_bytes(d, 2**16, 2**16) == 0  # B·budget = 2^32
    assert lib.lla_rope_workspace_bytes(ctypes.byref(d), 2**21) == 0
    assert lib.lla_reconstruct_workspace_bytes(ctypes.byref(d), 2**21) == 0
    # just inside the limit the queries answer
    assert lla.lla_workspace_bytes(d, 2**20 - 1, 1) >= 0
    assert lla.lla_workspace_bytes(d, 1, 2) > 0  # a 2-row chunk over 4097 slots splits


def test_heads_past_a_launch_dimension_are_refused():
    """Heads index a launch dimension of at most 65535 workgroups: H = 65536 is an invalid
    descriptor (every query answers 0), H = 65535 is accepted (the rebuilt K/V always need
    workspace; the LLA-2D rotary read always holds its absorbed queries there)."""
    lib = lla.library()
    for H, ok in ((65535, True), (65536, False)):
        d = lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, H, 64, 1, 32, 32, 16)
        d2 = lla.make_desc(lla.LLA_2D, lla.LLA_BF16, H, 64, 1, 64, 64, 16)
        assert (lib.lla_rope_workspace_bytes(ctypes.byref(d2), 1) > 0) == ok
        assert (lib.lla_reconstruct_workspace_bytes(ctypes.byref(d), 1) > 0) == ok
        assert lla.lla_workspace_bytes(d, 1, 2) == 0 or ok
