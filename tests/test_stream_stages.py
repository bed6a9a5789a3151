"""Stage indices of the decode streaming kernel (csrc/stream.hip), enumerated
on the CPU.

stream_loop keeps D stages of 128 K-values in flight per wave. For one unit
it requests stages 0 .. D-1 (or, at a unit boundary, the next unit's first D
stages), then its main loop consumes stages st0 .. st0+D-1 and requests
st0+D .. st0+2D-1 while st0 + 2D <= S (S = K / 128), and its last D stages
are consumed after the loop while the next unit's first stages (or, after the
block's last unit, a re-read of stages S-D .. S-1) are requested. The
launchers accept a depth only where S is a multiple of D and S >= D
(stream_depth_ok); launch_stream picks D = 8 / 4 / 1 (MXFP4) and 4 / 4 / 1
(int8) by divisibility, launch_stream_fused uses 8 and 4 with K a multiple
of 1024.

This model of that index arithmetic checks, for every K the library accepts
(128 .. 16384 in steps of 128) and every depth a launcher would instantiate,
that every requested stage lies in [0, S) and that every stage is consumed
exactly once, after it was requested; and that the host rule rejects every
depth for which the loop would not cover S.
"""
import pytest

DEPTHS_MX = (8, 4, 1)      # launch_stream, MXFP4 pass
DEPTHS_I8 = {8: 4, 4: 4, 1: 1}  # int8 depth paired with each MXFP4 depth
FUSED = (8, 4)


def depth_ok(K, D):
    S = K >> 7
    return K % 128 == 0 and S >= D and S % D == 0


def launch_stream_depths(K):
    S = K // 128
    da = 8 if S % 8 == 0 else 4 if S % 4 == 0 else 1
    return da, DEPTHS_I8[da]


def unit_stages(S, D, P, more):
    """(requests, consumptions) of one unit in program order, plus the next
    unit's first requests, as the kernel's loops issue them."""
    req, use = [("cur", i) for i in range(D)], []
    st0 = 0
    while st0 + 2 * D <= S:
        for i in range(0, D, P):
            use += [("cur", st0 + i + j) for j in range(P)]
            req += [("cur", st0 + i + j + D) for j in range(P)]
        st0 += D
    nst = 0 if more else S - D
    for i in range(0, D, P):
        use += [("cur", st0 + i + j) for j in range(P)]
        req += [("nxt" if more else "cur", nst + i + j) for j in range(P)]
    return req, use


def check(S, D, P):
    for more in (True, False):
        req, use = unit_stages(S, D, P, more)
        for _, st in req:
            assert 0 <= st < S, (S, D, P, more, st)
        consumed = [st for _, st in use]
        assert sorted(consumed) == list(range(S)), (S, D, P, consumed)
        # every stage is requested (in the current unit) before it is consumed
        first_req = {}
        for n, (who, st) in enumerate(req):
            if who == "cur":
                first_req.setdefault(st, n)
        for n, st in enumerate(consumed):
            assert st in first_req, (S, D, P, st)


@pytest.mark.parametrize("K", range(128, 16384 + 1, 128))
def test_launch_stream_depths_cover_k(K):
    S = K // 128
    da, db = launch_stream_depths(K)
    assert depth_ok(K, da) and depth_ok(K, db)
    check(S, da, 2 if da % 2 == 0 else 1)  # MXFP4: stage pairs when D is even
    check(S, db, 1)                         # int8


@pytest.mark.parametrize("K", range(1024, 16384 + 1, 1024))
def test_fused_depths_cover_k(K):
    S = K // 128
    assert depth_ok(K, FUSED[0]) and depth_ok(K, FUSED[1])
    check(S, FUSED[0], 2)
    check(S, FUSED[1], 1)


def test_host_rule_rejects_uncovered_depths():
    """A depth that does not divide S would leave stages unconsumed; the host
    rule rejects exactly those (and D > S)."""
    for S in range(1, 129):
        for D in (1, 2, 3, 4, 5, 6, 8, 10, 12, 16):
            ok = depth_ok(S * 128, D)
            assert ok == (S >= D and S % D == 0)
            if S >= D and S % D:
                req, use = unit_stages(S, D, 1, True)
                assert sorted(st for _, st in use) != list(range(S))
                assert all(0 <= st < S for _, st in req)  # the loop form itself stays in bounds


def test_kernel_source_matches_model():
    """The model above follows these lines of the kernel and launchers."""
    import os
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "mxfp4_moe_expert_amd", "csrc", "stream.hip")).read()
    assert "for (; st0 + 2 * D <= S; st0 += D) {" in src
    assert "const int nst = more ? 0 : S - D;" in src
    assert "return K % 128 == 0 && S >= D && S % D == 0;" in src
    assert "constexpr int kDA = 8, kDB = 4;" in src
    assert "constexpr int P = (FMT != kFmtI8 && D % 2 == 0) ? 2 : 1;" in src
