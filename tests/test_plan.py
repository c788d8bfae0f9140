"""Host-side planning for other device geometries (no GPU): the argument and
planning code of the library (csrc/gla_plan.cpp, which has no HIP dependency)
is compiled here on its own with every symbol visible, and its planner is
called for an MI355X (256 compute units in 8 XCDs), a 4-XCD / 128-CU device and
a single-XCD device."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "recurrent_vision_backbone_key_amd", "csrc")

from recurrent_vision_backbone_key_amd import gla  # noqa: E402


class Geom(ctypes.Structure):
    _fields_ = [("cus", ctypes.c_int), ("xcds", ctypes.c_int)]


class Plan(ctypes.Structure):
    """Mirror of ``gla_plan`` (csrc/gla_plan.h)."""
    _fields_ = [("L", ctypes.c_int), ("nchunks", ctypes.c_int), ("seg_chunks", ctypes.c_int),
                ("nseg", ctypes.c_int), ("onepass", ctypes.c_int), ("xcd_local", ctypes.c_int),
                ("xcd_tasks", ctypes.c_int), ("xcds", ctypes.c_int), ("one_round", ctypes.c_int),
                ("group", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t), ("off_flags", ctypes.c_size_t),
                ("off_agg", ctypes.c_size_t), ("off_incl", ctypes.c_size_t),
                ("off_slots", ctypes.c_size_t), ("proj_fused", ctypes.c_int),
                ("off_z", ctypes.c_size_t), ("tau", ctypes.c_float), ("scale", ctypes.c_float),
                ("eps", ctypes.c_float)]


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("plan") / "libgla_plan_host.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-I" + os.path.join(ROOT, "include"),
                    "-I" + CSRC, os.path.join(CSRC, "gla_plan.cpp"), "-o", out], check=True)
    h = ctypes.CDLL(out)
    h.gla_make_plan.restype = ctypes.c_int
    h.gla_make_plan.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(gla.GlaOpts), ctypes.c_int,
                                                     ctypes.POINTER(Geom), ctypes.POINTER(Plan)]
    return h


def plan(h, geom, B, NH, H, W, seg=0, algorithm=0):
    o = gla.make_opts(B, NH, 64, 64, gla.F16, segment_chunks=seg, algorithm=algorithm)
    p = Plan()
    g = Geom(*geom) if geom else None
    st = h.gla_make_plan(0, H, W, 64, ctypes.byref(o), 0, ctypes.byref(g) if g else None,
                         ctypes.byref(p))
    assert st == 0
    return p


def workgroups(p, B, NH):
    return p.xcds * p.xcd_tasks if p.xcd_local else B * NH * p.nseg


def test_default_geometry_is_mi355x(planner):
    a = plan(planner, None, 1, 6, 40, 40)
    b = plan(planner, (256, 8), 1, 6, 40, 40)
    assert (a.seg_chunks, a.xcd_local, a.xcd_tasks, a.xcds) == (b.seg_chunks, b.xcd_local,
                                                                  b.xcd_tasks, b.xcds)
    # 6 scans of 25 chunks: one-chunk segments, one scan per XCD, one round
    assert (b.onepass, b.seg_chunks, b.nseg, b.xcd_local, b.xcd_tasks, b.one_round) == \
        (1, 1, 25, 1, 25, 1)


def capacity(seg, cus):
    """Workgroups resident at once: one per compute unit."""
    return cus


def test_four_xcd_geometry(planner):
    """128 compute units in 4 XCDs (32 each): the 1.6K-token frame with 6 heads
    needs two-chunk segments to fit one round, two scans per XCD."""
    p = plan(planner, (128, 4), 1, 6, 40, 40)
    assert (p.onepass, p.seg_chunks, p.nseg, p.xcds) == (1, 2, 13, 4)
    assert p.xcd_local == 1 and p.xcd_tasks == 2 * 13 and p.one_round == 1
    assert workgroups(p, 1, 6) == 4 * 26
    # 8 images: 48 scans do not fit one round even in eight-chunk segments
    # (the longest, fewest workgroups); scans divide evenly over 4 XCDs
    q = plan(planner, (128, 4), 8, 6, 40, 40)
    assert q.onepass == 1 and q.seg_chunks == 8 and q.xcd_local == 1
    assert q.xcd_tasks == 12 * 4 and q.one_round == 0
    # the same batch on an MI355X: five-chunk segments in one round
    r = plan(planner, (256, 8), 8, 6, 40, 40)
    assert (r.seg_chunks, r.nseg, r.one_round) == (5, 5, 1)


def test_segments_longer_than_five_chunks(planner):
    """Segments of six to eight chunks (the eight-chunk instance) when shorter
    ones would need a second round: the shortest that fits one round, else
    eight chunks."""
    # 8 x 6 scans of 28 chunks: 6-chunk segments, 30 workgroups per XCD
    p = plan(planner, (256, 8), 8, 6, 42, 42)
    assert (p.seg_chunks, p.nseg, p.xcd_local, p.xcd_tasks, p.one_round) == (6, 5, 1, 30, 1)
    # 6 scans of 256 chunks: 7-chunk segments, 222 workgroups chip-wide
    p = plan(planner, (256, 8), 1, 6, 128, 128)
    assert (p.seg_chunks, p.nseg, p.xcd_local, p.one_round) == (7, 37, 0, 1)
    # 48 scans of 256 chunks fit no single round: eight-chunk segments
    p = plan(planner, (256, 8), 8, 6, 128, 128)
    assert (p.seg_chunks, p.nseg, p.one_round) == (8, 32, 0)


def test_single_xcd_geometry_is_chip_wide(planner):
    """One XCD (a partitioned device): no XCD-local placement."""
    p = plan(planner, (32, 1), 1, 6, 40, 40)
    assert p.onepass == 1 and p.xcd_local == 0 and p.xcds == 1
    assert p.one_round == (6 * p.nseg <= capacity(p.seg_chunks, 32))
    assert workgroups(p, 1, 6) == 6 * p.nseg


def test_one_round_matches_the_grid(planner):
    """The one-round flag holds exactly when every workgroup of the launch has a
    compute unit of its own (a scheme that waits on every earlier segment needs
    them all resident)."""
    for geom in ((256, 8), (128, 4), (64, 2), (32, 1)):
        cus, xcds = geom
        for B, NH, H, W in ((1, 6, 40, 40), (8, 6, 40, 40), (1, 12, 80, 80), (2, 3, 17, 23),
                            (8, 6, 128, 128), (1, 1, 8, 8)):
            p = plan(planner, geom, B, NH, H, W)
            if not p.onepass:
                continue
            if p.xcd_local:
                assert p.one_round == (p.xcd_tasks <= capacity(p.seg_chunks, cus // xcds))
                units_x = -(-B * NH // xcds)
                assert p.xcd_tasks == units_x * p.nseg
            else:
                assert p.one_round == (B * NH * p.nseg <= capacity(p.seg_chunks, cus))


def test_exchange_group_sizes(planner):
    """Group size of the two-level exchange: one level below 24 segments;
    from 24 on ceil(sqrt(nseg)), or one more when that folds no more
    transfers at the worst segment and at most 8 (one round of loads);
    every segment's fold (j / G combined transfers, j mod G aggregates)
    checked by brute force against that bound."""
    planner.gla_exchange_group.restype = ctypes.c_int
    planner.gla_exchange_group.argtypes = [ctypes.c_int]
    want = {1: 1, 5: 5, 23: 23, 24: 5, 25: 6, 26: 7, 27: 7, 28: 6, 29: 6, 30: 6, 36: 6, 37: 7, 65: 9}
    for n, g in want.items():
        assert planner.gla_exchange_group(n) == g, (n, planner.gla_exchange_group(n), g)

    def most(n, g):
        return max(j // g + j % g for j in range(n))
    for n in range(24, 66):
        g = planner.gla_exchange_group(n)
        g0 = 1
        while g0 * g0 < n:
            g0 += 1
        assert g in (g0, g0 + 1)
        if g == g0 + 1:
            assert most(n, g) <= min(most(n, g0), 8)
        else:
            assert most(n, g0 + 1) > min(most(n, g0), 8)


def test_plan_carries_the_exchange_group(planner):
    """A one-round single-pass plan of 25 one-chunk segments (a 40x40 frame,
    6 heads) carries groups of 6; a 5-segment plan (8 frames) one level."""
    p = plan(planner, None, 1, 6, 40, 40)
    assert (p.onepass, p.nseg, p.one_round, p.group) == (1, 25, 1, 6)
    p = plan(planner, None, 8, 6, 40, 40)
    assert (p.onepass, p.nseg, p.one_round, p.group) == (1, 5, 1, 5)
