"""CPU checks of the decode schedule (csrc/schedule.hpp), the integer
arithmetic both decode kernels use to split a step's work over their
persistent workgroups.

The header is compiled for the host and every piece of every workgroup's
range is enumerated, as the kernels walk them. Checked for single-tile
units (the stream kernel) and four-tile units (the other kernels), with
and without empty lead units, over the shapes the GPU suite uses and over
random ragged batches:

* every tile of every segment is covered exactly once, and a workgroup's
  pieces are consecutive segments;
* p0 and p1 are exactly the first and last workgroups holding the segment,
  every workgroup in between holds part of it, and all its pieces agree;
* the partial slots of the split merge: a shared piece is either its
  range's first piece (slot 0, wg != p0) or its last (slot 1, wg == p0), so
  each of a workgroup's two slots is written at most once per launch, every
  slot index is < 2 P, and the slots a merge reads (slot 1 of p0, slot 0 of
  p0 + 1 .. p1) are exactly the ones the segment's pieces wrote;
* the split is even: ranges differ by at most one unit (lead units counted).
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from gqa_kv_cache_decode_amd import _lib, build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def sched(tmp_path_factory):
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    so = str(tmp_path_factory.mktemp("sched") / "libsched_host.so")
    cmd = [cc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-I", build.CSRC, os.path.join(HERE, "sched_host.cpp"), "-o", so]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    lib = ctypes.CDLL(so)
    lib.sched_pieces.restype = ctypes.c_int
    lib.sched_pieces.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    return lib


def pieces(lib, ut, lens, ngroups, lead, P):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    cap = 4096
    while True:
        out = np.zeros((cap, 10), dtype=np.int32)
        n = lib.sched_pieces(ut, lens.ctypes.data, len(lens), ngroups, lead, P, out.ctypes.data, cap)
        if n <= cap:
            return out[:n]
        cap = n


def check(lib, ut, lens, ngroups, lead, P):
    rows = pieces(lib, ut, lens, ngroups, lead, P)
    tiles = [(int(L) + 31) // 32 for L in lens]
    parts = int(rows[0, 9]) if len(rows) else 0
    # coverage: every tile of every segment exactly once
    seen = {}
    for wg, k, s, grp, tb, te, p0, p1, more, _ in rows:
        assert 0 <= s < len(lens) and 0 <= grp < ngroups and 0 <= tb < te <= tiles[s], (wg, s, grp, tb, te)
        assert tb % ut == 0
        seen.setdefault((s, grp), []).append((tb, te, wg, k, p0, p1, more))
    for s in range(len(lens)):
        for grp in range(ngroups):
            got = sorted(seen.get((s, grp), []))
            if tiles[s] == 0:
                assert not got
                continue
            pos = 0
            for tb, te, *_ in got:
                assert tb == pos, (s, grp, got)
                pos = te
            assert pos == tiles[s], (s, grp, got)
            # owners: exactly the workgroups p0 .. p1, one piece each, in order
            wgs = [w for _, _, w, *_ in got]
            p0s = {r[4] for r in got}
            p1s = {r[5] for r in got}
            assert len(p0s) == 1 and len(p1s) == 1
            p0, p1 = p0s.pop(), p1s.pop()
            assert wgs == list(range(p0, p1 + 1)), (s, grp, wgs, p0, p1)
            assert 0 <= p0 <= p1 < P
    # a workgroup's pieces: consecutive segments, contiguous real tiles
    by_wg = {}
    for r in rows:
        by_wg.setdefault(int(r[0]), []).append(r)
    for wg, rs in by_wg.items():
        assert [int(r[1]) for r in rs] == list(range(len(rs)))
        order = [(int(r[2]), int(r[3])) for r in rs]
        assert order == sorted(order) and len(set(order)) == len(order)
        for r in rs[1:]:
            assert r[4] == 0, "only a range's first piece may start inside a segment"
        for r in rs[:-1]:
            assert r[5] == tiles[r[2]], "only a range's last piece may end inside a segment"
        # the split-merge slots
        used = []
        for r in rs:
            wg_, k, s, grp, tb, te, p0, p1, more, _ = (int(x) for x in r)
            if p0 == p1:
                continue
            slot = 1 if wg_ == p0 else 0
            if slot == 0:
                assert k == 0, "a piece that does not start its segment is its range's first"
            else:
                assert k == len(rs) - 1, "a shared piece that starts its segment is its range's last"
            idx = 2 * wg_ + slot
            assert idx < 2 * P
            used.append(idx)
        assert len(used) == len(set(used)), f"workgroup {wg} writes a slot twice"
    # the even split: real plus lead units per range differ by at most one
    if parts:
        T = sum(ngroups * ((-(-int(L) // (32 * ut)) + lead) if int(L) > 0 else 0) for L in lens)
        sizes = [(w + 1) * T // parts - w * T // parts for w in range(parts)]
        assert max(sizes) - min(sizes) <= 1
        assert sum(sizes) == T
    return rows


def test_failing_64_head_shape_of_the_unit_kernel(sched):
    # b = 2, h = 64, g = 1 (one 64-head segment per sequence), lengths 200 and
    # 131: the edge shape whose four-wave instance gave wrong results and once
    # did not finish after unrelated edits; its schedule covers, merges and
    # uses its slots as intended at every grid size and lead
    p = ctypes.c_int()
    w = ctypes.c_int()
    lib = _lib.load() if os.path.exists(build.LIB_PATH) else None
    grids = [1, 2, 3, 4, 7, 64, 2048]
    if lib is not None:
        assert lib.gqa_decode_plan(2, 64, 1, 128, 128, 256, 200, _lib.BF16, 0, 0, ctypes.byref(p),
                                   ctypes.byref(w)) == 0
        grids.append(w.value)
    for P in grids:
        for lead in (0, 3, 5):
            rows = check(sched, 4, [200, 131], 1, lead, P)
            assert len(rows) >= 2


@pytest.mark.parametrize("ut,lead", [(1, 0), (1, 4), (1, 6), (1, 8), (4, 0), (4, 2), (4, 5)])
def test_workload_shapes(sched, ut, lead):
    rng = np.random.default_rng(1003)
    llama = rng.integers(1024, 8193, 16) + 1
    for lens, ngroups in ((llama, 8), ([2049] * 64, 4), ([4097] * 8, 1), ([32769] * 4, 32), ([32769] * 4, 1),
                          ([38, 65], 2)):
        for P in (1, 5, 64, 256, 512, 2048):
            check(sched, ut, lens, ngroups, lead, P)


def test_random_ragged_batches(sched):
    rng = np.random.default_rng(77)
    for _ in range(300):
        b = int(rng.integers(1, 70))
        lens = rng.integers(0, 3000, b)
        lens[rng.random(b) < 0.2] = 0
        lens[rng.random(b) < 0.1] = rng.integers(1, 40)
        ngroups = int(rng.choice([1, 2, 3, 8, 16]))
        ut = int(rng.choice([1, 4]))
        lead = int(rng.choice([0, 1, 2, 5, 8]))
        P = int(rng.choice([1, 2, 3, 17, 64, 256, 2048]))
        check(sched, ut, lens, ngroups, lead, P)


def test_all_empty_and_single_tile(sched):
    assert len(pieces(sched, 1, [0, 0, 0], 4, 8, 256)) == 0
    rows = check(sched, 1, [1], 1, 8, 256)
    assert len(rows) == 1 and rows[0, 6] == rows[0, 7]
